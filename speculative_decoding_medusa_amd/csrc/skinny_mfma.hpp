// Skinny bf16 matrix products on MFMA: R <= 256 node rows (the tree tokens)
// times V weight rows of length K, the weights streamed from HBM once.  Used
// for the base model's lm_head over the tree nodes (argmax fused into the
// epilogue), for the decoder layer's projections (split over the
// contraction, fp32 partial sums per split), and for the heads' vocabulary
// projection of up to 8 sequences (per-head top-k fused into the epilogue).
//
// Weights are read in the packed fragment order (pack.hip): for every block
// of 16 rows and every 32-wide step of the contraction, the 16 x 32 tile is
// one contiguous 1 KB fragment laid out exactly as the A operand of
// v_mfma_f32_16x16x32_bf16 sits in a wave (lane l: row l % 16, k = 8 (l / 16)
// .. +7), so every weight load of a wave is one coalesced 1 KB read; the
// fragments of one k-step lie side by side over all row blocks, so a wave's
// consecutive fragments are one k-step of the whole matrix apart.
//
// Grid (ceil(V / (16 WAVES RB)), ceil(R / NODES), splits); WAVES waves per
// workgroup, each owning RB 16-row blocks against NODES node rows.  Weight fragments stream
// into registers (non-temporal) up to D - 1 k-chunks ahead; the node rows are
// staged in LDS in k-chunks shared by the waves (double-buffered, one
// barrier per chunk).  Every load is issued unconditionally -- rows past the
// end read a clamped valid row whose results the epilogue discards -- so the
// compiler can count outstanding loads exactly and wait for each chunk alone.
#pragma once

#include "common.hpp"

namespace medusa {

// ARGMAX: per-workgroup argmax candidates (base greedy);  PARTIAL: fp32 sums
// per contraction split;  SWIGLU (unsplit gate|up with gate and up rows
// interleaved in 16-row blocks): bf16(SiLU(gate) * up);  TOPK (16 node rows:
// rows 0..7 the bf16 heads of up to 8 sequences' inputs, rows 8..15 their
// bf16 remainders; one weight matrix per grid row y): per-workgroup top-k
// candidates of each sequence;  SILU (node rows: the R <= 16 sequences'
// bf16 hidden states; one weight matrix per grid row y): the residual-SiLU
// block z[b][y][row] = h[b][row] + SiLU(score + bias[y][row])
enum { SKINNY_ARGMAX = 0, SKINNY_PARTIAL = 1, SKINNY_SWIGLU = 2, SKINNY_TOPK = 3, SKINNY_SILU = 4 };

// packed fragment geometry
constexpr int PACK_ROWS = 16;                      // rows per fragment
constexpr int PACK_K = 32;                         // contraction elements per fragment
constexpr int PACK_FRAG = PACK_ROWS * PACK_K;      // elements per fragment (1 KB of bf16)

// node blocks of 16 rows for R node rows (R <= 256), and the k-chunk width
inline int lmh_nblk(int R) { return R <= 64 ? 4 : R <= 128 ? 8 : 16; }
inline int lmh_kc(int nblk) { return nblk <= 8 ? 64 : 32; }

constexpr int LMH_WAVES = 4;                       // waves per workgroup of the products
constexpr int LMH_ROWS = LMH_WAVES * PACK_ROWS;    // weight rows per workgroup

template <int NBLK, int WAVES = LMH_WAVES>
struct LmhCfg {
    static constexpr int NODES = NBLK * 16;
    static constexpr int NT = WAVES * 64;
    // k per chunk and register-ring depth (measured on 64 x 4096 x 32000:
    // 64-wide chunks four deep beat 128 three deep and 256 two deep); 256
    // node rows use 32-wide chunks so the node ring stays small; 16 node rows
    // use chunks wide enough that every thread stages one 16-byte piece
    static constexpr int KC = NBLK == 1 ? NT / 2 : NBLK <= 8 ? 64 : 32;
    static constexpr int KS = KC / PACK_K;             // MFMA k-steps per chunk
    // LDS rows of the node tile.  Tiles of >= 64 rows: unpadded rows whose
    // 16-byte column c sits at c ^ swz(row) -- measured with the LDS
    // bank-conflict counter on gfx950, both the MFMA fragment reads (16 rows x
    // 4 columns a wave) and the staging writes (KC / 8 pieces a row) are then
    // conflict-free, where padded rows cost twice the cycles on the reads.
    // 16-row tiles (wide chunks, little LDS traffic) keep padded rows.
    static constexpr bool SWZ = NBLK > 1;
    static constexpr int LDW = SWZ ? KC : KC + 8;
    static __device__ __forceinline__ int swz(int row) { return SWZ ? (row >> 1) & (KC / 8 - 1) : 0; }
    static constexpr int PIECES = NODES * KC / 8;           // 16-byte node pieces per chunk
    static constexpr int NPT = (PIECES + NT - 1) / NT;     // per thread (the last round may be partial)
    static constexpr bool EVEN = NPT * NT == PIECES;
    static constexpr int D = NBLK == 1 && WAVES > 4 ? 3 : NBLK <= 4 ? 4 : 3;  // chunks in flight per ring
};

// Pipeline (one barrier per chunk): step c issues the node rows and then the
// weight fragments of chunk c + D - 1 (the last chunk again past the end)
// into register rings, runs chunk c's MFMAs from LDS stage c & 1, publishes
// the node rows of chunk c + 1 into the other stage, and synchronises.  Node
// loads go out before the weight loads of the same step: vector-memory loads
// complete in issue order, so waiting for a chunk's node rows never waits for
// younger weight fragments.
// RB (ARGMAX and TOPK): 16-row weight blocks per wave; every node fragment
// read from LDS then feeds RB products, which halves the LDS traffic per
// product at RB = 2 (the bound of the 128- and 256-node tiles), and a
// workgroup stages its node rows once for RB times the weight rows.  With
// TOPK and RB > 1 the weight ring is two chunks deep (each chunk already
// holds RB times the fragments): fewer bytes in flight per CU measured
// faster (see the packed vocabulary projection in heads.hip).
// NS (ARGMAX only): the waves split the node blocks into NS groups -- wave w
// takes row group w / NS and node blocks (w % NS) NBLK / NS .. -- so each wave
// reads 1/NS of the node fragments per chunk; the NS waves of a row group
// load the same weight fragments (the second load hits the caches), and a
// workgroup has NS times as many waves for the same weight rows, which hide
// each other's LDS and MFMA latencies.
template <int NBLK, int EPI, int WAVES = LMH_WAVES, int RB = 1, int NS = 1>
__global__ __launch_bounds__(WAVES * 64) void skinny_mfma_kernel(const bf16_t* __restrict__ n,   // [R][K] node rows
                                                          const bf16_t* __restrict__ Wp,  // packed, V rows of K
                                                          int R, int K, int V, int chunks_per_split,
                                                          float* __restrict__ cand_val,
                                                          int* __restrict__ cand_idx,  // ARGMAX: [R][G]
                                                          float* __restrict__ out,
                                                          float rs_eps = -1.f,
                                                          int topk = 0, int nseq = 0, long long n_stride = 0,
                                                          long long w_stride = 0,
                                                          const bf16_t* __restrict__ bias = nullptr) {
    // ARGMAX: out = optional logits [R][V]; with rs_eps >= 0 each node row's
    // scores times its RMSNorm factor rsqrt(mean(n^2) + rs_eps), accumulated
    // from the node rows as they are staged (a positive factor: the argmax is
    // that of the unscaled scores);  PARTIAL: out = [splits][R][V];  SWIGLU: out = bf16 [R][V / 2];
    // TOPK: grid row y is matrix y (node rows at n + y n_stride, weights at
    // Wp + y w_stride); out = optional logits [nseq][gridDim.y][V];
    // candidates [nseq][gridDim.y][G][topk]
    using C = LmhCfg<NBLK, WAVES>;
    constexpr int D = EPI == SKINNY_TOPK && RB > 1 ? 2 : C::D;
    constexpr int NT = C::NT;
    __shared__ __attribute__((aligned(16))) bf16_t ns[2][C::NODES][C::LDW];
    constexpr int RG = WAVES / NS;      // row groups of a workgroup
    constexpr int NBW = NBLK / NS;      // node blocks per wave
    __shared__ float red_v[RG][EPI == SKINNY_ARGMAX ? C::NODES : 1];
    __shared__ int red_i[RG][EPI == SKINNY_ARGMAX ? C::NODES : 1];
    __shared__ f32x4 xup[EPI == SKINNY_SWIGLU ? WAVES / 2 : 1][EPI == SKINNY_SWIGLU ? NBLK : 1][64];
    __shared__ float tkv[EPI == SKINNY_TOPK ? WAVES * PACK_ROWS * RB : 1][8];  // TOPK: the workgroup's rows x sequences
    static_assert((EPI != SKINNY_TOPK && EPI != SKINNY_SILU) || NBLK == 1, "top-k / SiLU epilogue: 16 node rows");
    static_assert(RB == 1 || EPI == SKINNY_ARGMAX || EPI == SKINNY_TOPK,
                  "several row blocks per wave: argmax and top-k epilogues only");
    static_assert(NS == 1 || (EPI == SKINNY_ARGMAX && NBLK % NS == 0 && WAVES % NS == 0), "node split: argmax only");
    if (EPI == SKINNY_TOPK || EPI == SKINNY_SILU) {
        n += (size_t)blockIdx.y * n_stride;
        Wp += (size_t)blockIdx.y * w_stride;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x;
    const int node0 = (EPI == SKINNY_TOPK || EPI == SKINNY_SILU) ? 0 : blockIdx.y * C::NODES;
    const int rgw = wave / NS, ngw = wave % NS;        // this wave's row group and node group
    const int rb = (blockIdx.x * RG + rgw) * RB;       // this wave's first 16-row block
    const int vw = rb * PACK_ROWS;                    // its first weight row
    const int lr = lane & 15, lk = lane >> 4;         // row / k-group within a 16x16x32 tile
    const int nrb = (V + PACK_ROWS - 1) / PACK_ROWS;

    f32x4 acc[RB * NBW];  // row block j, the wave's node block b: acc[j * NBW + b]
#pragma unroll
    for (int b = 0; b < RB * NBW; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const bf16_t* wb[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) wb[j] = Wp + (size_t)min(rb + j, nrb - 1) * PACK_FRAG + lane * 8;
    const size_t kstride = (size_t)nrb * PACK_FRAG;  // elements from one k-step's fragment to the next

    // the node row of each of this thread's pieces is the same in every chunk
    const bf16_t* nrow[C::NPT];
    int k8p[C::NPT];
#pragma unroll
    for (int e = 0; e < C::NPT; ++e) {
        const int p = min(tid + e * NT, C::PIECES - 1);  // past the stage: re-read the last piece, not stored
        const int r = p / (C::KC / 8);
        k8p[e] = p - r * (C::KC / 8);
        nrow[e] = n + (size_t)min(node0 + r, R - 1) * K;
    }

    // this workgroup's k-range: chunks [c_lo, c_lo + nchunk), nchunk >= 1
    const int c_lo = blockIdx.z * chunks_per_split;
    const int nchunk = min(K / C::KC - c_lo, chunks_per_split);  // host guarantees K % KC == 0
    u32x4 aring[D][C::KS * RB];
    u32x4 nring[D][C::NPT];
    auto load_a = [&](u32x4(&dst)[C::KS * RB], int c) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
#pragma unroll
            for (int j = 0; j < RB; ++j)
                dst[s * RB + j] = ld_stream(wb[j] + (size_t)((c_lo + c) * C::KS + s) * kstride);
    };
    auto load_n = [&](u32x4(&dst)[C::NPT], int c) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) dst[e] = *(const u32x4*)(nrow[e] + (size_t)(c_lo + c) * C::KC + k8p[e] * 8);
    };
    auto store_n = [&](const u32x4(&src)[C::NPT], int stage) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            const int p = tid + e * NT;
            const int r = p / (C::KC / 8);
            if (C::EVEN || p < C::PIECES) *(u32x4*)(&ns[stage][r][(k8p[e] ^ C::swz(r)) * 8]) = src[e];
        }
    };

    // ARGMAX with logits: per-thread sums of squares of the node pieces it
    // stages (each chunk once; pieces of one row per chunk lie in KC / 8
    // consecutive threads)
    const bool want_rs = EPI == SKINNY_ARGMAX && out != nullptr && rs_eps >= 0.f;
    float rss[C::NPT];
#pragma unroll
    for (int e = 0; e < C::NPT; ++e) rss[e] = 0.f;
    auto add_sq = [&](const u32x4(&src)[C::NPT]) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            if (C::EVEN || tid + e * NT < C::PIECES) {
                float v[8];
                Elem<bf16_t>::expand(src[e], v);
#pragma unroll
                for (int j = 0; j < 8; ++j) rss[e] = fmaf(v[j], v[j], rss[e]);
            }
        }
    };

#pragma unroll
    for (int u = 0; u < D - 1; ++u) {
        const int cu = min(u, nchunk - 1);
        load_n(nring[u], cu);
        load_a(aring[u], cu);
    }
    store_n(nring[0], 0);
    if (want_rs) add_sq(nring[0]);
    __syncthreads();
    for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int c = c0 + u;  // ring slot of chunk c is c % D == u
            const int cn = min(c + D - 1, nchunk - 1);
            load_n(nring[(u + D - 1) % D], cn);
            load_a(aring[(u + D - 1) % D], cn);
            if (c < nchunk) {
                const int stage = c & 1;
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
#pragma unroll
                    for (int b = 0; b < NBW; ++b) {
                        const u32x4 bv = *(const u32x4*)(
                            &ns[stage][(ngw * NBW + b) * 16 + lr][((s * 4 + lk) ^ C::swz(lr)) * 8]);
#pragma unroll
                        for (int j = 0; j < RB; ++j)
                            acc[j * NBW + b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, aring[u][s * RB + j]), __builtin_bit_cast(bf16x8, bv),
                                acc[j * NBW + b], 0, 0, 0);
                    }
            }
            // the other stage was last read before the previous barrier
            store_n(nring[(u + 1) % D], (c + 1) & 1);
            if (want_rs && c + 1 < nchunk) add_sq(nring[(u + 1) % D]);
            __syncthreads();
        }
    }

    // epilogue: lane holds rows vw + 4*lk + r of node column b*16 + lr
    if (EPI == SKINNY_SWIGLU) {
        // waves 2j (gate rows) and 2j + 1 (up rows) hold the same 16 output
        // columns in the same lane layout; the up wave hands its sums over
        static_assert(WAVES % 2 == 0, "gate and up blocks pair up within a workgroup");
        if (wave & 1) {
#pragma unroll
            for (int b = 0; b < NBLK; ++b) xup[wave >> 1][b][lane] = acc[b];
        }
        __syncthreads();
        if (wave & 1) return;
        const int F = V / 2;
        const int c0 = (rb >> 1) * PACK_ROWS + lk * 4;  // this lane's 4 output columns
        bf16_t* a = (bf16_t*)out;
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int node = node0 + b * 16 + lr;
            if (node >= R || c0 >= F) continue;
            const f32x4 g = acc[b], u = xup[wave >> 1][b][lane];
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = g[r] / (1.f + __expf(-g[r])) * u[r];
            *(uint2*)(a + (size_t)node * F + c0) = (uint2){pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
        return;
    }
    if (EPI == SKINNY_SILU) {
        // lane (lr, lk) holds output rows vw + 4 lk + r of sequence lr (node
        // rows past R are clamped copies; their columns are not written)
        const int nm = gridDim.y, m = blockIdx.y;
        if (lr < R) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = vw + lk * 4 + r;
                if (v < V) {
                    const float pre = acc[0][r] + bf16_to_f32(bias[(size_t)m * V + v]);
                    const float sl = pre / (1.f + __expf(-pre));
                    out[((size_t)lr * nm + m) * V + v] = bf16_to_f32(n[(size_t)lr * K + v]) + sl;
                }
            }
        }
        return;
    }
    if (EPI == SKINNY_TOPK) {
        // lane (lr, lk) holds rows vw + 16 j + 4 lk + r of node column lr;
        // sequence b's score adds its remainder column b + 8, held by lane lr ^ 8
        const int nm = gridDim.y, m = blockIdx.y;
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = acc[j * NBW][r] + __shfl_xor(acc[j * NBW][r], 8, 64);
                const int v = vw + j * PACK_ROWS + lk * 4 + r;
                if (lr < 8) {
                    tkv[(wave * RB + j) * PACK_ROWS + lk * 4 + r][lr] = v < V ? x : -INFINITY;
                    if (out != nullptr && lr < nseq && v < V) out[((size_t)lr * nm + m) * V + v] = x;
                }
            }
        __syncthreads();
        // each wave takes sequences wave, wave + WAVES, ...: every lane keeps a
        // sorted list of the rows it scans, then the wave extracts the winners
        constexpr int ROWS = WAVES * PACK_ROWS * RB;
        for (int b = wave; b < nseq; b += WAVES) {
            float lv[MEDUSA_MAX_TOPK_DEV];
            int li[MEDUSA_MAX_TOPK_DEV];
#pragma unroll
            for (int t = 0; t < MEDUSA_MAX_TOPK_DEV; ++t) { lv[t] = -INFINITY; li[t] = 0x7FFFFFFF; }
            for (int r = lane; r < ROWS; r += 64) {
                const int v = blockIdx.x * ROWS + r;
                if (v < V) sorted_insert<MEDUSA_MAX_TOPK_DEV>(lv, li, tkv[r][b], v);
            }
            const size_t base = (((size_t)b * nm + m) * G + blockIdx.x) * topk;
            for (int t = 0; t < topk; ++t) {
                float bv = lv[0];
                int bi = li[0];
                wave_argmax(bv, bi);
                if (lane == 0) { cand_val[base + t] = bv; cand_idx[base + t] = bi; }
                if (lv[0] == bv && li[0] == bi) sorted_pop<MEDUSA_MAX_TOPK_DEV>(lv, li);
            }
        }
        return;
    }
    if (EPI == SKINNY_PARTIAL) {
        float* part = out + (size_t)blockIdx.z * R * V;
        const int v0 = vw + lk * 4;
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int node = node0 + b * 16 + lr;
            if (node >= R) continue;
            if (v0 + 3 < V && (V & 3) == 0) {
                *(f32x4*)(part + (size_t)node * V + v0) = acc[b];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (v0 + r < V) part[(size_t)node * V + v0 + r] = acc[b][r];
            }
        }
        return;
    }
    // ARGMAX: the node rows' RMSNorm factors (rows past R: clamped copies, unused)
    __shared__ float rs_l[EPI == SKINNY_ARGMAX ? C::NODES : 1];
    if (EPI == SKINNY_ARGMAX && want_rs) {
        constexpr int PPR = C::KC / 8;
        static_assert(64 % PPR == 0 && NT % PPR == 0, "a row's pieces within one wave");
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            float v = rss[e];
#pragma unroll
            for (int m = 1; m < PPR; m <<= 1) v += __shfl_xor(v, m, 64);
            const int p = tid + e * NT;
            if ((C::EVEN || p < C::PIECES) && p % PPR == 0) rs_l[p / PPR] = rsqrtf(v / (float)K + rs_eps);
        }
        __syncthreads();
    }
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        const int nb = ngw * NBW + b;  // node block within the workgroup's tile
        const int node = node0 + nb * 16 + lr;
        const float sc = (want_rs && node < R) ? rs_l[nb * 16 + lr] : 1.f;
#pragma unroll
        for (int j = 0; j < RB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = vw + j * PACK_ROWS + lk * 4 + r;
                const float x = acc[j * NBW + b][r];
                if (v < V) {
                    if (out != nullptr && node < R) out[(size_t)node * V + v] = x * sc;
                    if (better(x, v, bv, bi)) { bv = x; bi = v; }
                }
            }
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int oi = __shfl_xor(bi, m, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (lane < 16) { red_v[rgw][nb * 16 + lane] = bv; red_i[rgw][nb * 16 + lane] = bi; }
    }
    __syncthreads();
    for (int j = tid; j < C::NODES; j += NT) {
        float bv = red_v[0][j];
        int bi = red_i[0][j];
#pragma unroll
        for (int w = 1; w < RG; ++w)
            if (better(red_v[w][j], red_i[w][j], bv, bi)) { bv = red_v[w][j]; bi = red_i[w][j]; }
        const int node = node0 + j;
        if (node < R) {
            cand_val[(size_t)node * G + blockIdx.x] = bv;
            cand_idx[(size_t)node * G + blockIdx.x] = bi;
        }
    }
}

}  // namespace medusa
