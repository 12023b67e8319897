// Skinny bf16 matrix products on MFMA: R <= 256 node rows (the tree tokens)
// times V weight rows of length H, streamed from HBM once.  Used for the base
// model's lm_head over the tree nodes (argmax fused into the epilogue) and
// for the decoder layer's projections (split over the contraction, fp32
// partial sums per split).
//
// Grid (ceil(V / 64), ceil(R / NODES), splits); 4 waves per workgroup, each
// wave owns 16 weight rows (one 16-row v_mfma_f32_16x16x32_bf16 block)
// against NODES node rows.  Weight fragments stream from HBM straight into
// registers (each lane reads 16 contiguous bytes; 4 lanes cover 64 contiguous
// bytes of a row), non-temporal, up to three k-chunks ahead; the node rows are
// staged in LDS in k-chunks shared by the 4 waves (double-buffered, one
// barrier per chunk).
#pragma once

#include "common.hpp"

namespace medusa {

enum { SKINNY_ARGMAX = 0, SKINNY_PARTIAL = 1 };

// node blocks of 16 rows for R node rows (R <= 256), and the k-chunk width
inline int lmh_nblk(int R) { return R <= 64 ? 4 : R <= 128 ? 8 : 16; }
inline int lmh_kc(int nblk) { return nblk <= 4 ? 256 : 512 / nblk; }

// Up to three weight matrices stacked along the output axis (e.g. q, k and
// v projections, or gate and up): logical row v is row v of w0 for v < n0,
// row v - n0 of w1 below n0 + n1, and of w2 after that.
struct WeightRows {
    const bf16_t* w0;
    const bf16_t* w1;
    const bf16_t* w2;
    int n0, n1;
    __device__ __forceinline__ const bf16_t* row(int v, int H) const {
        if (v < n0) return w0 + (size_t)v * H;
        if (v < n0 + n1) return w1 + (size_t)(v - n0) * H;
        return w2 + (size_t)(v - n0 - n1) * H;
    }
};

constexpr int LMH_WAVES = 4;
constexpr int LMH_VB = 1;                          // 16-row vocabulary blocks per wave
constexpr int LMH_ROWS = LMH_WAVES * LMH_VB * 16;  // vocabulary rows per workgroup

template <int NBLK>
struct LmhCfg {
    static constexpr int NODES = NBLK * 16;
    // k per chunk and ring depth (measured on 64 x 4096 x 32000: 256-wide
    // chunks two deep beat 128-wide chunks three deep); larger node tiles use
    // narrower chunks so a node stage stays at 8192 elements
    static constexpr int KC = NBLK <= 4 ? 256 : 512 / NBLK;
    static constexpr int KS = KC / 32;                 // MFMA k-steps per chunk
    static constexpr int LDW = KC + 8;                 // padded LDS row (bf16)
    static constexpr int NPT = NODES * KC / 8 / 256;   // 16-byte node pieces per thread per chunk
    static constexpr int D = NBLK <= 4 ? 2 : 3;        // chunks in flight per register ring
};

// Pipeline (one barrier per chunk): step c issues the node rows and then the
// lm_head fragments of chunk c + D - 1 into register rings, runs chunk c's
// MFMAs from LDS stage c & 1, publishes the node rows of chunk c + 1 into the
// other LDS stage, and synchronises.  Node loads are issued before the
// lm_head loads of the same step: vector-memory loads complete in issue
// order, so waiting for a chunk's node rows never waits for younger lm_head
// fragments, and about two chunks of lm_head stay in flight at all times.
template <int NBLK, int EPI>
__global__ __launch_bounds__(256) void skinny_mfma_kernel(const bf16_t* __restrict__ n,  // [R][H] node rows
                                                          WeightRows W,                   // V rows of H
                                                          int R, int H, int V, int chunks_per_split,
                                                          float* __restrict__ cand_val,
                                                          int* __restrict__ cand_idx,  // ARGMAX: [R][G]
                                                          float* __restrict__ out) {
    // ARGMAX: out = optional logits [R][V];  PARTIAL: out = [splits][R][V]
    using C = LmhCfg<NBLK>;
    constexpr int D = C::D;
    __shared__ __attribute__((aligned(16))) bf16_t ns[2][C::NODES][C::LDW];
    __shared__ float red_v[LMH_WAVES][C::NODES];
    __shared__ int red_i[LMH_WAVES][C::NODES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int G = gridDim.x;
    const int node0 = blockIdx.y * C::NODES;
    const int vw = blockIdx.x * LMH_ROWS + wave * (LMH_VB * 16);  // first vocab row of this wave
    const int lr = lane & 15, lk = lane >> 4;                      // row / k-group within a 16x16x32 tile

    f32x4 acc[LMH_VB][NBLK];
#pragma unroll
    for (int a = 0; a < LMH_VB; ++a)
#pragma unroll
        for (int b = 0; b < NBLK; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const bf16_t* wrow[LMH_VB];
    bool wvalid[LMH_VB];
#pragma unroll
    for (int a = 0; a < LMH_VB; ++a) {
        const int v = vw + a * 16 + lr;
        wvalid[a] = v < V;
        wrow[a] = W.row(wvalid[a] ? v : 0, H) + lk * 8;
    }

    // this workgroup's k-range: chunks [c_lo, c_lo + nchunk)
    const int c_lo = blockIdx.z * chunks_per_split;
    const int nchunk = min(H / C::KC - c_lo, chunks_per_split);  // host guarantees H % KC == 0
    u32x4 aring[D][C::KS][LMH_VB];
    u32x4 nring[D][C::NPT];
    auto load_a = [&](u32x4(&dst)[C::KS][LMH_VB], int c) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
#pragma unroll
            for (int a = 0; a < LMH_VB; ++a)
                dst[s][a] = wvalid[a] ? ld_stream(wrow[a] + (c_lo + c) * C::KC + s * 32) : (u32x4){0u, 0u, 0u, 0u};
    };
    auto load_n = [&](u32x4(&dst)[C::NPT], int c) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            const int p = tid + e * 256;
            const int r = p / (C::KC / 8), k8 = p - r * (C::KC / 8);
            const int node = node0 + r;
            dst[e] = node < R ? *(const u32x4*)(n + (size_t)node * H + (c_lo + c) * C::KC + k8 * 8)
                              : (u32x4){0u, 0u, 0u, 0u};
        }
    };
    auto store_n = [&](const u32x4(&src)[C::NPT], int stage) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            const int p = tid + e * 256;
            const int r = p / (C::KC / 8), k8 = p - r * (C::KC / 8);
            *(u32x4*)(&ns[stage][r][k8 * 8]) = src[e];
        }
    };
    auto compute = [&](const u32x4(&src)[C::KS][LMH_VB], int stage) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
#pragma unroll
            for (int b = 0; b < NBLK; ++b) {
                const u32x4 bv = *(const u32x4*)(&ns[stage][b * 16 + lr][s * 32 + lk * 8]);
#pragma unroll
                for (int a = 0; a < LMH_VB; ++a)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, src[s][a]),
                                                                        __builtin_bit_cast(bf16x8, bv), acc[a][b], 0,
                                                                        0, 0);
            }
        }
    };

#pragma unroll
    for (int u = 0; u < D - 1; ++u)
        if (u < nchunk) {
            load_n(nring[u], u);
            load_a(aring[u], u);
        }
    store_n(nring[0], 0);
    __syncthreads();
    for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int c = c0 + u;  // ring slot of chunk c is c % D == u
            if (c < nchunk) {
                if (c + D - 1 < nchunk) {
                    load_n(nring[(u + D - 1) % D], c + D - 1);
                    load_a(aring[(u + D - 1) % D], c + D - 1);
                }
                compute(aring[u], c & 1);
                if (c + 1 < nchunk) store_n(nring[(u + 1) % D], (c + 1) & 1);
                __syncthreads();
            }
        }
    }

    // epilogue: lane holds rows vw + a*16 + 4*lk + r of node column b*16 + lr
    if (EPI == SKINNY_PARTIAL) {
        float* part = out + (size_t)blockIdx.z * R * V;
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int node = node0 + b * 16 + lr;
            if (node >= R) continue;
#pragma unroll
            for (int a = 0; a < LMH_VB; ++a) {
                const int v0 = vw + a * 16 + lk * 4;
                if (v0 + 3 < V && (V & 3) == 0) {
                    *(f32x4*)(part + (size_t)node * V + v0) = acc[a][b];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (v0 + r < V) part[(size_t)node * V + v0 + r] = acc[a][b][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        const int node = node0 + b * 16 + lr;
#pragma unroll
        for (int a = 0; a < LMH_VB; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = vw + a * 16 + lk * 4 + r;
                const float x = acc[a][b][r];
                if (v < V) {
                    if (out != nullptr && node < R) out[(size_t)node * V + v] = x;
                    if (better(x, v, bv, bi)) { bv = x; bi = v; }
                }
            }
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            const float ov = __shfl_xor(bv, m, 64);
            const int oi = __shfl_xor(bi, m, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (lane < 16) { red_v[wave][b * 16 + lane] = bv; red_i[wave][b * 16 + lane] = bi; }
    }
    __syncthreads();
    for (int j = tid; j < C::NODES; j += 256) {
        float bv = red_v[0][j];
        int bi = red_i[0][j];
#pragma unroll
        for (int w = 1; w < LMH_WAVES; ++w)
            if (better(red_v[w][j], red_i[w][j], bv, bi)) { bv = red_v[w][j]; bi = red_i[w][j]; }
        const int node = node0 + j;
        if (node < R) {
            cand_val[(size_t)node * G + blockIdx.x] = bv;
            cand_idx[(size_t)node * G + blockIdx.x] = bi;
        }
    }
}

}  // namespace medusa
