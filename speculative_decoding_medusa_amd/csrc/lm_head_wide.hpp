// Wide-tree lm_head argmax: 256-row node tiles against the packed bf16
// lm_head on v_mfma_f32_32x32x16_bf16, the argmax over the workgroup's
// weight rows fused into the epilogue.  The per-workgroup candidates have
// the layout of skinny_mfma_kernel's argmax epilogue ([R][G]) and go to the
// same merge.  Two kernels: lm_head_argmax_wide_kernel (128 weight rows a
// workgroup, loader waves) for vocabularies too small to give 256-row weight
// tiles 256 workgroups (32,000 rows), and lm_head_argmax_wide256_kernel
// (256 weight rows a workgroup, below) for the others.
//
// lm_head_argmax_wide_kernel.  Workgroup: 128 weight rows against one
// 256-row node tile, 8 waves in two
// roles.  Waves 0-3 (one per SIMD) are matrix waves: wave w owns the 32-row
// weight blocks 2 (w / 2) and 2 (w / 2) + 1 against node rows 128 (w % 2) ..
// + 127 (2 x 4 accumulator tiles of 32 x 32), so every k-step reads 2 weight
// and 4 node fragments from LDS for 8 products (with one weight block
// against all 256 nodes it read 1 + 8: LDS time was the tighter bound).
// They issue no global load, so no product ever waits behind a weight
// fragment still on its way from HBM.  Waves 4-7 are loader waves: they
// stream each 64-wide k-chunk's weight pieces and node rows into a register
// ring D chunks deep and publish chunk c + 1 into the idle one of two LDS
// stages while the matrix waves work on chunk c (one barrier per chunk for
// all 8 waves).  One chunk ahead measured fastest: 79 us against 82 with two
// and 85 with four at 256 x 4096 x 32000 (each workgroup then keeps about
// 48 KB of loads in flight instead of up to 192 KB).
//
// Operands (lane l of a matrix wave, k-step s of 16 within a chunk):
//   A, weights: row l % 32 of a 32-row block, k = 16 s + 8 (l / 32) .. +7 --
//     in the packed fragment order one 16-byte piece of the fragment of
//     16-row block 2 (32-row block) + (l % 32) / 16; LDS keeps the pieces in
//     lane order, [stage][32-row block][s][lane], so the matrix waves read
//     them linearly.
//   B, nodes: node row 32 t + l % 32, the same k, from the LDS node tile.
//   D: element r of lane l is weight row 8 (r / 4) + 4 (l / 32) + r % 4,
//     node l % 32 of tile t.
// LDS node tile: 128-byte rows without padding, 16-byte column c of row r at
// c ^ ((r >> 1) & 7): measured with the LDS bank-conflict counter on gfx950,
// both the B-fragment reads (32 rows x 2 columns a wave) and the staging
// writes (8 rows x 8 columns a wave) are then conflict-free.
// The last k-step of every chunk has its operands read before the chunk's
// barrier and its products issued after it, so the matrix pipe has 8
// products queued while the waves meet.
//
// Measured (256 x 4096 x 32000, random bf16 data): 79 us against 90 us for
// the 8-wave 16 x 16 x 32 node-split product.  Each workgroup carries 3 MB
// through its CU's vector-memory path (its 1 MB of weights from HBM, the
// 2 MB node tile from L2) and its LDS carries 96 KB of operand reads and
// 48 KB of loader writes per chunk; the products alone take 65 us (random
// bf16 operands keep the matrix cores at about 1.4 PFLOP/s, well under the
// constant-data rate).  Where there are enough workgroups the 256-row
// kernel below, which stages each node row for twice the weight rows, is
// faster (this one: 635 us at 512 x 4096 x 128256, that one 555).
//
// Grid: ceil(G / 8) * 8 * T workgroups for G = ceil(V / 128) row tiles and T
// node tiles.  Workgroup L runs on XCD L % 8 (round-robin dispatch); the T
// node tiles of one row tile are consecutive workgroups of one XCD, so they
// run together and the second reads the weights from that XCD's L2.
#pragma once

#include "common.hpp"
#include "skinny_mfma.hpp"

namespace medusa {

constexpr int LMW_NODES = 256;  // node rows per tile
constexpr int LMW_ROWS = 128;   // weight rows per workgroup
constexpr int LMW_KC = 64;      // contraction elements per chunk

inline int lmw_groups(int V) { return (V + LMW_ROWS - 1) / LMW_ROWS; }
inline int lmw_tiles(int R) { return (R + LMW_NODES - 1) / LMW_NODES; }

template <int D>
__global__ __launch_bounds__(512) void lm_head_argmax_wide_kernel(const bf16_t* __restrict__ n,   // [R][K]
                                                                  const bf16_t* __restrict__ Wp,  // packed [V][K]
                                                                  int R, int K, int V, int T, int G,
                                                                  float* __restrict__ cand_val,  // [R][G]
                                                                  int* __restrict__ cand_idx) {
    constexpr int KC = LMW_KC;
    constexpr int KS = KC / 16;                   // 32 x 32 x 16 k-steps per chunk
    constexpr int NTL = LMW_NODES / 32;           // accumulator tiles per matrix wave
    constexpr int NPL = LMW_NODES * (KC / 8) / 256;  // node pieces per loader thread per chunk
    constexpr int APL = 4 * KS * 64 / 256;           // weight pieces per loader thread per chunk
    static_assert(KC == 64 && NPL == 8 && APL == 4, "the swizzle and the loader split assume 64-wide chunks");
    __shared__ __attribute__((aligned(16))) bf16_t ns[2][LMW_NODES][KC];  // node tile, swizzled columns
    __shared__ u32x4 as[2][4][KS][64];  // weight pieces in the lane order of the A operand
    __shared__ float red_v[2][LMW_NODES];  // per row group of the matrix waves
    __shared__ int red_i[2][LMW_NODES];

    const int L = blockIdx.x, j = L >> 3;
    const int y = j % T, x = (j / T) * 8 + (L & 7);  // node tile, row tile
    if (x >= G) return;                               // padding of the grid to whole XCD rounds

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int node0 = y * LMW_NODES;
    const int nrb = (V + PACK_ROWS - 1) / PACK_ROWS;
    const int nchunk = K / KC;  // host guarantees K % KC == 0

    if (wave >= 4) {
        // ---- loader waves: chunk j's weight and node pieces into registers
        // D chunks ahead, published into LDS stage j & 1 one step before use
        const int lt = tid - 256;
        // weight pieces e = 0..3: 32-row block e, k-step s = lt / 64, lane l = lt % 64
        const int s = lt >> 6, l = lt & 63;
        const bf16_t* wa[APL];
#pragma unroll
        for (int e = 0; e < APL; ++e) {
            const int pb = min((x * 4 + e) * 2 + ((l & 31) >> 4), nrb - 1);  // past the end: clamped, discarded
            wa[e] = Wp + ((size_t)(s >> 1) * nrb + pb) * PACK_FRAG + ((2 * (s & 1) + (l >> 5)) * PACK_ROWS + (l & 15)) * 8;
        }
        const size_t cstride = (size_t)(KC / 32) * nrb * PACK_FRAG;  // one chunk of the packed matrix
        // node pieces e = 0..7: row (lt >> 3) + 32 e, 16-byte column lt & 7 (the
        // swizzle term (row >> 1) & 7 is the same for every e)
        const int col = lt & 7, row0 = lt >> 3;
        const int wcol = (col ^ ((row0 >> 1) & 7)) * 8;
        const bf16_t* nrow[NPL];
#pragma unroll
        for (int e = 0; e < NPL; ++e) nrow[e] = n + (size_t)min(node0 + row0 + 32 * e, R - 1) * K + col * 8;

        u32x4 nr[D][NPL], ar[D][APL];
        auto load = [&](int slot, int c) {
            c = min(c, nchunk - 1);  // past the end: the last chunk again, never published
#pragma unroll
            for (int e = 0; e < NPL; ++e) nr[slot][e] = *(const u32x4*)(nrow[e] + (size_t)c * KC);
#pragma unroll
            for (int e = 0; e < APL; ++e) ar[slot][e] = ld_stream(wa[e] + (size_t)c * cstride);
        };
        auto publish = [&](int slot, int st) {
#pragma unroll
            for (int e = 0; e < NPL; ++e) *(u32x4*)(&ns[st][row0 + 32 * e][wcol]) = nr[slot][e];
#pragma unroll
            for (int e = 0; e < APL; ++e) as[st][e][s][l] = ar[slot][e];
        };
#pragma unroll
        for (int u = 0; u < D; ++u) load(u, u);
        publish(0, 0);
        load(0, D);
        __syncthreads();
        // step c: chunk c + 1 into the idle stage (last read before the previous
        // barrier), then chunk c + 1 + D into the freed slot
        for (int c0 = 0; c0 < nchunk; c0 += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                const int c = c0 + u;
                if (c < nchunk) {
                    publish((u + 1) % D, (c + 1) & 1);
                    load((u + 1) % D, c + 1 + D);
                    __syncthreads();
                }
            }
        }
    } else {
        // ---- matrix waves: wave w owns the workgroup's 32-row weight blocks
        // 2 (w / 2) and 2 (w / 2) + 1 against its 32-node tiles 4 (w % 2) .. + 3
        constexpr int WB = 2;         // 32-row weight blocks per matrix wave
        constexpr int WT = NTL / 2;   // 32-node tiles per matrix wave
        const int rg = wave >> 1, nh = wave & 1;
        const int l32 = lane & 31, hi = lane >> 5;
        const int rsw = (l32 >> 1) & 7;  // swizzle of this lane's B-fragment row
        f32x16 acc[WB * WT];             // weight block j, node tile t: acc[j * WT + t]
#pragma unroll
        for (int t = 0; t < WB * WT; ++t) acc[t] = (f32x16){};
        auto read_b = [&](int st, int s, int t) {
            return __builtin_bit_cast(bf16x8,
                                      *(const u32x4*)(&ns[st][(nh * WT + t) * 32 + l32][((2 * s + hi) ^ rsw) * 8]));
        };
        auto read_a = [&](int st, int s, int j) { return __builtin_bit_cast(bf16x8, as[st][2 * rg + j][s][lane]); };
        auto mfma = [&](bf16x8 a, bf16x8 b, f32x16& d) {
            d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
        };
        // the previous chunk's last k-step (zeros before the first chunk): its
        // products are issued after the barrier that ends the chunk, so the
        // matrix pipe has 8 products queued while the waves meet
        bf16x8 bl[WT], al[WB];
#pragma unroll
        for (int t = 0; t < WT; ++t) bl[t] = (bf16x8){};
#pragma unroll
        for (int j = 0; j < WB; ++j) al[j] = (bf16x8){};
        __syncthreads();
        // scheduling fences keep every phase in place: the operands of a k-step
        // (2 weight and 4 node fragments for 8 products) are read one whole
        // k-step before their use
        for (int c = 0; c < nchunk; ++c) {
            const int st = c & 1;
            bf16x8 bc[WT], ac[WB];
#pragma unroll
            for (int j = 0; j < WB; ++j) ac[j] = read_a(st, 0, j);
#pragma unroll
            for (int t = 0; t < WT; ++t) bc[t] = read_b(st, 0, t);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < WB; ++j)
#pragma unroll
                for (int t = 0; t < WT; ++t) mfma(al[j], bl[t], acc[j * WT + t]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (s + 1 < KS) {
                    bf16x8 bn[WT], an[WB];
#pragma unroll
                    for (int j = 0; j < WB; ++j) an[j] = read_a(st, s + 1, j);
#pragma unroll
                    for (int t = 0; t < WT; ++t) bn[t] = read_b(st, s + 1, t);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < WB; ++j)
#pragma unroll
                        for (int t = 0; t < WT; ++t) mfma(ac[j], bc[t], acc[j * WT + t]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int j = 0; j < WB; ++j) ac[j] = an[j];
#pragma unroll
                    for (int t = 0; t < WT; ++t) bc[t] = bn[t];
                } else {
#pragma unroll
                    for (int j = 0; j < WB; ++j) al[j] = ac[j];
#pragma unroll
                    for (int t = 0; t < WT; ++t) bl[t] = bc[t];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < WB; ++j)
#pragma unroll
            for (int t = 0; t < WT; ++t) mfma(al[j], bl[t], acc[j * WT + t]);

        // best (value, lower index) per node over the wave's 64 rows, then over
        // the lane pair l, l ^ 32
#pragma unroll
        for (int t = 0; t < WT; ++t) {
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < WB; ++j) {
                const int vw = (x * 4 + 2 * rg + j) * 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int v = vw + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const float sc = acc[j * WT + t][r];
                    if (v < V && better(sc, v, bv, bi)) { bv = sc; bi = v; }
                }
            }
            const float ov = __shfl_xor(bv, 32, 64);
            const int oi = __shfl_xor(bi, 32, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            const int node = (nh * WT + t) * 32 + l32;
            if (hi == 0) { red_v[rg][node] = bv; red_i[rg][node] = bi; }
        }
    }
    __syncthreads();
    // over the 2 row groups: one node per thread of the first 256
    if (tid < LMW_NODES) {
        float bv = red_v[0][tid];
        int bi = red_i[0][tid];
        if (better(red_v[1][tid], red_i[1][tid], bv, bi)) { bv = red_v[1][tid]; bi = red_i[1][tid]; }
        const int node = node0 + tid;
        if (node < R) {
            cand_val[(size_t)node * G + x] = bv;
            cand_idx[(size_t)node * G + x] = bi;
        }
    }
}

// The same product for vocabularies that give 256-row weight tiles enough
// workgroups (two node tiles of a 128,256-row vocabulary): each workgroup
// holds 256 weight rows against one 256-row node tile, so every node row it
// stages from L2 feeds twice the weight rows of the 128-row tile above (that
// tile moved 4 GB of node rows at 512 x 128,256 and was bound by it).  8
// waves, two per SIMD; wave w owns the 32-row weight blocks 2 (w / 2) and
// 2 (w / 2) + 1 against node rows 128 (w % 2) .. + 127, the operands of each
// k-step read from LDS as above.  No wave role split (two matrix waves per
// SIMD leave no registers for loader waves): every thread loads a quarter of
// a chunk's 2,048 weight pieces and 2,048 node pieces into a register ring
// one chunk deep and publishes them into the idle LDS stage while the
// chunk before is computed.  Measured at 512 x 4096 x 128256: 555 us against
// 628 for the 16 x 16 x 32 product; without its loads it takes 426 us and
// without its products 404 us (each workgroup then has about 64 KB of loads
// in flight; a second chunk of registers would not fit beside the
// accumulators, and a third LDS stage would not fit either).
inline int lmw256_groups(int V) { return (V + 255) / 256; }

__global__ __launch_bounds__(512) void lm_head_argmax_wide256_kernel(const bf16_t* __restrict__ n,   // [R][K]
                                                                     const bf16_t* __restrict__ Wp,  // packed [V][K]
                                                                     int R, int K, int V, int T, int G,
                                                                     float* __restrict__ cand_val,  // [R][G]
                                                                     int* __restrict__ cand_idx) {
    constexpr int KC = LMW_KC;
    constexpr int KS = KC / 16;                 // 32 x 32 x 16 k-steps per chunk
    constexpr int NB = 8;                       // 32-row weight blocks per workgroup
    constexpr int PPT = 4;                      // weight pieces and node pieces per thread per chunk
    constexpr int WB = 2, WT = 4;               // per wave: 32-row weight blocks, 32-node tiles
    static_assert(KC == 64 && NB * KS * 64 == 512 * PPT && LMW_NODES * (KC / 8) == 512 * PPT, "piece split");
    __shared__ __attribute__((aligned(16))) bf16_t ns[2][LMW_NODES][KC];  // node tile, swizzled columns
    __shared__ u32x4 as[2][NB][KS][64];  // weight pieces in the lane order of the A operand
    __shared__ float red_v[4][LMW_NODES];  // per row group of waves
    __shared__ int red_i[4][LMW_NODES];

    const int L = blockIdx.x, j0 = L >> 3;
    const int y = j0 % T, x = (j0 / T) * 8 + (L & 7);  // node tile, row tile (256 rows)
    if (x >= G) return;                                 // padding of the grid to whole XCD rounds

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int node0 = y * LMW_NODES;
    const int nrb = (V + PACK_ROWS - 1) / PACK_ROWS;
    const int nchunk = K / KC;  // host guarantees K % KC == 0

    // this thread's pieces e = 0..3: weight block 2 e + tid / 256, k-step
    // (tid / 64) % 4, lane tid % 64; node row tid / 8 + 64 e, column tid % 8
    const int ps = (tid >> 6) & 3, pl = tid & 63, pbh = tid >> 8;
    const bf16_t* wa[PPT];
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
        const int pb = min((x * NB + 2 * e + pbh) * 2 + ((pl & 31) >> 4), nrb - 1);  // past the end: clamped
        wa[e] = Wp + ((size_t)(ps >> 1) * nrb + pb) * PACK_FRAG + ((2 * (ps & 1) + (pl >> 5)) * PACK_ROWS + (pl & 15)) * 8;
    }
    const size_t cstride = (size_t)(KC / 32) * nrb * PACK_FRAG;
    const int col = tid & 7, row0 = tid >> 3;
    const int wcol = (col ^ ((row0 >> 1) & 7)) * 8;
    const bf16_t* nrow[PPT];
#pragma unroll
    for (int e = 0; e < PPT; ++e) nrow[e] = n + (size_t)min(node0 + row0 + 64 * e, R - 1) * K + col * 8;
    u32x4 nr[PPT], ar[PPT];
    auto load = [&](int c) {
        c = min(c, nchunk - 1);  // past the end: the last chunk again, never published
#pragma unroll
        for (int e = 0; e < PPT; ++e) nr[e] = *(const u32x4*)(nrow[e] + (size_t)c * KC);
#pragma unroll
        for (int e = 0; e < PPT; ++e) ar[e] = ld_stream(wa[e] + (size_t)c * cstride);
    };
    auto publish = [&](int st) {
#pragma unroll
        for (int e = 0; e < PPT; ++e) *(u32x4*)(&ns[st][row0 + 64 * e][wcol]) = nr[e];
#pragma unroll
        for (int e = 0; e < PPT; ++e) as[st][2 * e + pbh][ps][pl] = ar[e];
    };

    const int rg = wave >> 1, nh = wave & 1;
    const int l32 = lane & 31, hi = lane >> 5;
    const int rsw = (l32 >> 1) & 7;
    f32x16 acc[WB * WT];
#pragma unroll
    for (int t = 0; t < WB * WT; ++t) acc[t] = (f32x16){};
    auto read_b = [&](int st, int s, int t) {
        return __builtin_bit_cast(bf16x8,
                                  *(const u32x4*)(&ns[st][(nh * WT + t) * 32 + l32][((2 * s + hi) ^ rsw) * 8]));
    };
    auto read_a = [&](int st, int s, int jb) { return __builtin_bit_cast(bf16x8, as[st][2 * rg + jb][s][lane]); };
    auto mfma = [&](bf16x8 a, bf16x8 b, f32x16& d) {
        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, d, 0, 0, 0);
    };

    load(0);
    publish(0);
    load(1);
    bf16x8 bl[WT], al[WB];
#pragma unroll
    for (int t = 0; t < WT; ++t) bl[t] = (bf16x8){};
#pragma unroll
    for (int jb = 0; jb < WB; ++jb) al[jb] = (bf16x8){};
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
        const int st = c & 1;
        bf16x8 bc[WT], ac[WB];
#pragma unroll
        for (int jb = 0; jb < WB; ++jb) ac[jb] = read_a(st, 0, jb);
#pragma unroll
        for (int t = 0; t < WT; ++t) bc[t] = read_b(st, 0, t);
        __builtin_amdgcn_sched_barrier(0);
        // the previous chunk's last k-step, after the barrier that ended it
#pragma unroll
        for (int jb = 0; jb < WB; ++jb)
#pragma unroll
            for (int t = 0; t < WT; ++t) mfma(al[jb], bl[t], acc[jb * WT + t]);
        __builtin_amdgcn_sched_barrier(0);
        // chunk c + 1 into the idle stage (last read before the previous
        // barrier), then chunk c + 2 into the registers just freed
        publish(st ^ 1);
        load(c + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (s + 1 < KS) {
                bf16x8 bn[WT], an[WB];
#pragma unroll
                for (int jb = 0; jb < WB; ++jb) an[jb] = read_a(st, s + 1, jb);
#pragma unroll
                for (int t = 0; t < WT; ++t) bn[t] = read_b(st, s + 1, t);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jb = 0; jb < WB; ++jb)
#pragma unroll
                    for (int t = 0; t < WT; ++t) mfma(ac[jb], bc[t], acc[jb * WT + t]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jb = 0; jb < WB; ++jb) ac[jb] = an[jb];
#pragma unroll
                for (int t = 0; t < WT; ++t) bc[t] = bn[t];
            } else {
#pragma unroll
                for (int jb = 0; jb < WB; ++jb) al[jb] = ac[jb];
#pragma unroll
                for (int t = 0; t < WT; ++t) bl[t] = bc[t];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int jb = 0; jb < WB; ++jb)
#pragma unroll
        for (int t = 0; t < WT; ++t) mfma(al[jb], bl[t], acc[jb * WT + t]);

    // best (value, lower index) per node over the wave's 64 rows, then over
    // the lane pair l, l ^ 32, then over the 4 row groups
#pragma unroll
    for (int t = 0; t < WT; ++t) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int jb = 0; jb < WB; ++jb) {
            const int vw = (x * NB + 2 * rg + jb) * 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int v = vw + 8 * (r >> 2) + 4 * hi + (r & 3);
                const float sc = acc[jb * WT + t][r];
                if (v < V && better(sc, v, bv, bi)) { bv = sc; bi = v; }
            }
        }
        const float ov = __shfl_xor(bv, 32, 64);
        const int oi = __shfl_xor(bi, 32, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        const int node = (nh * WT + t) * 32 + l32;
        if (hi == 0) { red_v[rg][node] = bv; red_i[rg][node] = bi; }
    }
    __syncthreads();
    if (tid < LMW_NODES) {
        float bv = red_v[0][tid];
        int bi = red_i[0][tid];
#pragma unroll
        for (int g = 1; g < 4; ++g)
            if (better(red_v[g][tid], red_i[g][tid], bv, bi)) { bv = red_v[g][tid]; bi = red_i[g][tid]; }
        const int node = node0 + tid;
        if (node < R) {
            cand_val[(size_t)node * G + x] = bv;
            cand_idx[(size_t)node * G + x] = bi;
        }
    }
}

}  // namespace medusa
