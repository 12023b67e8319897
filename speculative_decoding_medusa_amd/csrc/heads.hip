// Medusa heads: residual-SiLU block (step a1) and vocabulary projection with
// fused per-head top-k (step a2).
//
// Both are matrix-vector products that stream a weight matrix from HBM once
// (B <= 8 right-hand sides), so they are written as HBM-streaming GEMVs on the
// vector ALUs, not as MFMA tiles: every weight byte is used B times, far below
// the MFMA ridge.
//
// Layout of the work: grid (G, K); workgroup g of head k owns a contiguous
// block of rows; its 4 waves take groups of R consecutive rows in turn, so
// each wave visits its rows in increasing order.  A lane owns 16-byte chunks
// c*64 + lane of a row (fully coalesced 1 KiB per wave per load), multiplies
// them with the right-hand sides staged once per workgroup in LDS as fp32,
// and the 64 partial sums are combined with an xor butterfly whose result is
// bitwise identical in every lane.  The reduction order depends only on the
// row length, so the projection of a given z is bitwise reproducible.
#include "common.hpp"

namespace medusa {

enum { EPI_SILU = 0, EPI_TOPK = 1 };

constexpr int GEMV_THREADS = 256;
constexpr int GEMV_WAVES = GEMV_THREADS / 64;

template <typename WT, int NB, int CPL, int R, int EPI>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_rows_kernel(
    const void* __restrict__ xsrc,   // SILU: h [B][H] (WT);  TOPK: z [B][K][H] fp32
    const WT* __restrict__ W,        // [K][nrows][H]
    const WT* __restrict__ bias,     // SILU: b1 [K][H]
    int B, int H, int nrows, int K, int rows_per_wg,
    float* __restrict__ out,         // SILU: z [B][K][H];  TOPK: logits [B][K][nrows] or null
    float* __restrict__ cand_val,    // TOPK: [B][K][G][topk]
    int* __restrict__ cand_idx, int topk) {
    extern __shared__ float xs[];    // [NB][H] fp32
    constexpr int PER = Elem<WT>::PER16;
    const int k = blockIdx.y;
    const int g = blockIdx.x;
    const int G = gridDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // Stage the right-hand sides (fp32) in LDS; padded batch slots are zero.
    for (int i = threadIdx.x; i < NB * H; i += GEMV_THREADS) {
        const int b = i / H, j = i - b * H;
        float v = 0.f;
        if (b < B) {
            if (EPI == EPI_SILU) v = Elem<WT>::load((const WT*)xsrc, (size_t)b * H + j);
            else v = ((const float*)xsrc)[((size_t)b * K + k) * H + j];
        }
        xs[i] = v;
    }
    __syncthreads();

    const int nchunks = H / PER;
    const int row0 = g * rows_per_wg;
    const int row1 = min(nrows, row0 + rows_per_wg);
    const WT* Wk = W + (size_t)k * nrows * H;

    // Per-wave top-k list, lane j < topk holds rank j of sequence b.
    float tv[NB];
    int ti[NB];
    float kth[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) { tv[b] = -INFINITY; ti[b] = 0x7FFFFFFF; kth[b] = -INFINITY; }

    for (int rb = row0 + wave * R; rb < row1; rb += GEMV_WAVES * R) {
        u32x4 wv[R][CPL];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = rb + j;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ci = c * 64 + lane;
                if (row < row1 && ci < nchunks)
                    wv[j][c] = *(const u32x4*)(Wk + (size_t)row * H + (size_t)ci * PER);
                else
                    wv[j][c] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
        float acc[R][NB];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[j][b] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ci = c * 64 + lane;
            if (ci < nchunks) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float xv[PER];
#pragma unroll
                    for (int t = 0; t < PER; t += 4) {
                        const f32x4 q = *(const f32x4*)(xs + b * H + ci * PER + t);
                        xv[t] = q.x; xv[t + 1] = q.y; xv[t + 2] = q.z; xv[t + 3] = q.w;
                    }
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        float e[PER];
                        Elem<WT>::expand(wv[j][c], e);
#pragma unroll
                        for (int t = 0; t < PER; ++t) acc[j][b] = fmaf(e[t], xv[t], acc[j][b]);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = rb + j;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float v = wave_sum(acc[j][b]);
                if (row >= row1 || b >= B) continue;
                if (EPI == EPI_SILU) {
                    if (lane == 0) {
                        const float pre = v + Elem<WT>::load(bias, (size_t)k * H + row);
                        const float s = pre / (1.f + __expf(-pre));
                        out[((size_t)b * K + k) * H + row] = xs[b * H + row] + s;
                    }
                } else {
                    if (out != nullptr && lane == 0) out[((size_t)b * K + k) * nrows + row] = v;
                    if (v > kth[b]) {
                        const bool gt = lane < topk && v > tv[b];
                        const uint64_t m = __ballot(gt);
                        const int p = __ffsll((unsigned long long)m) - 1;
                        const float upv = __shfl_up(tv[b], 1, 64);
                        const int upi = __shfl_up(ti[b], 1, 64);
                        if (lane > p && lane < topk) { tv[b] = upv; ti[b] = upi; }
                        if (lane == p) { tv[b] = v; ti[b] = row; }
                        kth[b] = __shfl(tv[b], topk - 1, 64);
                    }
                }
            }
        }
    }

    if (EPI == EPI_TOPK) {
        // Merge the 4 per-wave sorted lists into the workgroup's top-k.
        __shared__ float sv[GEMV_WAVES][NB][MEDUSA_MAX_TOPK_DEV];
        __shared__ int si[GEMV_WAVES][NB][MEDUSA_MAX_TOPK_DEV];
        if (lane < topk) {
#pragma unroll
            for (int b = 0; b < NB; ++b) { sv[wave][b][lane] = tv[b]; si[wave][b][lane] = ti[b]; }
        }
        __syncthreads();
        if (threadIdx.x < B) {
            const int b = threadIdx.x;
            int head[GEMV_WAVES] = {0, 0, 0, 0};
            const size_t base = (((size_t)b * K + k) * G + g) * topk;
            for (int t = 0; t < topk; ++t) {
                int best = 0;
                for (int w = 1; w < GEMV_WAVES; ++w)
                    if (better(sv[w][b][head[w]], si[w][b][head[w]], sv[best][b][head[best]],
                               si[best][b][head[best]]))
                        best = w;
                cand_val[base + t] = sv[best][b][head[best]];
                cand_idx[base + t] = si[best][b][head[best]];
                if (head[best] < topk - 1) ++head[best];
                else sv[best][b][head[best]] = -INFINITY, si[best][b][head[best]] = 0x7FFFFFFF;
            }
        }
    }
}

// Final merge: per (b, k) pick the top-k of G * topk workgroup candidates.
// All candidate indices are distinct rows, so "strictly after the previous
// winner in (value desc, index asc) order" identifies the next one.
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ cand_val,
                                                        const int* __restrict__ cand_idx, int M,
                                                        int topk, int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_val) {
    const int bk = blockIdx.x;
    const int lane = threadIdx.x;
    const float* cv = cand_val + (size_t)bk * M;
    const int* ci = cand_idx + (size_t)bk * M;
    float pv = INFINITY;
    int pi = -1;
    for (int t = 0; t < topk; ++t) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
        for (int m = lane; m < M; m += 64) {
            const float v = cv[m];
            const int i = ci[m];
            if (better(pv, pi, v, i) && better(v, i, bv, bi)) { bv = v; bi = i; }
        }
        wave_argmax(bv, bi);
        if (lane == 0) {
            topk_idx[(size_t)bk * topk + t] = bi;
            topk_val[(size_t)bk * topk + t] = bv;
        }
        pv = bv;
        pi = bi;
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int pick_nb(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }
static int pick_cpl(int nchunks) {
    const int c = (nchunks + 63) / 64;
    return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 16;
}

constexpr int GEMV_R = 2;

template <typename WT, int NB, int CPL, int EPI>
static void launch_gemv_t(const void* x, const WT* W, const WT* bias, int B, int H, int nrows, int K,
                          int rows_per_wg, int G, float* out, float* cv, int* ci, int topk,
                          hipStream_t s, const char* name) {
    auto kern = gemv_rows_kernel<WT, NB, CPL, GEMV_R, EPI>;
    const size_t shmem = (size_t)NB * H * sizeof(float);
    if (shmem > 65536) hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    MEDUSA_LAUNCH(name, kern, dim3(G, K), dim3(GEMV_THREADS), shmem, s, x, W, bias, B, H, nrows, K,
                  rows_per_wg, out, cv, ci, topk);
}

template <typename WT, int EPI>
static void launch_gemv_nb(int NB, int CPL, const void* x, const WT* W, const WT* bias, int B, int H,
                           int nrows, int K, int rows_per_wg, int G, float* out, float* cv, int* ci,
                           int topk, hipStream_t s, const char* name) {
#define MEDUSA_GEMV_CASE(nb, cpl)                                                                  \
    if (NB == nb && CPL == cpl)                                                                    \
        return launch_gemv_t<WT, nb, cpl, EPI>(x, W, bias, B, H, nrows, K, rows_per_wg, G, out, cv, \
                                               ci, topk, s, name);
#define MEDUSA_GEMV_NB(nb) \
    MEDUSA_GEMV_CASE(nb, 1) MEDUSA_GEMV_CASE(nb, 2) MEDUSA_GEMV_CASE(nb, 4) MEDUSA_GEMV_CASE(nb, 8) MEDUSA_GEMV_CASE(nb, 16)
    MEDUSA_GEMV_NB(1) MEDUSA_GEMV_NB(2) MEDUSA_GEMV_NB(4) MEDUSA_GEMV_NB(8)
#undef MEDUSA_GEMV_NB
#undef MEDUSA_GEMV_CASE
}

// rows per workgroup: a multiple of the rows one pass of the 4 waves covers,
// sized so that the whole launch has about `target` workgroups.
static int rows_per_wg_for(int nrows, int K, int target) {
    const int quantum = GEMV_WAVES * GEMV_R;
    long long total = (long long)nrows * K;
    long long r = (total + target - 1) / target;
    r = ((r + quantum - 1) / quantum) * quantum;
    if (r < quantum) r = quantum;
    if (r > nrows) r = ((nrows + quantum - 1) / quantum) * quantum;
    return (int)r;
}

int vocab_topk_groups(int V, int K) {
    const int rpw = rows_per_wg_for(V, K, 1024);
    return (V + rpw - 1) / rpw;
}

void launch_resid_silu(const void* h, const void* w1, const void* b1, int B, int H, int K, bool bf16,
                       float* z, hipStream_t s) {
    const int rpw = rows_per_wg_for(H, K, 1024);
    const int G = (H + rpw - 1) / rpw;
    const int PER = bf16 ? 8 : 4;
    const int NB = pick_nb(B), CPL = pick_cpl(H / PER);
    if (bf16)
        launch_gemv_nb<bf16_t, EPI_SILU>(NB, CPL, h, (const bf16_t*)w1, (const bf16_t*)b1, B, H, H, K, rpw,
                                         G, z, nullptr, nullptr, 0, s, "resid_silu_gemv");
    else
        launch_gemv_nb<float, EPI_SILU>(NB, CPL, h, (const float*)w1, (const float*)b1, B, H, H, K, rpw, G,
                                        z, nullptr, nullptr, 0, s, "resid_silu_gemv");
}

void launch_vocab_topk_named(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                             float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s,
                             const char* gemv_name, const char* merge_name) {
    const int rpw = rows_per_wg_for(V, K, 1024);
    const int G = (V + rpw - 1) / rpw;
    const int PER = bf16 ? 8 : 4;
    const int NB = pick_nb(B), CPL = pick_cpl(H / PER);
    if (bf16)
        launch_gemv_nb<bf16_t, EPI_TOPK>(NB, CPL, z, (const bf16_t*)w2, nullptr, B, H, V, K, rpw, G, logits,
                                         cv, ci, topk, s, gemv_name);
    else
        launch_gemv_nb<float, EPI_TOPK>(NB, CPL, z, (const float*)w2, nullptr, B, H, V, K, rpw, G, logits, cv,
                                        ci, topk, s, gemv_name);
    MEDUSA_LAUNCH(merge_name, topk_merge_kernel, dim3(B * K), dim3(64), 0, s, cv, ci, G * topk, topk,
                  topk_idx, topk_val);
}

void launch_vocab_topk(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                       float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s) {
    launch_vocab_topk_named(z, w2, B, H, V, K, topk, bf16, logits, topk_idx, topk_val, cv, ci, s,
                            "vocab_proj_topk", "topk_merge");
}

}  // namespace medusa
