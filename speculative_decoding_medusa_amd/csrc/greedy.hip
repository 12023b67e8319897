// Base model's greedy choice after every tree node (step a5):
// n_r = x_r * rsqrt(mean(x_r^2) + eps) (bf16-rounded for bf16 weights), then
// greedy[r] = argmax_v lm_head[v] . n_r  (lower index first among equal values).
//
// bf16: the product of the node rows with lm_head is a dense contraction
// (64-512 rows share every lm_head byte), so it runs on MFMA
// (v_mfma_f32_16x16x32_bf16) with the argmax fused into the epilogue:
//   grid (ceil(V / 64), ceil(R / NODES)); 4 waves per workgroup, each wave
//   owns 16 vocabulary rows (one 16-row MFMA block) against NODES node rows,
//   so the 32000-row vocabulary gives 500 workgroups (about two per CU).
//   lm_head fragments stream from HBM straight into registers (each lane
//   reads 16 contiguous bytes; 4 lanes cover 64 contiguous bytes of a row),
//   non-temporal, up to three k-chunks ahead; the node rows are staged in LDS in
//   k-chunks shared by the 4 waves (double-buffered, one barrier per chunk).
//   Each workgroup writes, per node, its best (value, index); a merge kernel
//   reduces them.
// float32: the vector-ALU GEMV of the heads (one pass per 8 rows).
#include "common.hpp"

namespace medusa {

// One block per row; writes n (float32 for the GEMV path, bf16 for MFMA).
template <typename T, typename OUT, bool ROUND_BF16>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* __restrict__ x, int H, float eps,
                                                           OUT* __restrict__ n) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const T* xr = x + (size_t)r * H;
    float ss = 0.f;
    for (int j = threadIdx.x; j < H; j += 256) {
        const float v = Elem<T>::load(xr, j);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rs = rsqrtf(tot / (float)H + eps);
    for (int j = threadIdx.x; j < H; j += 256) {
        float v = Elem<T>::load(xr, j) * rs;
        if (ROUND_BF16) v = bf16_to_f32(f32_to_bf16(v));
        Elem<OUT>::store(n, (size_t)r * H + j, v);
    }
}

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
template <int NBLK>
__global__ __launch_bounds__(256) void lm_head_argmax_kernel(const bf16_t* __restrict__ n,  // [R][H]
                                                             const bf16_t* __restrict__ W,  // [V][H]
                                                             int R, int H, int V, float* __restrict__ cand_val,
                                                             int* __restrict__ cand_idx,  // [R][G]
                                                             float* __restrict__ logits) {
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
        wrow[a] = W + (size_t)(wvalid[a] ? v : 0) * H + lk * 8;
    }

    const int nchunk = H / C::KC;  // host guarantees H % KC == 0
    u32x4 aring[D][C::KS][LMH_VB];
    u32x4 nring[D][C::NPT];
    auto load_a = [&](u32x4(&dst)[C::KS][LMH_VB], int c) {
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
#pragma unroll
            for (int a = 0; a < LMH_VB; ++a)
                dst[s][a] = wvalid[a] ? ld_stream(wrow[a] + c * C::KC + s * 32) : (u32x4){0u, 0u, 0u, 0u};
    };
    auto load_n = [&](u32x4(&dst)[C::NPT], int c) {
#pragma unroll
        for (int e = 0; e < C::NPT; ++e) {
            const int p = tid + e * 256;
            const int r = p / (C::KC / 8), k8 = p - r * (C::KC / 8);
            const int node = node0 + r;
            dst[e] = node < R ? *(const u32x4*)(n + (size_t)node * H + c * C::KC + k8 * 8) : (u32x4){0u, 0u, 0u, 0u};
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
                    if (logits != nullptr && node < R) logits[(size_t)node * V + v] = x;
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

// greedy[r] = best of the G workgroup candidates of row r
__global__ __launch_bounds__(64) void argmax_merge_kernel(const float* __restrict__ cand_val,
                                                          const int* __restrict__ cand_idx, int G,
                                                          int32_t* __restrict__ greedy) {
    const int r = blockIdx.x;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int g = threadIdx.x; g < G; g += 64) {
        const float v = cand_val[(size_t)r * G + g];
        const int i = cand_idx[(size_t)r * G + g];
        if (better(v, i, bv, bi)) { bv = v; bi = i; }
    }
    wave_argmax(bv, bi);
    if (threadIdx.x == 0) greedy[r] = bi;
}

void launch_vocab_topk_named(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                             float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s,
                             const char* gemv_name, const char* merge_name);
int vocab_topk_groups(int B, int V, int K);

// workgroups of the float32 GEMV path over any chunk of <= 8 rows
static int gemv_groups_max(int V) {
    int g = 0;
    for (int nb = 1; nb <= 8; ++nb) g = vocab_topk_groups(nb, V, 1) > g ? vocab_topk_groups(nb, V, 1) : g;
    return g;
}

static int lmh_nblk(int R) { return R <= 64 ? 4 : R <= 128 ? 8 : 16; }
static int lmh_kc(int nblk) { return nblk <= 4 ? 256 : 512 / nblk; }

static bool use_mfma(bool bf16, int H, int R) { return bf16 && H % lmh_kc(lmh_nblk(R)) == 0; }

static size_t a256(size_t x) { return (x + 255) / 256 * 256; }

size_t greedy_workspace_bytes(int R, int H, int V, bool bf16) {
    if (use_mfma(bf16, H, R)) {
        const size_t G = (V + LMH_ROWS - 1) / LMH_ROWS;
        return a256((size_t)R * H * 2) + a256((size_t)R * G * 4) * 2;
    }
    const int G = gemv_groups_max(V);
    return a256((size_t)R * H * 4) + a256((size_t)8 * G * 4) * 2 + a256((size_t)R * 4);
}

void launch_base_greedy(const void* x, const void* lm_head, int R, int H, int V, float eps, bool bf16,
                        int32_t* greedy, float* logits, void* ws, hipStream_t s) {
    char* p = (char*)ws;
    if (use_mfma(bf16, H, R)) {
        bf16_t* n = (bf16_t*)p;
        p += a256((size_t)R * H * 2);
        const int G = (V + LMH_ROWS - 1) / LMH_ROWS;
        float* cv = (float*)p;
        int* ci = (int*)(p + a256((size_t)R * G * 4));
        MEDUSA_LAUNCH("rmsnorm_rows", (rmsnorm_rows_kernel<bf16_t, bf16_t, false>), dim3(R), dim3(256), 0, s,
                      (const bf16_t*)x, H, eps, n);
        const int nblk = lmh_nblk(R);
        const dim3 grid(G, (R + nblk * 16 - 1) / (nblk * 16));
        if (nblk == 4)
            MEDUSA_LAUNCH("lm_head_argmax", lm_head_argmax_kernel<4>, grid, dim3(256), 0, s, n, (const bf16_t*)lm_head,
                          R, H, V, cv, ci, logits);
        else if (nblk == 8)
            MEDUSA_LAUNCH("lm_head_argmax", lm_head_argmax_kernel<8>, grid, dim3(256), 0, s, n, (const bf16_t*)lm_head,
                          R, H, V, cv, ci, logits);
        else
            MEDUSA_LAUNCH("lm_head_argmax", lm_head_argmax_kernel<16>, grid, dim3(256), 0, s, n,
                          (const bf16_t*)lm_head, R, H, V, cv, ci, logits);
        MEDUSA_LAUNCH("argmax_merge", argmax_merge_kernel, dim3(R), dim3(64), 0, s, cv, ci, G, greedy);
        return;
    }
    float* n = (float*)p;
    p += a256((size_t)R * H * 4);
    const int G = gemv_groups_max(V);
    float* cv = (float*)p;
    int* ci = (int*)(p + a256((size_t)8 * G * 4));
    p += a256((size_t)8 * G * 4) * 2;
    float* gval = (float*)p;
    if (bf16)
        MEDUSA_LAUNCH("rmsnorm_rows", (rmsnorm_rows_kernel<bf16_t, float, true>), dim3(R), dim3(256), 0, s,
                      (const bf16_t*)x, H, eps, n);
    else
        MEDUSA_LAUNCH("rmsnorm_rows", (rmsnorm_rows_kernel<float, float, false>), dim3(R), dim3(256), 0, s,
                      (const float*)x, H, eps, n);
    for (int r0 = 0; r0 < R; r0 += 8) {
        const int nb = R - r0 < 8 ? R - r0 : 8;
        launch_vocab_topk_named(n + (size_t)r0 * H, lm_head, nb, H, V, 1, 1, bf16,
                                logits ? logits + (size_t)r0 * V : nullptr, greedy + r0, gval + r0, cv, ci, s,
                                "lm_head_gemv", "lm_head_gemv_merge");
    }
}

}  // namespace medusa
