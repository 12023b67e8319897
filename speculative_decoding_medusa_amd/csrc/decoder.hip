// The tree-verify forward pass through a Llama-shaped decoder: every tree
// token runs through every layer at once, each attending to the layer's KV
// prefix plus its own tree ancestors, and the base model's greedy choice is
// taken after every node.
//
// Per layer (pre-norm): n = bf16(RMSNorm(x)); [q|k|v] = n W_qkv^T with RoPE
// on q and k at position cache_len + depth; o = tree attention (which also
// writes the tree keys/values into the layer's cache slots P..P+N-1);
// x += o W_o^T; n' = bf16(RMSNorm(x)); a = bf16(SiLU(n' W_gate^T) * (n' W_up^T));
// x += a W_down^T.  The residual stream x is float32; RMSNorm has unit
// weight.  After the last layer: greedy = argmax lm_head . bf16(RMSNorm(x)).
//
// The projections are skinny products (R = B*N <= 256 node rows against
// 4096-22016 weight rows): the packed weight matrix (q|k|v and gate|up each
// stacked into one) streams once from HBM through skinny_mfma_kernel, split
// along the contraction into whole rounds of workgroups over the CUs; each
// split writes fp32 partial sums and a small epilogue kernel adds them and
// applies RoPE, the residual (with the next RMSNorm) or SwiGLU.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "skinny_mfma.hpp"
#include "tree.hpp"

namespace medusa {

void launch_tree_attention(const void* q, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                           const int32_t* cache_len, int max_cache_len, const TreeDev& t, int B, int nH,
                           int nKV, int D, int Lmax, float scale, bool bf16, void* out, float* part_o,
                           float* part_ml, hipStream_t s, int target_wg);
size_t attn_workspace_bytes(int B, int nH, int N, int D, int max_cache_len, bool bf16);
void attn_carve(int B, int nH, int N, int D, int max_cache_len, bool bf16, void* ws, float** part_o,
                float** part_ml);
size_t lm_head_greedy_workspace_bytes(int R, int H, int V);
void launch_lm_head_greedy(const bf16_t* n, const bf16_t* lm_head, int R, int H, int V, int32_t* greedy,
                           void* ws, hipStream_t s);

// x[r][:] = embedding[tok[r]] (fp32); ids outside [0, V) read row 0.
__global__ __launch_bounds__(256) void embed_rows_kernel(const int32_t* __restrict__ tok, const bf16_t* __restrict__ E,
                                                         int H, int V, float* __restrict__ x) {
    const int r = blockIdx.x;
    int t = tok[r];
    if (t < 0 || t >= V) t = 0;
    const bf16_t* e = E + (size_t)t * H;
    for (int j = threadIdx.x * 8; j < H; j += 256 * 8) {
        float v[8];
        Elem<bf16_t>::expand(*(const u32x4*)(e + j), v);
        *(f32x4*)(x + (size_t)r * H + j) = (f32x4){v[0], v[1], v[2], v[3]};
        *(f32x4*)(x + (size_t)r * H + j + 4) = (f32x4){v[4], v[5], v[6], v[7]};
    }
}

// n[r][:] = bf16(x[r][:] * rsqrt(mean(x[r]^2) + eps)), x fp32.
__global__ __launch_bounds__(256) void rmsnorm_f32_bf16_kernel(const float* __restrict__ x, int H, float eps,
                                                               bf16_t* __restrict__ n) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const float* xr = x + (size_t)r * H;
    float ss = 0.f;
    for (int j = threadIdx.x * 4; j < H; j += 256 * 4) {
        const f32x4 v = *(const f32x4*)(xr + j);
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
    for (int j = threadIdx.x * 4; j < H; j += 256 * 4) {
        const f32x4 v = *(const f32x4*)(xr + j);
        *(uint2*)(n + (size_t)r * H + j) = (uint2){(uint32_t)f32_to_bf16(v.x * rs) | ((uint32_t)f32_to_bf16(v.y * rs) << 16),
                                                   (uint32_t)f32_to_bf16(v.z * rs) | ((uint32_t)f32_to_bf16(v.w * rs) << 16)};
    }
}

// The pass's first per-row work in one launch, one block per node row r:
// x[r] = embedding[tok[r]] (fp32; ids outside [0, V) read row 0), n[r] =
// bf16(x[r] * rsqrt(mean(x[r]^2) + eps)) with the sum taken in the order of
// rmsnorm_f32_bf16_kernel (so n is bitwise that kernel's), and the row's
// angle table cs[r][i] = (cos, sin) of pos[r] * base^(-2i/D) in double, as
// rope_table_kernel computes it.
__global__ __launch_bounds__(256) void embed_norm_rope_kernel(const int32_t* __restrict__ tok,
                                                              const bf16_t* __restrict__ E, int H, int V, float eps,
                                                              const int32_t* __restrict__ pos, int D,
                                                              double log2_base, float* __restrict__ x,
                                                              bf16_t* __restrict__ n, float2* __restrict__ cs) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    int t = tok[r];
    if (t < 0 || t >= V) t = 0;
    const bf16_t* e = E + (size_t)t * H;
    float* xr = x + (size_t)r * H;
    float ss = 0.f;
    for (int j = threadIdx.x * 4; j < H; j += 256 * 4) {
        const uint2 w = *(const uint2*)(e + j);
        const f32x4 v = (f32x4){bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        *(f32x4*)(xr + j) = v;
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    const int half = D / 2;
    for (int i = threadIdx.x; i < half; i += 256) {
        const double ang = (double)pos[r] * exp2(-2.0 * (double)i / (double)D * log2_base);
        double sn, c;
        sincos(ang, &sn, &c);
        cs[(size_t)r * half + i] = make_float2((float)c, (float)sn);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
    for (int j = threadIdx.x * 4; j < H; j += 256 * 4) {
        const f32x4 v = *(const f32x4*)(xr + j);
        *(uint2*)(n + (size_t)r * H + j) = (uint2){(uint32_t)f32_to_bf16(v.x * rs) | ((uint32_t)f32_to_bf16(v.y * rs) << 16),
                                                   (uint32_t)f32_to_bf16(v.z * rs) | ((uint32_t)f32_to_bf16(v.w * rs) << 16)};
    }
}

// out[e] = float(in[e])
__global__ __launch_bounds__(256) void widen_bf16_kernel(const bf16_t* __restrict__ in, size_t n, float* __restrict__ out) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        out[e] = bf16_to_f32(in[e]);
}

// a = sum over s < S of part[s * stride + off_a] (b likewise at off_b), added
// in order of s; the loads go out four splits at a time for both sums
// together (one memory round trip per four splits instead of one per split)
__device__ __forceinline__ void sum_splits2(const float* __restrict__ part, int S, size_t stride, size_t off_a,
                                            size_t off_b, float& a, float& b) {
    a = 0.f;
    b = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
        float ta[4], tb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = s0 + u < S;
            ta[u] = in ? part[(size_t)(s0 + u) * stride + off_a] : 0.f;
            tb[u] = in ? part[(size_t)(s0 + u) * stride + off_b] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (s0 + u < S) {
                a += ta[u];
                b += tb[u];
            }
    }
}

// cs[r][i] = (cos, sin) of the angle pos[r] * base^(-2i/D), computed in double
// (the RoPE building-block call; the verify pass takes the same table from
// embed_norm_rope_kernel, once per call, since every layer rotates at the
// same positions).
__global__ void rope_table_kernel(const int32_t* __restrict__ pos, int D, double log2_base, float2* __restrict__ cs) {
    const int r = blockIdx.x, half = D / 2;
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        const double ang = (double)pos[r] * exp2(-2.0 * (double)i / (double)D * log2_base);
        double sn, c;
        sincos(ang, &sn, &c);
        cs[(size_t)r * half + i] = make_float2((float)c, (float)sn);
    }
}

// Block (r, head): sum the S partials of node r's q|k|v columns of one head;
// heads 0..nH-1 (q) and nH..nH+nKV-1 (k) rotate the pair (i, i + D/2) by the
// table angle; the last nKV heads are v.  Stores bf16 q [R][nH][D], k and v
// [R][nKV][D].  blockDim = D / 2.
__global__ __launch_bounds__(64) void qkv_rope_kernel(const float* __restrict__ part, int S, int R, int nH, int nKV,
                                                      int D, const float2* __restrict__ cs, bf16_t* __restrict__ q,
                                                      bf16_t* __restrict__ k, bf16_t* __restrict__ v) {
    const int r = blockIdx.x, head = blockIdx.y, i = threadIdx.x;
    const int half = D / 2;
    const int ncols = (nH + 2 * nKV) * D;
    const size_t stride = (size_t)R * ncols;
    const size_t c0 = (size_t)r * ncols + (size_t)head * D + i;
    float x1, x2;
    sum_splits2(part, S, stride, c0, c0 + half, x1, x2);
    if (head >= nH + nKV) {
        bf16_t* dst = v + ((size_t)r * nKV + (head - nH - nKV)) * D;
        dst[i] = f32_to_bf16(x1);
        dst[i + half] = f32_to_bf16(x2);
        return;
    }
    const float2 t = cs[(size_t)r * half + i];
    const float y1 = x1 * t.x - x2 * t.y;
    const float y2 = x2 * t.x + x1 * t.y;
    bf16_t* dst = head < nH ? q + ((size_t)r * nH + head) * D : k + ((size_t)r * nKV + (head - nH)) * D;
    dst[i] = f32_to_bf16(y1);
    dst[i + half] = f32_to_bf16(y2);
}

// One block per row r: x[r] += sum of the S partials of row r ([S][R][H]),
// then n[r] = bf16(x[r] * rsqrt(mean(x[r]^2) + eps)).  The row stays in
// registers between the two passes (H <= 16384 with 512 threads).
constexpr int RN_THREADS = 512;
__global__ __launch_bounds__(RN_THREADS) void residual_rmsnorm_kernel(const float* __restrict__ part, int S, int R,
                                                                      int H, float eps, float* __restrict__ x,
                                                                      bf16_t* __restrict__ n) {
    __shared__ float red[RN_THREADS / 64];
    const int r = blockIdx.x;
    float* xr = x + (size_t)r * H;
    const size_t stride = (size_t)R * H;
    // the thread's pieces of the row and of four splits at a time are all
    // requested before the first is added (the splits in order of s)
    f32x4 xv[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int j = (it * RN_THREADS + threadIdx.x) * 4;
        xv[it] = j < H ? *(const f32x4*)(xr + j) : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < S; s0 += 4) {
        f32x4 pv[8][4];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int j = (it * RN_THREADS + threadIdx.x) * 4;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                pv[it][u] = j < H && s0 + u < S ? *(const f32x4*)(part + (size_t)(s0 + u) * stride + (size_t)r * H + j)
                                                : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (s0 + u < S) xv[it] += pv[it][u];
    }
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int j = (it * RN_THREADS + threadIdx.x) * 4;
        if (j < H) {
            const f32x4 a = xv[it];
            *(f32x4*)(xr + j) = a;
            ss = fmaf(a.x, a.x, ss);
            ss = fmaf(a.y, a.y, ss);
            ss = fmaf(a.z, a.z, ss);
            ss = fmaf(a.w, a.w, ss);
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < RN_THREADS / 64; ++w) tot += red[w];
    const float rs = rsqrtf(tot / (float)H + eps);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int j = (it * RN_THREADS + threadIdx.x) * 4;
        if (j < H) {
            const f32x4 a = xv[it];
            *(uint2*)(n + (size_t)r * H + j) =
                (uint2){(uint32_t)f32_to_bf16(a.x * rs) | ((uint32_t)f32_to_bf16(a.y * rs) << 16),
                        (uint32_t)f32_to_bf16(a.z * rs) | ((uint32_t)f32_to_bf16(a.w * rs) << 16)};
        }
    }
}

// a[r][c] = bf16(SiLU(g) * u) from the summed gate|up partials [S][R][2F],
// whose columns interleave gate and up in blocks of 16: g at column
// 32 (c / 16) + c % 16, u 16 columns later.  Grid (ceil(F / 256), R).  (An
// unsplit gate|up product applies this in its own epilogue instead.)
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ part, int S, int R, int F,
                                                     bf16_t* __restrict__ a) {
    const int r = blockIdx.y;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= F) return;
    const size_t stride = (size_t)R * 2 * F;
    const size_t row = (size_t)r * 2 * F;
    const size_t gc = row + (size_t)(c / 16) * 32 + c % 16;
    float g, u;
    sum_splits2(part, S, stride, gc, gc + 16, g, u);
    a[(size_t)r * F + c] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct GemmSplit {
    int S;      // splits of the contraction
    int cps;    // k-chunks per split
    int waves;  // waves per workgroup (16 weight rows each)
};

// Workgroup shape and splits of the contraction (whole k-chunks each, at most
// 16), from a cost model measured on the Llama-7B projections with 64 node
// rows: a product runs one workgroup per CU per round, so it takes about
// rounds x (16-row weight blocks per workgroup) x (k-chunks per split), and
// every split beyond the first costs ~3% more (its fp32 partial sums).  Over
// 4, 6 and 8 waves per workgroup this picks q|k|v (768 blocks): 6 waves x 2
// splits = 256 workgroups (23.4 us against 25.2 with 8 waves, which leave 64
// CUs idle); gate|up (1376 blocks, unsplit for the SwiGLU epilogue): 6 waves,
// 230 workgroups (37.2 us against 40.0 with 8 waves on 172 CUs); o and down
// (256 blocks): 4 waves x 4 splits.  A split gate|up also needs its own SwiGLU
// kernel: split_extra = 50 (about 5 us in the same units) is added to its cost,
// so only narrow gate|up products with long rows split.
constexpr int GPU_CUS = 256;
constexpr double GATE_UP_SPLIT_EXTRA = 50.0;
static GemmSplit gemm_split(int R, int K, int ncols, double split_extra = 0.0) {
    const int nblk = lmh_nblk(R);
    const int nchunk = K / lmh_kc(nblk);
    const long long node_tiles = (R + nblk * 16 - 1) / (nblk * 16);
    const long long nrb = (ncols + 15) / 16;
    GemmSplit best{1, nchunk, LMH_WAVES};
    double best_cost = -1.0;
    for (int waves : {4, 6, 8}) {
        for (int S = 1; S <= std::min(16, nchunk); ++S) {
            const int cps = (nchunk + S - 1) / S;
            const int Se = (nchunk + cps - 1) / cps;
            const long long wgs = (nrb + waves - 1) / waves * node_tiles * Se;
            const long long rounds = (wgs + GPU_CUS - 1) / GPU_CUS;
            const double cost = (double)rounds * waves * cps * (1.0 + 0.03 * (Se - 1)) + (Se > 1 ? split_extra : 0.0);
            if (best_cost < 0 || cost < best_cost - 1e-9) {
                best_cost = cost;
                best = GemmSplit{Se, cps, waves};
            }
        }
    }
    return best;
}

static void launch_skinny_partial(const bf16_t* n, const bf16_t* w, int R, int K, int ncols, const GemmSplit& sp,
                                  float* part, hipStream_t s, const char* name) {
    const int nblk = lmh_nblk(R);
    const dim3 grid((ncols + 16 * sp.waves - 1) / (16 * sp.waves), (R + nblk * 16 - 1) / (nblk * 16), sp.S);
#define SKINNY_PARTIAL_LAUNCH(NB, WV)                                                                              \
    MEDUSA_LAUNCH(name, (skinny_mfma_kernel<NB, SKINNY_PARTIAL, WV>), grid, dim3(WV * 64), 0, s, n, w, R, K, ncols, \
                  sp.cps, nullptr, nullptr, part)
    if (sp.waves == 8) {
        if (nblk == 4) SKINNY_PARTIAL_LAUNCH(4, 8);
        else if (nblk == 8) SKINNY_PARTIAL_LAUNCH(8, 8);
        else SKINNY_PARTIAL_LAUNCH(16, 8);
    } else if (sp.waves == 6) {
        if (nblk == 4) SKINNY_PARTIAL_LAUNCH(4, 6);
        else if (nblk == 8) SKINNY_PARTIAL_LAUNCH(8, 6);
        else SKINNY_PARTIAL_LAUNCH(16, 6);
    } else {
        if (nblk == 4) SKINNY_PARTIAL_LAUNCH(4, 4);
        else if (nblk == 8) SKINNY_PARTIAL_LAUNCH(8, 4);
        else SKINNY_PARTIAL_LAUNCH(16, 4);
    }
#undef SKINNY_PARTIAL_LAUNCH
}

// unsplit gate|up product with the SwiGLU epilogue: a = bf16(SiLU(g) * u)
static void launch_skinny_swiglu(const bf16_t* n, const bf16_t* w, int R, int K, int F, const GemmSplit& sp, bf16_t* a,
                                 hipStream_t s) {
    const int nblk = lmh_nblk(R);
    const dim3 grid((2 * F + 16 * sp.waves - 1) / (16 * sp.waves), (R + nblk * 16 - 1) / (nblk * 16), 1);
    float* out = (float*)a;
#define SKINNY_SWIGLU_LAUNCH(NB, WV)                                                                             \
    MEDUSA_LAUNCH("dec_gemm_gate_up", (skinny_mfma_kernel<NB, SKINNY_SWIGLU, WV>), grid, dim3(WV * 64), 0, s, n, w, \
                  R, K, 2 * F, sp.cps, nullptr, nullptr, out)
    if (sp.waves == 8) {
        if (nblk == 4) SKINNY_SWIGLU_LAUNCH(4, 8);
        else if (nblk == 8) SKINNY_SWIGLU_LAUNCH(8, 8);
        else SKINNY_SWIGLU_LAUNCH(16, 8);
    } else if (sp.waves == 6) {
        if (nblk == 4) SKINNY_SWIGLU_LAUNCH(4, 6);
        else if (nblk == 8) SKINNY_SWIGLU_LAUNCH(8, 6);
        else SKINNY_SWIGLU_LAUNCH(16, 6);
    } else {
        if (nblk == 4) SKINNY_SWIGLU_LAUNCH(4, 4);
        else if (nblk == 8) SKINNY_SWIGLU_LAUNCH(8, 4);
        else SKINNY_SWIGLU_LAUNCH(16, 4);
    }
#undef SKINNY_SWIGLU_LAUNCH
}

static size_t a256(size_t x) { return (x + 255) / 256 * 256; }

struct DecoderWs {
    float* x;
    bf16_t *n, *q, *kt, *vt, *o, *a;
    float* part;
    float *att_o, *att_ml;
    float2* rope;
    void* greedy_ws;
};

static size_t partial_floats(int R, int H, int nH, int nKV, int D, int F) {
    size_t m = 0;
    const int qkv = (nH + 2 * nKV) * D;
    const GemmSplit a = gemm_split(R, H, qkv), b = gemm_split(R, nH * D, H),
                    c = gemm_split(R, H, 2 * F, GATE_UP_SPLIT_EXTRA), d = gemm_split(R, F, H);
    m = std::max(m, (size_t)a.S * R * qkv);
    m = std::max(m, (size_t)b.S * R * H);
    m = std::max(m, (size_t)c.S * R * 2 * F);
    m = std::max(m, (size_t)d.S * R * H);
    return m;
}

size_t decoder_workspace_bytes(int B, int N, int H, int nH, int nKV, int D, int F, int V, int max_cache_len) {
    const size_t R = (size_t)B * N;
    return a256(R * H * 4) + a256(R * H * 2) + a256(R * nH * D * 2) + 2 * a256(R * nKV * D * 2) + a256(R * H * 2) +
           a256(R * F * 2) + a256(partial_floats((int)R, H, nH, nKV, D, F) * 4) +
           a256(attn_workspace_bytes(B, nH, N, D, max_cache_len, true)) + a256(R * (D / 2) * sizeof(float2)) +
           a256(lm_head_greedy_workspace_bytes((int)R, H, V));
}

static DecoderWs carve(void* ws, int B, int N, int H, int nH, int nKV, int D, int F, int max_cache_len) {
    const size_t R = (size_t)B * N;
    char* p = (char*)ws;
    DecoderWs w;
    w.x = (float*)p; p += a256(R * H * 4);
    w.n = (bf16_t*)p; p += a256(R * H * 2);
    w.q = (bf16_t*)p; p += a256(R * nH * D * 2);
    w.kt = (bf16_t*)p; p += a256(R * nKV * D * 2);
    w.vt = (bf16_t*)p; p += a256(R * nKV * D * 2);
    w.o = (bf16_t*)p; p += a256(R * H * 2);
    w.a = (bf16_t*)p; p += a256(R * F * 2);
    w.part = (float*)p; p += a256(partial_floats((int)R, H, nH, nKV, D, F) * 4);
    attn_carve(B, nH, N, D, max_cache_len, true, p, &w.att_o, &w.att_ml);
    p += a256(attn_workspace_bytes(B, nH, N, D, max_cache_len, true));
    w.rope = (float2*)p; p += a256(R * (D / 2) * sizeof(float2));
    w.greedy_ws = p;
    return w;
}

// packed weights of one layer: q|k|v stacked ((nH + 2 nKV) D rows of H),
// o (H rows of nH D), gate|up interleaved in 16-row blocks (2F rows of H),
// down (H rows of F)
struct LayerPtrs {
    const bf16_t *wqkv, *wo, *w_gate_up, *w_down;
};

void launch_decoder_verify(const LayerPtrs* layers, int n_layers, const bf16_t* E, const bf16_t* lm_head,
                           const TreeDev& t, const int32_t* node_tok, const int32_t* node_pos,
                           const int32_t* cache_len, int max_cache_len, bf16_t* k_cache, bf16_t* v_cache,
                           int64_t layer_stride, int B, int H, int nH, int nKV, int D, int F, int V, int Lmax,
                           float eps, float rope_base, int32_t* greedy, float* hidden, void* ws, hipStream_t s) {
    const int N = t.N;
    const int R = B * N;
    const DecoderWs w = carve(ws, B, N, H, nH, nKV, D, F, max_cache_len);
    const int qkv = (nH + 2 * nKV) * D;
    const GemmSplit sp_qkv = gemm_split(R, H, qkv), sp_o = gemm_split(R, nH * D, H),
                    sp_gu = gemm_split(R, H, 2 * F, GATE_UP_SPLIT_EXTRA), sp_d = gemm_split(R, F, H);
    const float scale = 1.0f / sqrtf((float)D);
    const double log2_base = log2((double)rope_base);
    const int ew_blocks = 1024;

    MEDUSA_LAUNCH("embed_norm_rope", embed_norm_rope_kernel, dim3(R), dim3(256), 0, s, node_tok, E, H, V, eps,
                  node_pos, D, log2_base, w.x, w.n, w.rope);
    for (int l = 0; l < n_layers; ++l) {
        // w.n holds bf16(RMSNorm(x)) of the layer input
        const LayerPtrs& L = layers[l];
        bf16_t* kc = k_cache + (size_t)l * layer_stride;
        bf16_t* vc = v_cache + (size_t)l * layer_stride;
        launch_skinny_partial(w.n, L.wqkv, R, H, qkv, sp_qkv, w.part, s, "dec_gemm_qkv");
        MEDUSA_LAUNCH("qkv_rope", qkv_rope_kernel, dim3(R, nH + 2 * nKV), dim3(D / 2), 0, s, w.part, sp_qkv.S, R, nH,
                      nKV, D, w.rope, w.q, w.kt, w.vt);
        launch_tree_attention(w.q, w.kt, w.vt, kc, vc, cache_len, max_cache_len, t, B, nH, nKV, D, Lmax, scale, true,
                              w.o, w.att_o, w.att_ml, s, 0);
        launch_skinny_partial(w.o, L.wo, R, nH * D, H, sp_o, w.part, s, "dec_gemm_o");
        MEDUSA_LAUNCH("residual_rmsnorm", residual_rmsnorm_kernel, dim3(R), dim3(RN_THREADS), 0, s, w.part, sp_o.S, R,
                      H, eps, w.x, w.n);
        if (sp_gu.S == 1) {
            launch_skinny_swiglu(w.n, L.w_gate_up, R, H, F, sp_gu, w.a, s);
        } else {
            launch_skinny_partial(w.n, L.w_gate_up, R, H, 2 * F, sp_gu, w.part, s, "dec_gemm_gate_up");
            MEDUSA_LAUNCH("swiglu", swiglu_kernel, dim3((F + 255) / 256, R), dim3(256), 0, s, w.part, sp_gu.S, R, F,
                          w.a);
        }
        launch_skinny_partial(w.a, L.w_down, R, F, H, sp_d, w.part, s, "dec_gemm_down");
        MEDUSA_LAUNCH("residual_rmsnorm", residual_rmsnorm_kernel, dim3(R), dim3(RN_THREADS), 0, s, w.part, sp_d.S, R,
                      H, eps, w.x, w.n);
    }
    launch_lm_head_greedy(w.n, lm_head, R, H, V, greedy, w.greedy_ws, s);
    if (hidden != nullptr) {
        // the final normalised rows, widened to fp32
        MEDUSA_LAUNCH("widen_rows", widen_bf16_kernel, dim3(ew_blocks), dim3(256), 0, s, w.n, (size_t)R * H, hidden);
    }
}

// ---------------------------------------------------------------------------
// Prefill: a prompt of T tokens through the same pass, C tokens at a time,
// the tree a chain of C nodes (each token sees the prefix and the chunk's
// earlier tokens: causal attention).  Pass j covers prompt tokens jC ..
// jC + C - 1 at prefix length cache_len + jC; the last pass is padded with
// copies of the last token, whose keys/values land past the new cache
// length, where no prompt token can see them.  After the last pass the
// greedy choice and final normalised row of the last prompt token are the
// first round's root and heads input, and the cache length grows by T.
// ---------------------------------------------------------------------------

// node_tok / node_pos / prefix length of pass j (one block per sequence)
__global__ __launch_bounds__(256) void prefill_chunk_kernel(const int32_t* __restrict__ tokens, int T, int C, int j,
                                                            const int32_t* __restrict__ cache_len,
                                                            int32_t* __restrict__ node_tok,
                                                            int32_t* __restrict__ node_pos,
                                                            int32_t* __restrict__ prefix) {
    const int b = blockIdx.x;
    const int P = cache_len[b] + j * C;
    for (int i = threadIdx.x; i < C; i += blockDim.x) {
        const int t = min(j * C + i, T - 1);
        node_tok[(size_t)b * C + i] = tokens[(size_t)b * T + t];
        node_pos[(size_t)b * C + i] = P + i;
    }
    if (threadIdx.x == 0) prefix[b] = P;
}

// after the last pass (row = the last prompt token's node): the next token,
// the heads' input (in T's storage; the row's values are bf16, so exact), the
// new cache length
template <typename TO>
__global__ __launch_bounds__(256) void prefill_finish_kernel(const int32_t* __restrict__ greedy,
                                                             const float* __restrict__ hidden, int C, int H, int row,
                                                             int T, int32_t* __restrict__ next_tok,
                                                             TO* __restrict__ h_out,
                                                             int32_t* __restrict__ cache_len) {
    const int b = blockIdx.x;
    const float* src = hidden + ((size_t)b * C + row) * H;
    for (int c = threadIdx.x; c < H; c += blockDim.x) Elem<TO>::store(h_out, (size_t)b * H + c, src[c]);
    if (threadIdx.x == 0) {
        next_tok[b] = greedy[(size_t)b * C + row];
        cache_len[b] += T;
    }
}

size_t prefill_workspace_bytes(int B, int C, int H, int nH, int nKV, int D, int F, int V, int T, int max_cache_len) {
    const int passes = (T + C - 1) / C;
    const size_t BC = (size_t)B * C;
    return 3 * a256(BC * 4) + a256((size_t)B * 4) + a256(BC * H * 4) +
           decoder_workspace_bytes(B, C, H, nH, nKV, D, F, V, max_cache_len + (passes - 1) * C);
}

void launch_prefill(const LayerPtrs* layers, int n_layers, const bf16_t* E, const bf16_t* lm_head, const TreeDev& chain,
                    const int32_t* tokens, int T, int32_t* cache_len, int max_cache_len, bf16_t* k_cache,
                    bf16_t* v_cache, int64_t layer_stride, int B, int H, int nH, int nKV, int D, int F, int V,
                    int Lmax, float eps, float rope_base, int32_t* next_tok, void* h_out, bool h_bf16, void* ws,
                    hipStream_t s) {
    const int C = chain.N;
    const int passes = (T + C - 1) / C;
    const size_t BC = (size_t)B * C;
    char* p = (char*)ws;
    int32_t* node_tok = (int32_t*)p; p += a256(BC * 4);
    int32_t* node_pos = (int32_t*)p; p += a256(BC * 4);
    int32_t* greedy = (int32_t*)p; p += a256(BC * 4);
    int32_t* prefix = (int32_t*)p; p += a256((size_t)B * 4);
    float* hidden = (float*)p; p += a256(BC * H * 4);
    void* dws = p;  // sized for the largest prefix bound of any pass
    const int max_len_last = max_cache_len + (passes - 1) * C;
    for (int j = 0; j < passes; ++j) {
        MEDUSA_LAUNCH("prefill_chunk", prefill_chunk_kernel, dim3(B), dim3(256), 0, s, tokens, T, C, j, cache_len,
                      node_tok, node_pos, prefix);
        // every pass carves the workspace for the last pass's bound, so the
        // carving is the same in all passes
        launch_decoder_verify(layers, n_layers, E, lm_head, chain, node_tok, node_pos, prefix, max_len_last, k_cache,
                              v_cache, layer_stride, B, H, nH, nKV, D, F, V, Lmax, eps, rope_base, greedy,
                              j == passes - 1 ? hidden : nullptr, dws, s);
    }
    const int row = T - 1 - (passes - 1) * C;
    if (h_bf16)
        MEDUSA_LAUNCH("prefill_finish", prefill_finish_kernel<bf16_t>, dim3(B), dim3(256), 0, s, greedy, hidden, C, H,
                      row, T, next_tok, (bf16_t*)h_out, cache_len);
    else
        MEDUSA_LAUNCH("prefill_finish", prefill_finish_kernel<float>, dim3(B), dim3(256), 0, s, greedy, hidden, C, H,
                      row, T, next_tok, (float*)h_out, cache_len);
}

// ---------------------------------------------------------------------------
// The layer's building blocks as calls of their own (same kernels as above;
// shapes checked by the caller)
// ---------------------------------------------------------------------------

// out[e] = sum over the S splits of part[s][e], e < n
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int S, size_t n,
                                                         float* __restrict__ out) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        float v, unused;
        sum_splits2(part, S, n, e, e, v, unused);
        out[e] = v;
    }
}

// out [R][ncols] fp32 = n [R][K] (bf16) times the packed weights' rows; the
// contraction is split as in the layer, the partial sums added by a second
// kernel (workspace: the partials, none when the product is unsplit)
size_t skinny_gemm_workspace_bytes(int R, int K, int ncols) {
    const GemmSplit sp = gemm_split(R, K, ncols);
    return sp.S > 1 ? (size_t)sp.S * R * ncols * sizeof(float) : 0;
}

void launch_skinny_gemm(const bf16_t* n, const bf16_t* w, int R, int K, int ncols, float* out, void* ws,
                        hipStream_t s) {
    const GemmSplit sp = gemm_split(R, K, ncols);
    if (sp.S == 1) {
        launch_skinny_partial(n, w, R, K, ncols, sp, out, s, "gemm_skinny");
        return;
    }
    float* part = (float*)ws;
    launch_skinny_partial(n, w, R, K, ncols, sp, part, s, "gemm_skinny");
    const size_t total = (size_t)R * ncols;
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    MEDUSA_LAUNCH("sum_splits", sum_splits_kernel, dim3(blocks), dim3(256), 0, s, part, sp.S, total, out);
}

void launch_embed(const int32_t* tok, const bf16_t* E, int R, int H, int V, float* x, hipStream_t s) {
    MEDUSA_LAUNCH("embed_rows", embed_rows_kernel, dim3(R), dim3(256), 0, s, tok, E, H, V, x);
}

void launch_rmsnorm_f32_bf16(const float* x, int R, int H, float eps, bf16_t* n, hipStream_t s) {
    MEDUSA_LAUNCH("rmsnorm_f32", rmsnorm_f32_bf16_kernel, dim3(R), dim3(256), 0, s, x, H, eps, n);
}

size_t rope_workspace_bytes(int R, int D) { return (size_t)R * (D / 2) * sizeof(float2); }

// q|k|v fp32 [R][(nH + 2 nKV) D] -> bf16 q [R][nH][D], k, v [R][nKV][D],
// q and k rotated at pos[r] (the angle table in the workspace)
void launch_rope(const float* qkv, const int32_t* pos, int R, int nH, int nKV, int D, float rope_base, bf16_t* q,
                 bf16_t* k, bf16_t* v, void* ws, hipStream_t s) {
    float2* cs = (float2*)ws;
    MEDUSA_LAUNCH("rope_table", rope_table_kernel, dim3(R), dim3(64), 0, s, pos, D, log2((double)rope_base), cs);
    MEDUSA_LAUNCH("qkv_rope", qkv_rope_kernel, dim3(R, nH + 2 * nKV), dim3(D / 2), 0, s, qkv, 1, R, nH, nKV, D, cs, q,
                  k, v);
}

// a [R][F] bf16 = SiLU(gate) * up from the fp32 product [R][2F] whose columns
// interleave gate and up in blocks of 16
void launch_swiglu(const float* gate_up, int R, int F, bf16_t* a, hipStream_t s) {
    MEDUSA_LAUNCH("swiglu", swiglu_kernel, dim3((F + 255) / 256, R), dim3(256), 0, s, gate_up, 1, R, F, a);
}

}  // namespace medusa
