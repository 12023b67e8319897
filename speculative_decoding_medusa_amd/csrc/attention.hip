// Tree-masked attention (step a4): every tree node attends to the cache
// prefix plus its own ancestors-or-self.
//
// Split-KV layout: grid (B * nH, S, query blocks).  Split s of sequence b
// covers keys [s * KPS, (s+1) * KPS) of the key space "prefix (cache_len[b]
// keys) followed by the N tree keys"; tree keys come straight from k_tree /
// v_tree and are visible to query i only where bit j of its ancestor row is
// set.  Each split keeps an online-softmax state (running max m, running sum l,
// unnormalised output) in base-2 exponent form, written as a partial; a
// combine kernel rescales and sums the partials.  Split 0 / query block 0 of
// every KV head also copies the tree keys/values into cache slots
// cache_len .. cache_len + N - 1.
//
// This is the vector-ALU variant (float32 or bf16 storage, float32 math).
#include "common.hpp"
#include "tree.hpp"

namespace medusa {

constexpr int ATT_THREADS = 256;
constexpr int ATT_QB = 16;   // queries per workgroup
constexpr int ATT_TK = 32;   // keys per tile

template <typename T, int D>
__global__ __launch_bounds__(ATT_THREADS) void tree_attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k_tree, const T* __restrict__ v_tree,
    T* __restrict__ k_cache, T* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    const uint64_t* __restrict__ mask, int N, int W, int nH, int nKV, int Lmax, int max_cache_len,
    float scale_log2, int KPS, float* __restrict__ part_o, float* __restrict__ part_ml) {
    constexpr int DE = D / 16;  // output columns per thread
    __shared__ float qs[ATT_QB][D];
    __shared__ float ks[ATT_TK][D + 1];
    __shared__ float vs[ATT_TK][D];
    __shared__ float ps[ATT_QB][ATT_TK];

    const int bh = blockIdx.x;
    const int b = bh / nH, h = bh - b * nH;
    const int grp = nH / nKV;
    const int kvh = h / grp;
    const int S = gridDim.y;
    const int s = blockIdx.y;
    const int q0 = blockIdx.z * ATT_QB;
    const int tid = threadIdx.x;
    // cache lengths above the host-declared bound are clamped (never read past Lmax)
    const int P = max(0, min(cache_len[b], max_cache_len));
    const int total = P + N;

    // tree K/V -> cache slots P..P+N-1 (one writer per KV head)
    if (s == 0 && blockIdx.z == 0 && h % grp == 0) {
        for (int e = tid; e < N * D; e += ATT_THREADS) {
            const int t = e / D, c = e - t * D;
            const size_t src = (((size_t)b * N + t) * nKV + kvh) * D + c;
            const size_t dst = (((size_t)b * nKV + kvh) * Lmax + P + t) * D + c;
            k_cache[dst] = k_tree[src];
            v_cache[dst] = v_tree[src];
        }
    }

    for (int e = tid; e < ATT_QB * D; e += ATT_THREADS) {
        const int qi = e / D, c = e - qi * D;
        const int i = q0 + qi;
        qs[qi][c] = i < N ? Elem<T>::load(q, (((size_t)b * N + i) * nH + h) * D + c) : 0.f;
    }

    const int qi = tid >> 4;        // query row of this thread (scores, softmax, output)
    const int kj = tid & 15;        // key columns kj and kj + 16 of a tile; output columns kj + 16 e
    const int i = q0 + qi;
    float m = -INFINITY, l = 0.f;
    float o[DE];
#pragma unroll
    for (int e = 0; e < DE; ++e) o[e] = 0.f;

    const int k_begin = s * KPS;
    const int k_end = min(total, k_begin + KPS);
    for (int t0 = k_begin; t0 < k_end; t0 += ATT_TK) {
        __syncthreads();
        for (int e = tid; e < ATT_TK * D; e += ATT_THREADS) {
            const int r = e / D, c = e - r * D;
            const int j = t0 + r;
            float kv = 0.f, vv = 0.f;
            if (j < k_end) {
                if (j < P) {
                    const size_t off = (((size_t)b * nKV + kvh) * Lmax + j) * D + c;
                    kv = Elem<T>::load(k_cache, off);
                    vv = Elem<T>::load(v_cache, off);
                } else {
                    const size_t off = (((size_t)b * N + (j - P)) * nKV + kvh) * D + c;
                    kv = Elem<T>::load(k_tree, off);
                    vv = Elem<T>::load(v_tree, off);
                }
            }
            ks[r][c] = kv;
            vs[r][c] = vv;
        }
        __syncthreads();
        float sc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int r = kj + 16 * u;
            const int j = t0 + r;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < D; ++c) acc = fmaf(qs[qi][c], ks[r][c], acc);
            bool vis = j < k_end && i < N;
            if (vis && j >= P) {
                const int t = j - P;
                vis = (mask[(size_t)i * W + (t >> 6)] >> (t & 63)) & 1ull;
            }
            sc[u] = vis ? acc * scale_log2 : -INFINITY;
        }
        float tmax = fmaxf(sc[0], sc[1]);
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, w, 16));
        const float m_new = fmaxf(m, tmax);
        float p0 = 0.f, p1 = 0.f, alpha = 1.f;
        if (m_new != -INFINITY) {
            p0 = exp2f(sc[0] - m_new);
            p1 = exp2f(sc[1] - m_new);
            alpha = exp2f(m - m_new);
        }
        float psum = p0 + p1;
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) psum += __shfl_xor(psum, w, 16);
        l = l * alpha + psum;
        m = m_new;
        ps[qi][kj] = p0;
        ps[qi][kj + 16] = p1;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < DE; ++e) {
            float acc = o[e] * alpha;
            const int c = kj + 16 * e;
#pragma unroll 8
            for (int r = 0; r < ATT_TK; ++r) acc = fmaf(ps[qi][r], vs[r][c], acc);
            o[e] = acc;
        }
    }
    if (i < N) {
        const size_t pr = (((size_t)bh * S + s) * N + i);
#pragma unroll
        for (int e = 0; e < DE; ++e) part_o[pr * D + kj + 16 * e] = o[e];
        if (kj == 0) { part_ml[pr * 2] = m; part_ml[pr * 2 + 1] = l; }
    }
}

// out[b][i][h][:] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
template <typename T, int D>
__global__ __launch_bounds__(D) void tree_attn_combine_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml, int S, int N,
                                                              int nH, T* __restrict__ out) {
    const int i = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / nH, h = bh - b * nH;
    const int c = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(((size_t)bh * S + s) * N + i) * 2]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < S; ++s) {
        const size_t pr = ((size_t)bh * S + s) * N + i;
        const float ms = part_ml[pr * 2];
        if (ms == -INFINITY) continue;
        const float f = exp2f(ms - M);
        L += f * part_ml[pr * 2 + 1];
        acc += f * part_o[pr * D + c];
    }
    Elem<T>::store(out, (((size_t)b * N + i) * nH + h) * D + c, acc / L);
}

int attn_splits(int B, int nH, int N, int max_total) {
    const int qblocks = (N + ATT_QB - 1) / ATT_QB;
    const int base = B * nH * qblocks;
    int S = (1024 + base - 1) / base;
    const int max_s = (max_total + ATT_TK - 1) / ATT_TK;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    return S;
}

int attn_keys_per_split(int S, int max_total) {
    int kps = (max_total + S - 1) / S;
    return ((kps + ATT_TK - 1) / ATT_TK) * ATT_TK;
}

void launch_tree_attention(const void* q, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                           const int32_t* cache_len, int max_cache_len, const TreeDev& t, int B, int nH,
                           int nKV, int D, int Lmax, float scale, bool bf16, void* out, float* part_o,
                           float* part_ml, hipStream_t s) {
    const int N = t.N;
    const int max_total = max_cache_len + N;
    const int S = attn_splits(B, nH, N, max_total);
    const int KPS = attn_keys_per_split(S, max_total);
    const dim3 grid(B * nH, S, (N + ATT_QB - 1) / ATT_QB);
    const float scale_log2 = scale * 1.4426950408889634f;
#define MEDUSA_ATT(T, DD)                                                                                   \
    do {                                                                                                    \
        MEDUSA_LAUNCH("tree_attn_split", (tree_attn_valu_kernel<T, DD>), grid, dim3(ATT_THREADS), 0, s,     \
                      (const T*)q, (const T*)k_tree, (const T*)v_tree, (T*)k_cache, (T*)v_cache, cache_len, \
                      t.mask, N, t.W, nH, nKV, Lmax, max_cache_len, scale_log2, KPS, part_o, part_ml);                     \
        MEDUSA_LAUNCH("tree_attn_combine", (tree_attn_combine_kernel<T, DD>), dim3(N, B * nH), dim3(DD), 0, \
                      s, part_o, part_ml, S, N, nH, (T*)out);                                               \
    } while (0)
    if (bf16) {
        if (D == 64) MEDUSA_ATT(bf16_t, 64); else MEDUSA_ATT(bf16_t, 128);
    } else {
        if (D == 64) MEDUSA_ATT(float, 64); else MEDUSA_ATT(float, 128);
    }
#undef MEDUSA_ATT
}

size_t attn_workspace_bytes(int B, int nH, int N, int D, int max_cache_len) {
    const int S = attn_splits(B, nH, N, max_cache_len + N);
    const size_t rows = (size_t)B * nH * S * N;
    return (rows * D * sizeof(float) + 255) / 256 * 256 + rows * 2 * sizeof(float);
}

void attn_carve(int B, int nH, int N, int D, int max_cache_len, void* ws, float** part_o, float** part_ml) {
    const int S = attn_splits(B, nH, N, max_cache_len + N);
    const size_t rows = (size_t)B * nH * S * N;
    *part_o = (float*)ws;
    *part_ml = (float*)((char*)ws + (rows * D * sizeof(float) + 255) / 256 * 256);
}

}  // namespace medusa
