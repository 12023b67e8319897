// Candidate tree (step a3) and greedy longest-branch acceptance with
// accepted-path KV compaction (steps a6 + a7).
#include "common.hpp"
#include "tree.hpp"

namespace medusa {

// node_tok[b][i] = root for i = 0, else topk_idx[b][depth-1][rank];
// node_pos[b][i] = cache_len[b] + depth.  Block b also copies the ancestor
// mask when b == 0.  Every global load is issued before the one barrier:
// the candidates the tree can use (heads 1 .. max_depth, ranks 0 ..
// max_rank; at most 16 x 16) are staged in LDS, so no load waits on another.
__global__ __launch_bounds__(256) void build_tree_kernel(const int* __restrict__ depth,
                                                         const int* __restrict__ rank,
                                                         const uint64_t* __restrict__ mask, int N, int W,
                                                         int max_depth, int max_rank,
                                                         const int32_t* __restrict__ topk_idx,
                                                         int K, int topk, const int32_t* __restrict__ root_tok,
                                                         const int32_t* __restrict__ cache_len,
                                                         int32_t* __restrict__ node_tok,
                                                         int32_t* __restrict__ node_pos,
                                                         uint64_t* __restrict__ anc_mask) {
    __shared__ int tk[MEDUSA_MAX_DEPTH_DEV * MEDUSA_MAX_TOPK_DEV];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int cols = max_rank + 1;  // K >= max_depth and topk > max_rank (checked on the host)
    for (int e = tid; e < max_depth * cols; e += blockDim.x) {
        const int r = e / cols, c = e - r * cols;
        tk[e] = topk_idx[((size_t)b * K + r) * topk + c];
    }
    const int root = root_tok[b];
    const int P = cache_len[b];
    // N <= 256 nodes: one per thread
    const int d = tid < N ? depth[tid] : 0;
    const int rk = tid < N ? rank[tid] : 0;
    if (b == 0 && anc_mask != nullptr)
        for (int i = tid; i < N * W; i += blockDim.x) anc_mask[i] = mask[i];
    __syncthreads();
    if (tid < N) {
        node_tok[(size_t)b * N + tid] = d == 0 ? root : tk[(d - 1) * cols + rk];
        node_pos[(size_t)b * N + tid] = P + d;
    }
}

void launch_build_tree(const TreeDev& t, const int32_t* topk_idx, int K, int topk, const int32_t* root_tok,
                       const int32_t* cache_len, int B, int32_t* node_tok, int32_t* node_pos,
                       uint64_t* anc_mask, hipStream_t s) {
    MEDUSA_LAUNCH("build_tree", build_tree_kernel, dim3(B), dim3(256), 0, s, t.depth, t.rank, t.mask, t.N,
                  t.W, t.max_depth, t.max_rank, topk_idx, K, topk, root_tok, cache_len, node_tok, node_pos,
                  anc_mask);
}

// ---------------------------------------------------------------------------
// Typical acceptance needs the base distribution after every node at the
// sampling temperature T: per logits row, with z = s / T, the maximum m, log Z
// with Z = sum exp(z - m), and the entropy H = log Z - (1/Z) sum exp(z - m)
// (z - m).  One block of 1024 threads per row, one pass: each thread keeps
// (m, Z, A = sum exp(z - m)(z - m)) of the values it reads (16-byte loads,
// four in flight), moving the reference to a larger maximum as it goes, and
// the states are combined across the block.  stats[r] = (m, log Z, H, 0).
// ---------------------------------------------------------------------------
constexpr int STATS_THREADS = 1024;

struct SoftStat {
    float m, Z, A;  // reference, sum exp(z - m), sum exp(z - m)(z - m)
};
// the state of the union of two value sets (either may be empty: Z == 0)
__device__ __forceinline__ SoftStat soft_combine(SoftStat x, SoftStat y) {
    if (x.Z == 0.f) return y;
    if (y.Z == 0.f) return x;
    const float m = fmaxf(x.m, y.m);
    const float fx = __expf(x.m - m), fy = __expf(y.m - m);
    return SoftStat{m, x.Z * fx + y.Z * fy, (x.A + x.Z * (x.m - m)) * fx + (y.A + y.Z * (y.m - m)) * fy};
}
// add n values (-inf ones, the padding, contribute nothing)
template <int NV>
__device__ __forceinline__ void soft_add(SoftStat& st, const float (&z)[NV]) {
    float mb = z[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) mb = fmaxf(mb, z[i]);
    if (mb == -INFINITY) return;
    if (st.Z == 0.f) {
        st = SoftStat{mb, 0.f, 0.f};
    } else if (mb > st.m) {
        const float f = __expf(st.m - mb);
        st.A = (st.A + st.Z * (st.m - mb)) * f;
        st.Z *= f;
        st.m = mb;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (z[i] == -INFINITY) continue;
        const float d = z[i] - st.m;
        const float e = __expf(d);
        st.Z += e;
        st.A = fmaf(e, d, st.A);
    }
}

__global__ __launch_bounds__(STATS_THREADS) void row_softmax_stats_kernel(const float* __restrict__ logits, int V,
                                                                          float inv_t, float4* __restrict__ stats) {
    constexpr int U = 4;  // 16-byte loads in flight per thread
    constexpr int WAVES = STATS_THREADS / 64;
    __shared__ float red[3][WAVES];
    const float* row = logits + (size_t)blockIdx.x * V;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    SoftStat st{0.f, 0.f, 0.f};
    // 16-byte loads over the row's 16-byte-aligned body, scalars around it
    const int head = (int)((4 - ((uintptr_t)row / 4) % 4) % 4) < V ? (int)((4 - ((uintptr_t)row / 4) % 4) % 4) : V;
    const int n4 = (V - head) / 4;
    const f32x4* row4 = (const f32x4*)(row + head);
    for (int i0 = tid; i0 < n4; i0 += U * STATS_THREADS) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * STATS_THREADS;
            v[u] = i < n4 ? row4[i] : (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        float z[4 * U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) z[4 * u + c] = v[u][c] * inv_t;
        soft_add(st, z);
    }
    // the scalars before and after the 16-byte body
    const int tail0 = head + 4 * n4;
    if (tid < head || (tid >= 4 && tail0 + tid - 4 < V)) {
        const float z[1] = {row[tid < head ? tid : tail0 + tid - 4] * inv_t};
        soft_add(st, z);
    }
    // combine across the wave, then across the waves
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const SoftStat other{__shfl_xor(st.m, o, 64), __shfl_xor(st.Z, o, 64), __shfl_xor(st.A, o, 64)};
        st = soft_combine(st, other);
    }
    if (lane == 0) { red[0][wave] = st.m; red[1][wave] = st.Z; red[2][wave] = st.A; }
    __syncthreads();
    if (tid == 0) {
        SoftStat t{red[0][0], red[1][0], red[2][0]};
        for (int w = 1; w < WAVES; ++w) t = soft_combine(t, SoftStat{red[0][w], red[1][w], red[2][w]});
        const float lz = __logf(t.Z);
        stats[blockIdx.x] = make_float4(t.m, lz, lz - t.A / t.Z, 0.f);
    }
}

// Arguments of the typical-acceptance rule (TYPICAL = true below).
struct TypicalArgs {
    const float* logits;  // [B][N][V]: base scores after every node
    const float4* stats;  // [B][N]: row_softmax_stats_kernel's output
    const float* uniform; // [B]: draws the extra token (draw_extra_kernel)
    int V;
    float inv_t, log_eps, log_delta;
};

// ---------------------------------------------------------------------------
// Acceptance + compaction.  Grid (B, S): every block of row b recomputes the
// acceptance of sequence b (N <= 256 nodes, one thread each: walk the chain
// to the root and AND the per-node tests), block (b, 0) writes the results,
// and block (b, s) compacts slice s of the caches: slice = (layer, KV head).
// Within a slice all source rows are read into registers before the barrier
// that precedes any write, so an accepted node that moves onto a slot another
// accepted node is read from cannot corrupt it; slices are disjoint.
// Greedy (TYPICAL = false): node i passes when its token is its parent's
// greedy choice; the extra token is the deepest node's greedy choice.
// Typical: node i passes when log p(token | parent) = s / T - m - log Z of
// the parent's row exceeds min(log eps, log delta - H) of that row; the extra
// token is left to draw_extra_kernel.
// ---------------------------------------------------------------------------
template <typename T, bool TYPICAL>
__global__ __launch_bounds__(256) void accept_compact_kernel(
    const int* __restrict__ parent, const int* __restrict__ depth, int N, int Dmax,
    const int32_t* __restrict__ node_tok, const int32_t* __restrict__ greedy,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes, int32_t* __restrict__ out_tokens,
    const int32_t* __restrict__ cache_len, int32_t* __restrict__ new_cache_len, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int nKV, int D, int Lmax, int64_t layer_stride, int n_slices, TypicalArgs ta,
    int* __restrict__ status) {
    __shared__ int s_best[256 / 64];
    __shared__ int s_par[256], s_tok[256], s_g[256];
    __shared__ int s_path[MEDUSA_MAX_DEPTH_DEV + 1];
    __shared__ int s_L, s_deepest, s_extra;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* tok = node_tok + (size_t)b * N;
    const int P = cache_len[b];

    // the sequence's nodes (N <= 256, one per thread) -> LDS in one round of
    // loads, so the walks below read no global memory; s_g holds the greedy
    // choices (greedy) or the per-node test (typical)
    int dep = 0;
    if (tid < N) {
        s_par[tid] = parent[tid];
        s_tok[tid] = tok[tid];
        dep = depth[tid];
        if constexpr (!TYPICAL) {
            s_g[tid] = greedy[(size_t)b * N + tid];
        } else {
            int pass = 0;
            if (tid > 0) {
                const int a = parent[tid], x = tok[tid];
                const size_t row = (size_t)b * N + a;
                if (x >= 0 && x < ta.V) {
                    const float4 st = ta.stats[row];
                    const float lp = fmaf(ta.logits[row * ta.V + x], ta.inv_t, -st.x) - st.y;
                    pass = lp > fminf(ta.log_eps, ta.log_delta - st.z);
                }
            }
            s_g[tid] = pass;
        }
    }
    __syncthreads();
    // accepted iff every node on the chain to the root passes its test
    int my = -1;
    if (tid < N) {
        bool ok = true;
        int j = tid;
        while (j > 0) {
            const int p = s_par[j];
            ok = ok && (TYPICAL ? s_g[j] != 0 : s_tok[j] == s_g[p]);
            j = p;
        }
        my = ok ? dep : -1;
    }
    // deepest accepted depth, then the lowest node index at that depth: the
    // largest key depth * 2^16 + (2^16 - 1 - index) over the block (the root
    // is always accepted at depth 0; nodes not accepted, and threads past N,
    // hold -1)
    int key = my >= 0 ? (my << 16) | (0xFFFF - tid) : -1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, __shfl_xor(key, m, 64));
    if ((tid & 63) == 0) s_best[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
        int best = s_best[0];
#pragma unroll
        for (int w = 1; w < 256 / 64; ++w) best = max(best, s_best[w]);
        const int L = best >> 16, deepest = 0xFFFF - (best & 0xFFFF);
        s_L = L;
        s_deepest = deepest;
        int j = deepest;
        for (int d = L; d >= 0; --d) { s_path[d] = j; j = d > 0 ? s_par[j] : 0; }
        s_extra = TYPICAL ? -1 : s_g[deepest];  // typical: draw_extra_kernel writes the extra token
    }
    __syncthreads();
    const int L = s_L;
    // caches whose tree slots P..P+N-1 would not fit: nothing is compacted,
    // the length is not advanced, and the tree's status word says so
    const bool overflow = k_cache != nullptr && (P < 0 || P + N > Lmax);

    if (blockIdx.y == 0 && tid <= Dmax) {
        const int d = tid;
        const size_t o = (size_t)b * (Dmax + 1) + d;
        if (d <= L) {
            accept_nodes[o] = s_path[d];
            out_tokens[o] = d < L ? s_tok[s_path[d + 1]] : s_extra;
        } else {
            accept_nodes[o] = -1;
            out_tokens[o] = -1;
        }
        if (d == 0) {
            accept_len[b] = L;
            new_cache_len[b] = overflow ? P : P + L + 1;
            if (overflow && status != nullptr) atomicOr(status, STATUS_CACHE_OVERFLOW);
        }
    }

    // nothing to move, or a cache length that would address past Lmax
    if (k_cache == nullptr || L == 0 || overflow) return;
    // slice s = layer * nKV + kv head
    const int s = blockIdx.y;
    if (s >= n_slices) return;
    const int layer = s / nKV, kvh = s - layer * nKV;
    const size_t base = (size_t)layer * layer_stride + (((size_t)b * nKV + kvh) * Lmax) * D;
    // rows d = 1..L (d = 0 is the root, already in place); elements per row D
    const int total = L * D;
    constexpr int PER_T = 8;  // elements per thread per tensor (L*D <= 16*128 = 2048)
    float kv_k[PER_T], kv_v[PER_T];
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
        const int idx = tid + e * 256;
        if (idx < total) {
            const int d = 1 + idx / D, c = idx - (idx / D) * D;
            const size_t src = base + (size_t)(P + s_path[d]) * D + c;
            kv_k[e] = Elem<T>::load(k_cache, src);
            kv_v[e] = Elem<T>::load(v_cache, src);
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER_T; ++e) {
        const int idx = tid + e * 256;
        if (idx < total) {
            const int d = 1 + idx / D, c = idx - (idx / D) * D;
            const size_t dst = base + (size_t)(P + d) * D + c;
            Elem<T>::store(k_cache, dst, kv_k[e]);
            Elem<T>::store(v_cache, dst, kv_v[e]);
        }
    }
}

// The extra token of typical acceptance: inverse transform sampling from the
// deepest accepted node's row, out_tokens[b][L] = the smallest token index
// whose cumulative weight exp(s / T - m) (index order) exceeds u[b] x the
// row's total.  One block of 1024 threads per sequence; the row is taken in
// chunks of 4096 tokens, thread t holding tokens 4t .. 4t + 3 of each chunk
// (16-byte loads, eight chunks in flight).  The chunk totals come from one
// block reduction per eight chunks; their prefix locates the chunk holding
// the crossing, and one block scan of that chunk the thread and the token.
constexpr int DRAW_THREADS = 1024;
constexpr int DRAW_CHUNK = 4 * DRAW_THREADS;  // tokens per chunk
constexpr int DRAW_GROUP = 8;                 // chunks loaded together
constexpr int DRAW_MAX_CHUNKS = 64;           // rows of up to 64 x 4096 tokens

// Block scan of one value per thread: the thread's exclusive and inclusive
// prefixes and the block total.  Neighbouring threads' intervals [excl, incl)
// meet exactly (the exclusive prefix is the previous lane's inclusive one),
// so exactly one thread's interval holds any point of [0, total).
__device__ __forceinline__ void block_scan(float x, float* wsum, float& excl, float& incl, float& total) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    float xp = __shfl_up(x, 1, 64);
    if (lane == 0) xp = 0.f;
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    float off = 0.f, tot = 0.f;
    for (int w = 0; w < DRAW_THREADS / 64; ++w) {
        const float v = wsum[w];
        if (w < wv) off += v;
        tot += v;
    }
    __syncthreads();  // wsum is reused by the next scan
    excl = off + xp;
    incl = off + x;
    total = tot;
}

// Inverse transform sampling over a row of V non-negative weights held by
// the block (DRAW_THREADS threads): the smallest token index whose cumulative
// weight (index order) exceeds u x the total; wt(j) returns the weights of
// tokens j .. j + 3 (0 past the row).  Chunks of 4096 tokens, thread t holding
// tokens 4t .. 4t + 3 of each: the chunk totals come from one block
// reduction per eight chunks, their prefix locates the chunk holding the
// crossing, one block scan of that chunk the thread and the token.  If float
// rounding leaves u x total past that scan, the chunk's last token.  Every
// thread returns the pick.  V <= DRAW_MAX_CHUNKS x 4096 (checked on the host).
template <typename WF>
__device__ int inverse_cdf_draw(const WF& wt, int V, float u) {
    __shared__ float wsum[DRAW_THREADS / 64];
    __shared__ float red[DRAW_THREADS / 64][DRAW_GROUP];
    __shared__ float s_C[DRAW_MAX_CHUNKS];
    __shared__ float s_base, s_target;
    __shared__ int s_chunk, s_pick;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
    for (int g0 = 0; g0 < nch; g0 += DRAW_GROUP) {
        f32x4 w[DRAW_GROUP];
#pragma unroll
        for (int q = 0; q < DRAW_GROUP; ++q) w[q] = wt((g0 + q) * DRAW_CHUNK + 4 * tid);
#pragma unroll
        for (int q = 0; q < DRAW_GROUP; ++q) {
            const float t = wave_sum((w[q][0] + w[q][1]) + (w[q][2] + w[q][3]));
            if (lane == 0) red[wv][q] = t;
        }
        __syncthreads();
        if (tid < DRAW_GROUP && g0 + tid < nch) {
            float t = 0.f;
            for (int w2 = 0; w2 < DRAW_THREADS / 64; ++w2) t += red[w2][tid];
            s_C[g0 + tid] = t;
        }
        __syncthreads();
    }
    if (tid == 0) {
        float total = 0.f;
        for (int c = 0; c < nch; ++c) total += s_C[c];
        const float target = u * total;
        float run = 0.f;
        int cs = nch - 1;
        for (int c = 0; c < nch; ++c) {
            if (target < run + s_C[c]) { cs = c; break; }
            if (c < nch - 1) run += s_C[c];
        }
        s_chunk = cs;
        s_base = run;
        s_target = target;
        s_pick = min(V, (cs + 1) * DRAW_CHUNK) - 1;
    }
    __syncthreads();
    const int j = s_chunk * DRAW_CHUNK + 4 * tid;
    const f32x4 w4 = wt(j);
    float ex, in, tot;
    block_scan((w4[0] + w4[1]) + (w4[2] + w4[3]), wsum, ex, in, tot);
    const float base = s_base, target = s_target;
    if (base + ex <= target && target < base + in) {
        float run = base + ex;
        int pick = min(j + 3, V - 1);
        for (int e = 0; e < 4; ++e) {
            run += w4[e];
            if (j + e < V && run > target) { pick = j + e; break; }
        }
        s_pick = pick;
    }
    __syncthreads();
    const int pick = s_pick;
    __syncthreads();  // s_pick may be reused by a later draw
    return pick;
}

// 16-byte or scalar loads of 4 consecutive floats of a row (-inf past V)
__device__ __forceinline__ f32x4 load4(const float* row, int j, int V, bool vec, float pad) {
    f32x4 v;
    if (vec && j + 3 < V) {
        v = *(const f32x4*)(row + j);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = j + e < V ? row[j + e] : pad;
    }
    return v;
}

// weights exp(s / T - m) of a scores row
struct SoftmaxWeights {
    const float* lg;
    int V;
    bool vec;
    float inv_t, m;
    __device__ f32x4 operator()(int j) const {
        f32x4 v = load4(lg, j, V, vec, -INFINITY);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __expf(fmaf(v[e], inv_t, -m));  // exp(-inf) = 0
        return v;
    }
};

// weights max(0, p - q) (the residual after a rejection), or p when q is null
struct ResidualWeights {
    const float *p, *q;
    int V;
    bool vec;
    __device__ f32x4 operator()(int j) const {
        f32x4 a = load4(p, j, V, vec, 0.f);
        if (q != nullptr) {
            const f32x4 c = load4(q, j, V, vec, 0.f);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = fmaxf(0.f, a[e] - c[e]);
        }
        return a;
    }
};

__global__ __launch_bounds__(DRAW_THREADS) void draw_extra_kernel(const float* __restrict__ logits,
                                                                  const float4* __restrict__ stats, int N, int V,
                                                                  float inv_t, const float* __restrict__ uniform,
                                                                  const int32_t* __restrict__ accept_len,
                                                                  const int32_t* __restrict__ accept_nodes, int Dmax,
                                                                  int32_t* __restrict__ out_tokens) {
    const int b = blockIdx.x;
    const int L = accept_len[b];
    if (L < 0 || L > Dmax) return;
    const int node = accept_nodes[(size_t)b * (Dmax + 1) + L];
    if (node < 0 || node >= N) return;
    const size_t row = (size_t)b * N + node;
    const float* lg = logits + row * V;
    const SoftmaxWeights wt{lg, V, ((uintptr_t)lg & 15) == 0, inv_t, stats[row].x};
    const int pick = inverse_cdf_draw(wt, V, uniform[b]);
    if (threadIdx.x == 0) out_tokens[(size_t)b * (Dmax + 1) + L] = pick;
}

// ---------------------------------------------------------------------------
// Speculative sampling on a chain of gamma drafts (draft-model speculative
// decoding): draft i is accepted when u_accept q_i(x) < p_i(x), i.e. with
// probability min(1, p/q); the round stops at the first rejection n and draws
// its token from max(0, p_n - q_n) (normalised), or, when all gamma drafts
// pass, the bonus token from p_gamma.  One block per sequence: thread 0
// walks the drafts, then the block draws.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(DRAW_THREADS) void speculative_sample_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ drafts,
    const float* __restrict__ u_accept, const float* __restrict__ u_resample, int gamma, int V,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ out_tokens) {
    __shared__ int s_n;
    const int b = blockIdx.x, tid = threadIdx.x;
    const float* pb = p + (size_t)b * (gamma + 1) * V;
    const float* qb = q + (size_t)b * gamma * V;
    if (tid == 0) {
        int n = gamma;
        for (int i = 0; i < gamma; ++i) {
            const int x = drafts[(size_t)b * gamma + i];
            const bool ok = x >= 0 && x < V && u_accept[(size_t)b * gamma + i] * qb[(size_t)i * V + x] <
                                                   pb[(size_t)i * V + x];
            if (!ok) { n = i; break; }
        }
        s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    const float* pr = pb + (size_t)n * V;
    const float* qr = n < gamma ? qb + (size_t)n * V : nullptr;
    const bool vec = ((uintptr_t)pr & 15) == 0 && (qr == nullptr || ((uintptr_t)qr & 15) == 0);
    const ResidualWeights wt{pr, qr, V, vec};
    const int pick = inverse_cdf_draw(wt, V, u_resample[(size_t)b * (gamma + 1) + n]);
    int32_t* out = out_tokens + (size_t)b * (gamma + 1);
    for (int i = tid; i <= gamma; i += DRAW_THREADS)
        out[i] = i < n ? drafts[(size_t)b * gamma + i] : i == n ? pick : -1;
    if (tid == 0) n_accepted[b] = n;
}

void launch_speculative_sample(const float* p, const float* q, const int32_t* drafts, const float* u_accept,
                               const float* u_resample, int B, int gamma, int V, int32_t* n_accepted,
                               int32_t* out_tokens, hipStream_t s) {
    MEDUSA_LAUNCH("speculative_sample", speculative_sample_kernel, dim3(B), dim3(DRAW_THREADS), 0, s, p, q, drafts,
                  u_accept, u_resample, gamma, V, n_accepted, out_tokens);
}

template <bool TYPICAL>
static void launch_accept_t(const TreeDev& t, const int32_t* node_tok, const int32_t* greedy, int B,
                            int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                            const int32_t* cache_len, int32_t* new_cache_len, void* k_cache, void* v_cache,
                            int n_layers, int64_t layer_stride, int nKV, int D, int Lmax, bool bf16,
                            const TypicalArgs& ta, hipStream_t s) {
    const int n_slices = k_cache ? n_layers * nKV : 1;
    const dim3 grid(B, n_slices);
    const char* name = TYPICAL ? "typical_accept_compact" : "accept_compact";
    if (bf16)
        MEDUSA_LAUNCH(name, (accept_compact_kernel<bf16_t, TYPICAL>), grid, dim3(256), 0, s, t.parent, t.depth,
                      t.N, t.max_depth, node_tok, greedy, accept_len, accept_nodes, out_tokens, cache_len,
                      new_cache_len, (bf16_t*)k_cache, (bf16_t*)v_cache, nKV, D, Lmax, layer_stride, n_slices, ta,
                      t.status);
    else
        MEDUSA_LAUNCH(name, (accept_compact_kernel<float, TYPICAL>), grid, dim3(256), 0, s, t.parent, t.depth,
                      t.N, t.max_depth, node_tok, greedy, accept_len, accept_nodes, out_tokens, cache_len,
                      new_cache_len, (float*)k_cache, (float*)v_cache, nKV, D, Lmax, layer_stride, n_slices, ta,
                      t.status);
}

void launch_accept(const TreeDev& t, const int32_t* node_tok, const int32_t* greedy, int B,
                   int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, const int32_t* cache_len,
                   int32_t* new_cache_len, void* k_cache, void* v_cache, int n_layers, int64_t layer_stride,
                   int nKV, int D, int Lmax, bool bf16, hipStream_t s) {
    launch_accept_t<false>(t, node_tok, greedy, B, accept_len, accept_nodes, out_tokens, cache_len, new_cache_len,
                           k_cache, v_cache, n_layers, layer_stride, nKV, D, Lmax, bf16, TypicalArgs{}, s);
}

size_t typical_accept_workspace_bytes(int B, int N) { return (size_t)B * N * sizeof(float4); }
int typical_max_vocab() { return DRAW_MAX_CHUNKS * DRAW_CHUNK; }

void launch_typical_accept(const TreeDev& t, const int32_t* node_tok, const float* logits, int B, int V,
                           float temperature, float eps, float delta, const float* uniform, int32_t* accept_len,
                           int32_t* accept_nodes, int32_t* out_tokens, const int32_t* cache_len,
                           int32_t* new_cache_len, void* k_cache, void* v_cache, int n_layers, int64_t layer_stride,
                           int nKV, int D, int Lmax, bool bf16, void* ws, hipStream_t s) {
    float4* stats = (float4*)ws;
    const float inv_t = 1.0f / temperature;
    MEDUSA_LAUNCH("row_softmax_stats", row_softmax_stats_kernel, dim3(B * t.N), dim3(STATS_THREADS), 0, s, logits, V,
                  inv_t, stats);
    const TypicalArgs ta{logits, stats, uniform, V, inv_t, logf(eps), logf(delta)};
    launch_accept_t<true>(t, node_tok, nullptr, B, accept_len, accept_nodes, out_tokens, cache_len, new_cache_len,
                          k_cache, v_cache, n_layers, layer_stride, nKV, D, Lmax, bf16, ta, s);
    MEDUSA_LAUNCH("draw_extra", draw_extra_kernel, dim3(B), dim3(DRAW_THREADS), 0, s, logits, stats, t.N, V, inv_t,
                  uniform, accept_len, accept_nodes, t.max_depth, out_tokens);
}

// ---------------------------------------------------------------------------
// Measurement aid, not a step of the method: with random weights the base
// model never agrees with the heads, so every round would accept nothing.
// This replaces the base model's choice after every node by a continuation
// drawn per sequence and depth from a rank prior -- the token after a depth-d
// node is head (d + 1)'s rank-r guess with probability alpha (1 - alpha)^r, or
// a token outside its top-k with the remaining probability -- so a round
// accepts the branch of ranks drawn, as far as the tree holds it.  The draw
// for (sequence b, depth d) is a counter hash of (seed, b, cache_len[b], d):
// a new prefix length gives a new continuation, and graph replays draw anew.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__global__ __launch_bounds__(256) void plant_greedy_kernel(const int* __restrict__ depth, int N, int max_depth,
                                                           const int32_t* __restrict__ topk_idx, int K, int topk,
                                                           const int32_t* __restrict__ cache_len, PlantAlphas pa,
                                                           uint64_t seed, int V, int32_t* __restrict__ greedy) {
    __shared__ int s_next[MEDUSA_MAX_DEPTH_DEV + 1];  // the token after a node of depth d
    const int b = blockIdx.x, tid = threadIdx.x;
    if (tid <= max_depth) {
        const int d = tid;
        const uint64_t z = mix64(mix64(mix64(seed ^ (uint64_t)b) ^ (uint64_t)(uint32_t)cache_len[b]) ^ (uint64_t)d);
        const float u = (float)(z >> 40) * (1.0f / 16777216.0f);
        const int32_t* cand = topk_idx + ((size_t)b * K + min(d, K - 1)) * topk;
        // the rank drawn: the first r with u < sum_{j <= r} alpha (1 - alpha)^j
        const float alpha = pa.a[min(d, MEDUSA_MAX_DEPTH_DEV - 1)];
        int r = topk;
        float cum = 0.f, pr = alpha;
        for (int j = 0; j < topk && d < K; ++j) {
            cum += pr;
            if (u < cum) { r = j; break; }
            pr *= 1.f - alpha;
        }
        int tok;
        if (r < topk) {
            tok = cand[r];
        } else {  // a token outside the head's top-k (at depth K: any token)
            tok = (int)((mix64(z) >> 33) % (uint64_t)V);
            for (int it = 0; it <= topk && d < K; ++it) {
                bool hit = false;
                for (int j = 0; j < topk; ++j) hit = hit || cand[j] == tok;
                if (!hit) break;
                tok = tok + 1 < V ? tok + 1 : 0;
            }
        }
        s_next[d] = tok;
    }
    __syncthreads();
    for (int i = tid; i < N; i += blockDim.x) greedy[(size_t)b * N + i] = s_next[depth[i]];
}

void launch_plant_greedy(const TreeDev& t, const int32_t* topk_idx, int B, int K, int topk,
                         const int32_t* cache_len, const PlantAlphas& pa, uint64_t seed, int V, int32_t* greedy,
                         hipStream_t s) {
    MEDUSA_LAUNCH("plant_greedy", plant_greedy_kernel, dim3(B), dim3(256), 0, s, t.depth, t.N, t.max_depth, topk_idx,
                  K, topk, cache_len, pa, seed, V, greedy);
}

// ---------------------------------------------------------------------------
// Acceptance statistics for choosing the tree from what rounds accept.  What
// a round reveals about sequence b: the base model's choice at every depth
// d <= L was the candidate on the accepted path (its rank is the node's
// rank), and at depth L + 1 <= K it was the bonus token, whose rank among
// head L + 1's guesses is found in topk_idx (or it is none of them: bucket
// topk); deeper depths are not observed.  counts [K][topk + 1] gathers them
// (atomic adds; one block per sequence).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void accept_stats_kernel(const int* __restrict__ rank, int Dmax,
                                                          const int32_t* __restrict__ accept_len,
                                                          const int32_t* __restrict__ accept_nodes,
                                                          const int32_t* __restrict__ out_tokens,
                                                          const int32_t* __restrict__ topk_idx, int K, int topk,
                                                          int32_t* __restrict__ counts) {
    const int b = blockIdx.x, d = threadIdx.x + 1;  // depth observed by this thread
    const int L = accept_len[b];
    if (L < 0 || L > Dmax || d > K) return;
    int r = -1;
    if (d <= L) {
        const int node = accept_nodes[(size_t)b * (Dmax + 1) + d];
        if (node >= 0) r = rank[node];
    } else if (d == L + 1) {
        const int tok = out_tokens[(size_t)b * (Dmax + 1) + L];
        const int32_t* cand = topk_idx + ((size_t)b * K + (d - 1)) * topk;
        r = topk;
        for (int j = 0; j < topk; ++j)
            if (cand[j] == tok) { r = j; break; }
    }
    if (r >= 0) atomicAdd(&counts[(d - 1) * (topk + 1) + r], 1);
}

void launch_accept_stats(const TreeDev& t, const int32_t* accept_len, const int32_t* accept_nodes,
                         const int32_t* out_tokens, const int32_t* topk_idx, int B, int K, int topk, int32_t* counts,
                         hipStream_t s) {
    MEDUSA_LAUNCH("accept_stats", accept_stats_kernel, dim3(B), dim3(64), 0, s, t.rank, t.max_depth, accept_len,
                  accept_nodes, out_tokens, topk_idx, K, topk, counts);
}

// ---------------------------------------------------------------------------
// Hand-off to the next round.  Block b reads sequence b's L and deepest
// accepted node (uniform over the block), gathers that node's final
// normalised row into h[b] (converted to T), sets the next root to the bonus
// token, appends the round's L + 1 tokens to the sequence's output and, when
// asked, copies the new cache length into the buffer the next round reads.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void advance_kernel(const int32_t* __restrict__ accept_len,
                                                      const int32_t* __restrict__ accept_nodes,
                                                      const int32_t* __restrict__ out_tokens,
                                                      const float* __restrict__ hidden, int N, int Dmax, int H,
                                                      int32_t* __restrict__ root_tok, T* __restrict__ h,
                                                      int32_t* __restrict__ tokens, int32_t* __restrict__ n_tokens,
                                                      int cap, const int32_t* __restrict__ new_cache_len,
                                                      int32_t* __restrict__ cache_len) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int L = accept_len[b];
    if (L < 0 || L > Dmax) return;  // not a medusa_accept result: leave the sequence unchanged
    const size_t row = (size_t)b * (Dmax + 1);
    const int node = accept_nodes[row + L];
    if (node < 0 || node >= N) return;
    const float* src = hidden + ((size_t)b * N + node) * H;
    for (int j = tid; j < H; j += blockDim.x) Elem<T>::store(h, (size_t)b * H + j, src[j]);
    if (tid == 0) {
        root_tok[b] = out_tokens[row + L];
        if (cache_len != nullptr) cache_len[b] = new_cache_len[b];
    }
    if (tokens != nullptr) {
        const int n0 = n_tokens[b];
        __syncthreads();  // every thread has read n0 before it is advanced
        if (tid <= L && n0 >= 0 && n0 + tid < cap) tokens[(size_t)b * cap + n0 + tid] = out_tokens[row + tid];
        if (tid == 0) n_tokens[b] = n0 + L + 1;
    }
}

void launch_advance(const TreeDev& t, const int32_t* accept_len, const int32_t* accept_nodes,
                    const int32_t* out_tokens, const float* hidden, int B, int H, bool bf16, int32_t* root_tok,
                    void* h, int32_t* tokens, int32_t* n_tokens, int cap, const int32_t* new_cache_len,
                    int32_t* cache_len, hipStream_t s) {
    if (bf16)
        MEDUSA_LAUNCH("advance", advance_kernel<bf16_t>, dim3(B), dim3(256), 0, s, accept_len, accept_nodes,
                      out_tokens, hidden, t.N, t.max_depth, H, root_tok, (bf16_t*)h, tokens, n_tokens, cap,
                      new_cache_len, cache_len);
    else
        MEDUSA_LAUNCH("advance", advance_kernel<float>, dim3(B), dim3(256), 0, s, accept_len, accept_nodes,
                      out_tokens, hidden, t.N, t.max_depth, H, root_tok, (float*)h, tokens, n_tokens, cap,
                      new_cache_len, cache_len);
}

}  // namespace medusa
