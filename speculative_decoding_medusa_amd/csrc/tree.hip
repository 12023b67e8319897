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
// Acceptance + compaction.  Grid (B, S): every block of row b recomputes the
// acceptance of sequence b (N <= 256 nodes, one thread each: walk the chain
// to the root and AND the matches), block (b, 0) writes the results, and
// block (b, s) compacts slice s of the caches: slice = (layer, KV head).
// Within a slice all source rows are read into registers before the barrier
// that precedes any write, so an accepted node that moves onto a slot another
// accepted node is read from cannot corrupt it; slices are disjoint.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void accept_compact_kernel(
    const int* __restrict__ parent, const int* __restrict__ depth, int N, int Dmax,
    const int32_t* __restrict__ node_tok, const int32_t* __restrict__ greedy,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes, int32_t* __restrict__ out_tokens,
    const int32_t* __restrict__ cache_len, int32_t* __restrict__ new_cache_len, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int nKV, int D, int Lmax, int64_t layer_stride, int n_slices) {
    __shared__ int s_acc_depth[256];
    __shared__ int s_par[256], s_tok[256], s_g[256];
    __shared__ int s_path[MEDUSA_MAX_DEPTH_DEV + 1];
    __shared__ int s_L, s_deepest;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t* tok = node_tok + (size_t)b * N;
    const int32_t* g = greedy + (size_t)b * N;
    const int P = cache_len[b];

    // the sequence's nodes (N <= 256, one per thread) -> LDS in one round of
    // loads, so the walks below read no global memory
    int dep = 0;
    if (tid < N) {
        s_par[tid] = parent[tid];
        s_tok[tid] = tok[tid];
        s_g[tid] = g[tid];
        dep = depth[tid];
    }
    if (tid == 0) { s_L = 0; s_deepest = 0; }
    __syncthreads();
    // accepted iff every node on the chain to the root matches its parent's choice
    int my = -1;
    if (tid < N) {
        bool ok = true;
        int j = tid;
        while (j > 0) {
            const int p = s_par[j];
            ok = ok && (s_tok[j] == s_g[p]);
            j = p;
        }
        my = ok ? dep : -1;
    }
    s_acc_depth[tid] = my;
    __syncthreads();
    // deepest accepted depth, then the lowest node index at that depth
    if (tid == 0) {
        int L = 0, deepest = 0;
        for (int i = 0; i < N; ++i)
            if (s_acc_depth[i] > L) { L = s_acc_depth[i]; deepest = i; }
        s_L = L;
        s_deepest = deepest;
        int j = deepest;
        for (int d = L; d >= 0; --d) { s_path[d] = j; j = d > 0 ? s_par[j] : 0; }
    }
    __syncthreads();
    const int L = s_L;

    if (blockIdx.y == 0 && tid <= Dmax) {
        const int d = tid;
        const size_t o = (size_t)b * (Dmax + 1) + d;
        if (d <= L) {
            accept_nodes[o] = s_path[d];
            out_tokens[o] = d < L ? s_tok[s_path[d + 1]] : s_g[s_deepest];
        } else {
            accept_nodes[o] = -1;
            out_tokens[o] = -1;
        }
        if (d == 0) {
            accept_len[b] = L;
            new_cache_len[b] = P + L + 1;
        }
    }

    // nothing to move, or a cache length that would address past Lmax
    if (k_cache == nullptr || L == 0 || P < 0 || P + N > Lmax) return;
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

void launch_accept(const TreeDev& t, const int32_t* node_tok, const int32_t* greedy, int B,
                   int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens, const int32_t* cache_len,
                   int32_t* new_cache_len, void* k_cache, void* v_cache, int n_layers, int64_t layer_stride,
                   int nKV, int D, int Lmax, bool bf16, hipStream_t s) {
    const int n_slices = k_cache ? n_layers * nKV : 1;
    const dim3 grid(B, n_slices);
    if (bf16)
        MEDUSA_LAUNCH("accept_compact", accept_compact_kernel<bf16_t>, grid, dim3(256), 0, s, t.parent, t.depth,
                      t.N, t.max_depth, node_tok, greedy, accept_len, accept_nodes, out_tokens, cache_len,
                      new_cache_len, (bf16_t*)k_cache, (bf16_t*)v_cache, nKV, D, Lmax, layer_stride, n_slices);
    else
        MEDUSA_LAUNCH("accept_compact", accept_compact_kernel<float>, grid, dim3(256), 0, s, t.parent, t.depth,
                      t.N, t.max_depth, node_tok, greedy, accept_len, accept_nodes, out_tokens, cache_len,
                      new_cache_len, (float*)k_cache, (float*)v_cache, nKV, D, Lmax, layer_stride, n_slices);
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
