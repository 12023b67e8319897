// Medusa heads: residual-SiLU block (step a1) and vocabulary projection with
// fused per-head top-k (step a2).
//
// Both are matrix-vector products that stream a weight matrix from HBM once
// (B <= 8 right-hand sides), so they are written as HBM-streaming GEMVs on the
// vector ALUs, not as MFMA tiles: every weight byte is used B times, far below
// the MFMA ridge.
//
// Layout of the work: grid (G, K); workgroup g of head k owns a contiguous
// block of rows; its waves take groups of R consecutive rows in turn, so each
// wave visits its rows in increasing order.  A lane owns 16-byte chunks
// c*64 + lane of a row (fully coalesced 1 KiB per wave per load), multiplies
// them with the right-hand sides staged once per workgroup in LDS as fp32,
// and the 64 partial sums are combined with an xor butterfly whose result is
// bitwise identical in every lane.  The reduction order depends only on the
// row length, so the projection of a given z is bitwise reproducible.
//
// The weight loads are non-temporal: every weight byte is read once per call,
// so it should not displace reused lines (z, the candidates) from the caches.
#include <type_traits>

#include "common.hpp"
#include "skinny_mfma.hpp"
#include "tree.hpp"

namespace medusa {

enum { EPI_SILU = 0, EPI_TOPK = 1 };

// Upper bound of the rows one workgroup owns (sizes the row-value LDS array).
constexpr int GEMV_MAX_ROWS_PER_WG = 512;

template <typename WT, int NB, int CPL, int R, int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_rows_kernel(
    const void* __restrict__ xsrc,   // SILU: h [B][H] (WT);  TOPK: z [B][K][H] fp32
    const WT* __restrict__ W,        // [K][nrows][H]
    const WT* __restrict__ bias,     // SILU: b1 [K][H]
    int B, int H, int nrows, int K, int rows_per_wg,
    float* __restrict__ out,         // SILU: z [B][K][H];  TOPK: logits [B][K][nrows] or null
    float* __restrict__ cand_val,    // TOPK: [B][K][G][topk]
    int* __restrict__ cand_idx, int topk) {
    // The right-hand sides and the row values live in separate LDS arrays, so
    // the compiler knows the row-value stores never touch x and can keep x in
    // registers across the row loop.
    extern __shared__ __attribute__((aligned(16))) float xs[];  // [NB][H] fp32
    __shared__ float rowv[EPI == EPI_TOPK ? NB * GEMV_MAX_ROWS_PER_WG : 1];  // TOPK: [NB][rows_per_wg]
    __shared__ float bsh[EPI == EPI_SILU ? GEMV_MAX_ROWS_PER_WG : 1];         // SILU: the rows' biases
    constexpr int NT = WAVES * 64;
    constexpr int PER = Elem<WT>::PER16;
    const int k = blockIdx.y;
    const int g = blockIdx.x;
    const int G = gridDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    const int nchunks = H / PER;
    const int row0 = g * rows_per_wg;
    const int row1 = min(nrows, row0 + rows_per_wg);
    const WT* Wk = W + (size_t)k * nrows * H;

    // Rows of H = CPL * 64 * PER elements and whole row groups take the
    // unchecked paths: the checks are wave-uniform, so the common case runs
    // without per-lane execution masks around every load and FMA block.
    const bool full_rows = nchunks == CPL * 64;
    auto load_rows = [&](u32x4(&wv)[R][CPL], int rb) {
        if (full_rows && rb + R <= row1) {
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    wv[j][c] = ld_stream(Wk + (size_t)(rb + j) * H + (size_t)(c * 64 + lane) * PER);
            return;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = rb + j;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int ci = c * 64 + lane;
                if (row < row1 && ci < nchunks)
                    wv[j][c] = ld_stream(Wk + (size_t)row * H + (size_t)ci * PER);
                else
                    wv[j][c] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    // The first weight rows of every wave are requested before the
    // right-hand sides are staged, so the stream starts at once.
    const int rb_first = row0 + wave * R;
    u32x4 wv[R][CPL];
    if (rb_first < row1) load_rows(wv, rb_first);

    // Stage the right-hand sides (fp32) in LDS with 16-byte loads; padded
    // batch slots are zero.  H % 8 == 0, so a chunk never straddles two rows.
    // The SiLU epilogue's biases of this workgroup's rows go to LDS as well.
    if (EPI == EPI_SILU)
        for (int i = threadIdx.x; i < row1 - row0; i += NT) bsh[i] = Elem<WT>::load(bias, (size_t)k * H + row0 + i);
    {
        constexpr int XE = EPI == EPI_SILU ? Elem<WT>::PER16 : 4;  // elements per 16-byte chunk of x
        const int cpr = H / XE;                                    // chunks per right-hand side
        for (int i = threadIdx.x; i < NB * cpr; i += NT) {
            const int b = i / cpr, j = (i - b * cpr) * XE;
            float v[XE];
            if (b < B) {
                if (EPI == EPI_SILU) {
                    Elem<WT>::expand(*(const u32x4*)((const WT*)xsrc + (size_t)b * H + j), v);
                } else {
                    const f32x4 q = *(const f32x4*)((const float*)xsrc + ((size_t)b * K + k) * H + j);
#pragma unroll
                    for (int t = 0; t < XE; ++t) v[t] = q[t];
                }
            } else {
#pragma unroll
                for (int t = 0; t < XE; ++t) v[t] = 0.f;
            }
#pragma unroll
            for (int t = 0; t < XE; t += 4)
                *(f32x4*)(xs + b * H + j + t) = (f32x4){v[t], v[t + 1], v[t + 2], v[t + 3]};
        }
    }
    __syncthreads();
    auto dot = [&](auto checked, const u32x4(&wv)[R][CPL], float(&acc)[R][NB]) {
        constexpr bool CHECKED = decltype(checked)::value;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ci = c * 64 + lane;
            if (!CHECKED || ci < nchunks) {
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
    };
    auto process = [&](const u32x4(&wv)[R][CPL], int rb) {
        float acc[R][NB];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[j][b] = 0.f;
        if (full_rows) dot(std::false_type{}, wv, acc);
        else dot(std::true_type{}, wv, acc);
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int row = rb + j;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float v = wave_sum(acc[j][b]);
                if (row >= row1 || b >= B) continue;
                if (EPI == EPI_SILU) {
                    if (lane == 0) {
                        const float pre = v + bsh[row - row0];
                        const float s = pre / (1.f + __expf(-pre));
                        out[((size_t)b * K + k) * H + row] = xs[b * H + row] + s;
                    }
                } else if (lane == 0) {
                    rowv[b * rows_per_wg + (row - row0)] = v;
                    if (out != nullptr) out[((size_t)b * K + k) * nrows + row] = v;
                }
            }
        }
    };

    for (int rb = rb_first; rb < row1; rb += WAVES * R) {
        if (rb != rb_first) load_rows(wv, rb);
        process(wv, rb);
    }

    if (EPI == EPI_TOPK) {
        // The workgroup's top-k of each sequence: wave w takes sequences
        // w, w + WAVES, ...  Each lane keeps a sorted register list of the rows
        // it scans; the wave then extracts the winners rank by rank.
        __syncthreads();
        const int nr = row1 - row0;
        for (int b = wave; b < B; b += WAVES) {
            float lv[MEDUSA_MAX_TOPK_DEV];
            int li[MEDUSA_MAX_TOPK_DEV];
#pragma unroll
            for (int t = 0; t < MEDUSA_MAX_TOPK_DEV; ++t) { lv[t] = -INFINITY; li[t] = 0x7FFFFFFF; }
            for (int r = lane; r < nr; r += 64) sorted_insert<MEDUSA_MAX_TOPK_DEV>(lv, li, rowv[b * rows_per_wg + r], row0 + r);
            const size_t base = (((size_t)b * K + k) * G + g) * topk;
            for (int t = 0; t < topk; ++t) {
                float bv = lv[0];
                int bi = li[0];
                wave_argmax(bv, bi);
                if (lane == 0) { cand_val[base + t] = bv; cand_idx[base + t] = bi; }
                if (lv[0] == bv && li[0] == bi) sorted_pop<MEDUSA_MAX_TOPK_DEV>(lv, li);
            }
        }
    }
}

// Final merge: per (b, k) the top-k of the G * topk workgroup candidates.
// Each thread keeps a sorted register list of the best TK candidates it reads
// (loads issued eight at a time: one round for up to 2048 candidates); each
// wave then extracts its own top-k rank by rank (wave-wide argmax of the lane
// list heads, the winning lane pops its head: no workgroup barrier), and wave
// 0 takes the top-k of the 4 waves' lists, one candidate a lane.  Candidate
// rows are distinct (padding entries rank last), so the (value desc, index
// asc) order is total.
// With a tree (node_tok not null) the workgroup of (b, k) also writes the
// tree nodes that take their token from head k, those at depth k + 1
// (node_tok = its rank-th choice, node_pos = P + depth), and the workgroup of
// head 0 the root (node_tok = root_tok[b], node_pos = P); (0, 0) copies the
// ancestor mask.  No node depends on another head, so the tree build needs no
// launch of its own.
template <int TK>
__global__ __launch_bounds__(256) void topk_merge_kernel(const float* __restrict__ cand_val,
                                                         const int* __restrict__ cand_idx, int M, int topk,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_val, int K = 1,
                                                         const int* __restrict__ depth = nullptr,
                                                         const int* __restrict__ rank = nullptr,
                                                         const uint64_t* __restrict__ mask = nullptr, int N = 0,
                                                         int W = 0, const int32_t* __restrict__ root_tok = nullptr,
                                                         const int32_t* __restrict__ cache_len = nullptr,
                                                         int32_t* __restrict__ node_tok = nullptr,
                                                         int32_t* __restrict__ node_pos = nullptr,
                                                         uint64_t* __restrict__ anc_mask = nullptr) {
    __shared__ int top_s[TK];
    static_assert(4 * TK <= 64, "the waves' lists fit one wave, a candidate a lane");
    __shared__ float wv_s[4 * TK];
    __shared__ int wi_s[4 * TK];
    const int bk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* cv = cand_val + (size_t)bk * M;
    const int* ci = cand_idx + (size_t)bk * M;
    // the tree's inputs for this thread's first node (and the first mask
    // word), loaded before the candidates: their round trip to memory
    // overlaps the merge instead of following it
    const int b = bk / K, k = bk - b * K;
    int P = 0, d0 = -1, r0 = 0;
    uint64_t m0 = 0;
    if (node_tok != nullptr) {
        P = cache_len[b];
        if (tid < N) { d0 = depth[tid]; r0 = rank[tid]; }
        if (bk == 0 && anc_mask != nullptr && tid < N * W) m0 = mask[tid];
    }
    float lv[TK];
    int li[TK];
#pragma unroll
    for (int t = 0; t < TK; ++t) { lv[t] = -INFINITY; li[t] = 0x7FFFFFFF; }
    for (int m0 = tid; m0 < M; m0 += 8 * 256) {
        float v[8];
        int i[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int m = m0 + u * 256;
            v[u] = m < M ? cv[m] : -INFINITY;
            i[u] = m < M ? ci[m] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) sorted_insert<TK>(lv, li, v[u], i[u]);
    }
    for (int t = 0; t < topk; ++t) {
        float bv = lv[0];
        int bi = li[0];
        wave_argmax(bv, bi);
        if (lane == 0) { wv_s[wave * TK + t] = bv; wi_s[wave * TK + t] = bi; }
        if (lv[0] == bv && li[0] == bi) sorted_pop<TK>(lv, li);  // the owner pops its head
    }
    __syncthreads();
    if (wave == 0) {
        float v = -INFINITY;
        int i = 0x7FFFFFFF;
        if (lane < 4 * TK && lane % TK < topk) { v = wv_s[lane]; i = wi_s[lane]; }
        for (int t = 0; t < topk; ++t) {
            float bv = v;
            int bi = i;
            wave_argmax(bv, bi);
            if (lane == 0) {
                topk_idx[(size_t)bk * topk + t] = bi;
                topk_val[(size_t)bk * topk + t] = bv;
                top_s[t] = bi;
            }
            if (v == bv && i == bi) { v = -INFINITY; i = 0x7FFFFFFF; }  // the owner drops it
        }
    }
    if (node_tok == nullptr) return;
    // the tree nodes of head k (see above)
    if (bk == 0 && anc_mask != nullptr)
        for (int e = tid; e < N * W; e += 256) anc_mask[e] = e == tid ? m0 : mask[e];
    __syncthreads();
    for (int n = tid; n < N; n += 256) {
        const int d = n == tid ? d0 : depth[n];
        if (d == k + 1) {
            node_tok[(size_t)b * N + n] = top_s[n == tid ? r0 : rank[n]];
            node_pos[(size_t)b * N + n] = P + d;
        } else if (d == 0 && k == 0) {
            node_tok[(size_t)b * N + n] = root_tok[b];
            node_pos[(size_t)b * N + n] = P;
        }
    }
}

void launch_topk_merge(const float* cv, const int* ci, int BK, int M, int topk, int32_t* topk_idx,
                       float* topk_val, hipStream_t s, const char* merge_name);

// the per-head merge of the workgroup candidates, alone or with the tree build
static void launch_merge(const float* cv, const int* ci, int B, int K, int M, int topk, int32_t* topk_idx,
                         float* topk_val, const TreeBuild* tb, hipStream_t s, const char* merge_name) {
    if (tb == nullptr) {
        launch_topk_merge(cv, ci, B * K, M, topk, topk_idx, topk_val, s, merge_name);
        return;
    }
    const TreeDev& t = *tb->t;
#define MEDUSA_TOPK_TREE(TK)                                                                                    \
    MEDUSA_LAUNCH("topk_tree", topk_merge_kernel<TK>, dim3(B * K), dim3(256), 0, s, cv, ci, M, topk, topk_idx, \
                  topk_val, K, t.depth, t.rank, t.mask, t.N, t.W, tb->root_tok, tb->cache_len, tb->node_tok,   \
                  tb->node_pos, tb->anc_mask)
    if (topk <= 4) MEDUSA_TOPK_TREE(4);
    else if (topk <= 8) MEDUSA_TOPK_TREE(8);
    else MEDUSA_TOPK_TREE(16);
#undef MEDUSA_TOPK_TREE
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static int pick_nb(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8; }
static int pick_cpl(int nchunks) {
    const int c = (nchunks + 63) / 64;
    return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 16;
}

// Launch shape of one GEMV: rows per workgroup and the number of workgroups
// per head.  Rows per workgroup are a multiple of the rows one pass of the
// waves covers, sized so that the launch has about `target` workgroups.
struct GemvPlan {
    int rows_per_wg;
    int G;
};

static GemvPlan gemv_plan(int nrows, int K, int target, int quantum) {
    long long total = (long long)nrows * K;
    long long r = (total + target - 1) / target;
    r = ((r + quantum - 1) / quantum) * quantum;
    if (r < quantum) r = quantum;
    if (r > nrows) r = ((nrows + quantum - 1) / quantum) * quantum;
    if (r > GEMV_MAX_ROWS_PER_WG) r = GEMV_MAX_ROWS_PER_WG;
    return GemvPlan{(int)r, (int)((nrows + r - 1) / r)};
}

// LDS of one workgroup: the fp32 right-hand sides (dynamic) and the
// statically sized arrays: the row values (top-k epilogue) or the row biases
// (SiLU epilogue).
static size_t gemv_dyn_lds_bytes(int NB, int H) { return (size_t)NB * H * sizeof(float); }
static size_t gemv_static_lds_bytes(int NB, bool topk) {
    return (size_t)(topk ? NB : 1) * GEMV_MAX_ROWS_PER_WG * sizeof(float);
}
static size_t gemv_lds_bytes(int NB, int H, bool topk) {
    return gemv_dyn_lds_bytes(NB, H) + gemv_static_lds_bytes(NB, topk);
}

template <typename WT, int NB, int CPL, int R, int EPI, int WAVES>
static void launch_gemv_t(const void* x, const WT* W, const WT* bias, int B, int H, int nrows, int K,
                          const GemvPlan& pl, float* out, float* cv, int* ci, int topk, hipStream_t s,
                          const char* name) {
    auto kern = gemv_rows_kernel<WT, NB, CPL, R, EPI, WAVES>;
    const size_t shmem = gemv_dyn_lds_bytes(NB, H);
    // allow the largest dynamic LDS that fits beside the static arrays (once per instantiation)
    static const bool lds_ok = [&] {
        const size_t stat = gemv_static_lds_bytes(NB, EPI == EPI_TOPK);
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)(160 * 1024 - stat - 1024)) == hipSuccess;
    }();
    (void)lds_ok;
    MEDUSA_LAUNCH(name, kern, dim3(pl.G, K), dim3(WAVES * 64), shmem, s, x, W, bias, B, H, nrows, K,
                  pl.rows_per_wg, out, cv, ci, topk);
}

// Production shapes, measured on the 7B head shapes (W1: 5 x 4096 rows, W2:
// 5 x 32000 and 5 x 128256 rows, of 4096 bf16) with the caches flushed
// between launches.  One right-hand side streams the weights: 4 waves x 1 row
// per step on ~2048 workgroups for W1 (29.3 us against 32.4 with 4 rows on
// ~512: small workgroups balance over the CUs), 8 waves x 2 rows on ~2048 for
// W2.  With 8 right-hand sides the kernel is bound by
// the vector ALUs and the LDS reads of the right-hand sides, which more rows
// per step amortise: 8 waves x 4 rows on ~256 workgroups for W1 (111 us
// against 235 with 2 rows), 4 waves x 8 rows on ~1024 for W2 (2.32 ms against
// 3.64).
struct GemvShape {
    int R, WAVES, target;
};
static GemvShape silu_shape(int NB) { return NB <= 2 ? GemvShape{1, 4, 2048} : GemvShape{4, 8, 256}; }
static GemvShape topk_shape(int NB) {
    return NB <= 2 ? GemvShape{2, 8, 2048} : NB <= 4 ? GemvShape{4, 4, 1024} : GemvShape{8, 4, 1024};
}

// Dispatch on the chunks per lane of one right-hand-side width NB.
template <typename WT, int NB, int EPI, int R, int WAVES>
static void launch_gemv_cpl(int CPL, const void* x, const WT* W, const WT* bias, int B, int H, int nrows, int K,
                            const GemvPlan& pl, float* out, float* cv, int* ci, int topk, hipStream_t s,
                            const char* name) {
#define MEDUSA_GEMV_CASE(cpl)                                                                               \
    if (CPL == cpl)                                                                                         \
        return launch_gemv_t<WT, NB, cpl, R, EPI, WAVES>(x, W, bias, B, H, nrows, K, pl, out, cv, ci, topk, s, \
                                                         name);
    MEDUSA_GEMV_CASE(1) MEDUSA_GEMV_CASE(2) MEDUSA_GEMV_CASE(4) MEDUSA_GEMV_CASE(8) MEDUSA_GEMV_CASE(16)
#undef MEDUSA_GEMV_CASE
}

// Dispatch on NB among the widths NBS (the widths a launch shape serves).
template <typename WT, int EPI, int R, int WAVES, int... NBS>
static void launch_gemv_nb(int NB, int CPL, const void* x, const WT* W, const WT* bias, int B, int H,
                           int nrows, int K, const GemvPlan& pl, float* out, float* cv, int* ci, int topk,
                           hipStream_t s, const char* name) {
    (void)((NB == NBS ? (launch_gemv_cpl<WT, NBS, EPI, R, WAVES>(CPL, x, W, bias, B, H, nrows, K, pl, out, cv, ci,
                                                                  topk, s, name),
                         true)
                      : false) ||
           ...);
}

static GemvPlan topk_plan(int V, int K, int NB) {
    const GemvShape sh = topk_shape(NB);
    return gemv_plan(V, K, sh.target, sh.WAVES * sh.R);
}

int vocab_topk_groups(int B, int V, int K) { return topk_plan(V, K, pick_nb(B)).G; }

size_t vocab_topk_lds_bytes(int B, int H, int V, int K) {
    const int NB = pick_nb(B);
    (void)V; (void)K;
    return gemv_lds_bytes(NB, H, true);
}

size_t resid_silu_lds_bytes(int B, int H) { return gemv_lds_bytes(pick_nb(B), H, false); }

void launch_resid_silu(const void* h, const void* w1, const void* b1, int B, int H, int K, bool bf16,
                       float* z, hipStream_t s) {
    const int PER = bf16 ? 8 : 4;
    const int NB = pick_nb(B), CPL = pick_cpl(H / PER);
    const GemvShape sh = silu_shape(NB);
    const GemvPlan pl = gemv_plan(H, K, sh.target, sh.WAVES * sh.R);
#define MEDUSA_SILU_GO(RR, WV, ...)                                                                            \
    do {                                                                                                       \
        if (bf16)                                                                                              \
            launch_gemv_nb<bf16_t, EPI_SILU, RR, WV, __VA_ARGS__>(NB, CPL, h, (const bf16_t*)w1, (const bf16_t*)b1, \
                                                                 B, H, H, K, pl, z, nullptr, nullptr, 0, s,      \
                                                                 "resid_silu_gemv");                             \
        else                                                                                                   \
            launch_gemv_nb<float, EPI_SILU, RR, WV, __VA_ARGS__>(NB, CPL, h, (const float*)w1, (const float*)b1, B, \
                                                                H, H, K, pl, z, nullptr, nullptr, 0, s,          \
                                                                "resid_silu_gemv");                              \
    } while (0)
    if (sh.WAVES == 4) MEDUSA_SILU_GO(1, 4, 1, 2); else MEDUSA_SILU_GO(4, 8, 4, 8);
#undef MEDUSA_SILU_GO
}

void launch_topk_merge(const float* cv, const int* ci, int BK, int M, int topk, int32_t* topk_idx,
                       float* topk_val, hipStream_t s, const char* merge_name) {
    if (topk <= 4)
        MEDUSA_LAUNCH(merge_name, topk_merge_kernel<4>, dim3(BK), dim3(256), 0, s, cv, ci, M, topk, topk_idx,
                      topk_val);
    else if (topk <= 8)
        MEDUSA_LAUNCH(merge_name, topk_merge_kernel<8>, dim3(BK), dim3(256), 0, s, cv, ci, M, topk, topk_idx,
                      topk_val);
    else
        MEDUSA_LAUNCH(merge_name, topk_merge_kernel<16>, dim3(BK), dim3(256), 0, s, cv, ci, M, topk, topk_idx,
                      topk_val);
}

static void vocab_topk_impl(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                            float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s,
                            const char* gemv_name, const char* merge_name, const TreeBuild* tb) {
    const int PER = bf16 ? 8 : 4;
    const int NB = pick_nb(B), CPL = pick_cpl(H / PER);
    const GemvShape sh = topk_shape(NB);
    const GemvPlan pl = topk_plan(V, K, NB);
#define MEDUSA_TOPK_GO(RR, WV, ...)                                                                               \
    do {                                                                                                          \
        if (bf16)                                                                                                 \
            launch_gemv_nb<bf16_t, EPI_TOPK, RR, WV, __VA_ARGS__>(NB, CPL, z, (const bf16_t*)w2, nullptr, B, H, V, K, \
                                                                 pl, logits, cv, ci, topk, s, gemv_name);          \
        else                                                                                                      \
            launch_gemv_nb<float, EPI_TOPK, RR, WV, __VA_ARGS__>(NB, CPL, z, (const float*)w2, nullptr, B, H, V, K,  \
                                                                pl, logits, cv, ci, topk, s, gemv_name);           \
    } while (0)
    if (sh.R == 2) MEDUSA_TOPK_GO(2, 8, 1, 2); else if (sh.R == 4) MEDUSA_TOPK_GO(4, 4, 4); else MEDUSA_TOPK_GO(8, 4, 8);
#undef MEDUSA_TOPK_GO
    launch_merge(cv, ci, B, K, pl.G * topk, topk, topk_idx, topk_val, tb, s, merge_name);
}

void launch_vocab_topk_named(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                             float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s,
                             const char* gemv_name, const char* merge_name) {
    vocab_topk_impl(z, w2, B, H, V, K, topk, bf16, logits, topk_idx, topk_val, cv, ci, s, gemv_name, merge_name,
                    nullptr);
}

void launch_vocab_topk_tree(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                            float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci,
                            const TreeBuild& tb, hipStream_t s) {
    vocab_topk_impl(z, w2, B, H, V, K, topk, bf16, logits, topk_idx, topk_val, cv, ci, s, "vocab_proj_topk",
                    "topk_merge", &tb);
}

// ---------------------------------------------------------------------------
// Vocabulary projection over packed W2 on MFMA (several sequences): every
// weight byte feeds 2 B scores, so the vector-ALU GEMV above is bound by its
// FMAs and by its LDS reads of z from B = 4 on; the MFMA product streams the
// packed weights at HBM speed.  z enters as a bf16 head and a bf16 remainder
// (17 significant bits, against the fp32 z: the scores stay within a few
// units of 2^-17 of the fp32 ones): node rows 0..7 of matrix k are the heads
// of sequences 0..7, rows 8..15 the remainders (absent sequences zero), and
// the epilogue adds the two columns of a sequence.
// ---------------------------------------------------------------------------
// Launch shape, measured at 8 sequences x 5 heads x 128,256 x 4,096 (per
// call, with the row split and the top-k merge): 4 waves of 4 16-row blocks
// each (256 weight rows a workgroup) with a two-chunk weight ring take 835
// us, against 913 for one block a wave with a four-chunk ring, 869 for two
// blocks, 840 for eight, and 866 for 2 waves of 4 blocks.  More rows a
// workgroup stage the 16 node rows for more weight bytes; a shallower ring
// keeps fewer bytes in flight.
constexpr int VT_WAVES = 4;  // waves per workgroup
constexpr int VT_RB = 4;     // 16-row weight blocks per wave: 256 weight rows a workgroup

// z [B][K][H] fp32 -> zs [K][16][H] bf16
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ z, int B, int K, int H,
                                                         bf16_t* __restrict__ zs) {
    const size_t n = (size_t)K * 8 * H;  // (k, b < 8, j)
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % H);
        const int b = (int)((e / H) % 8);
        const int k = (int)(e / ((size_t)8 * H));
        const float x = b < B ? z[((size_t)b * K + k) * H + j] : 0.f;
        const bf16_t hi = f32_to_bf16(x);
        zs[((size_t)k * 16 + b) * H + j] = hi;
        zs[((size_t)k * 16 + 8 + b) * H + j] = f32_to_bf16(x - bf16_to_f32(hi));
    }
}

int vocab_topk_packed_groups(int V) { return (V + 16 * VT_WAVES * VT_RB - 1) / (16 * VT_WAVES * VT_RB); }
int vocab_topk_packed_kc() { return LmhCfg<1, VT_WAVES>::KC; }

static size_t a256h(size_t n) { return (n + 255) / 256 * 256; }
size_t vocab_topk_packed_ws_bytes(int B, int H, int V, int K, int topk) {
    const size_t cand = (size_t)B * K * vocab_topk_packed_groups(V) * topk;
    return a256h((size_t)K * 16 * H * 2) + 2 * a256h(cand * 4);
}

static void vocab_topk_packed_impl(const float* z, const void* w2p, int B, int H, int V, int K, int topk,
                                   float* logits, int32_t* topk_idx, float* topk_val, void* ws, const TreeBuild* tb,
                                   hipStream_t s) {
    const int G = vocab_topk_packed_groups(V);
    const size_t cand = (size_t)B * K * G * topk;
    bf16_t* zs = (bf16_t*)ws;
    float* cv = (float*)((char*)ws + a256h((size_t)K * 16 * H * 2));
    int* ci = (int*)((char*)cv + a256h(cand * 4));
    MEDUSA_LAUNCH("split_rows", split_rows_kernel, dim3(256), dim3(256), 0, s, z, B, K, H, zs);
    const long long w_stride = (long long)((V + PACK_ROWS - 1) / PACK_ROWS) * PACK_ROWS * H;
    MEDUSA_LAUNCH("vocab_proj_topk_mfma", (skinny_mfma_kernel<1, SKINNY_TOPK, VT_WAVES, VT_RB>), dim3(G, K),
                  dim3(VT_WAVES * 64), 0, s, zs, (const bf16_t*)w2p, 16, H, V, H / LmhCfg<1, VT_WAVES>::KC, cv, ci,
                  logits, -1.f, topk, B, (long long)16 * H, w_stride);
    launch_merge(cv, ci, B, K, G * topk, topk, topk_idx, topk_val, tb, s, "topk_merge");
}

void launch_vocab_topk_packed(const float* z, const void* w2p, int B, int H, int V, int K, int topk, float* logits,
                              int32_t* topk_idx, float* topk_val, void* ws, hipStream_t s) {
    vocab_topk_packed_impl(z, w2p, B, H, V, K, topk, logits, topk_idx, topk_val, ws, nullptr, s);
}

void launch_vocab_topk_packed_tree(const float* z, const void* w2p, int B, int H, int V, int K, int topk,
                                   float* logits, int32_t* topk_idx, float* topk_val, void* ws, const TreeBuild& tb,
                                   hipStream_t s) {
    vocab_topk_packed_impl(z, w2p, B, H, V, K, topk, logits, topk_idx, topk_val, ws, &tb, s);
}

// Residual-SiLU block over packed W1 on MFMA (several sequences): the bf16
// hidden states are the node rows (exact, no split), grid (H / 32, K), one
// packed H x H matrix per grid row; the epilogue adds the bias, applies SiLU
// and the residual.  Two-wave workgroups (32 weight rows): at 5 x 4096 x 4096
// the 4-wave grid has 320 workgroups, so a quarter of the CUs stream two
// while the rest stream one (39.4 us); 640 two-wave workgroups spread the
// rows more evenly (33.6 us; one-wave workgroups with six chunks in flight
// 33.1, four blocks a wave 38.1, with the weights evicted from the caches
// between calls).
constexpr int SILU_MF_WAVES = 2;

int resid_silu_packed_kc() { return LmhCfg<1, SILU_MF_WAVES>::KC; }

void launch_resid_silu_packed(const void* h, const void* w1p, const void* b1, int B, int H, int K, float* z,
                              hipStream_t s) {
    const int G = (H + 16 * SILU_MF_WAVES - 1) / (16 * SILU_MF_WAVES);
    const long long w_stride = (long long)((H + PACK_ROWS - 1) / PACK_ROWS) * PACK_ROWS * H;
    MEDUSA_LAUNCH("resid_silu_mfma", (skinny_mfma_kernel<1, SKINNY_SILU, SILU_MF_WAVES>), dim3(G, K),
                  dim3(SILU_MF_WAVES * 64), 0, s, (const bf16_t*)h, (const bf16_t*)w1p, B, H, H,
                  H / LmhCfg<1, SILU_MF_WAVES>::KC, nullptr, nullptr, z, -1.f, 0, 0, 0LL, w_stride,
                  (const bf16_t*)b1);
}

void launch_vocab_topk(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                       float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s) {
    launch_vocab_topk_named(z, w2, B, H, V, K, topk, bf16, logits, topk_idx, topk_val, cv, ci, s,
                            "vocab_proj_topk", "topk_merge");
}

}  // namespace medusa
