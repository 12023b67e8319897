// Base model's greedy choice after every tree node (step a5):
// n_r = x_r * rsqrt(mean(x_r^2) + eps) (unit weight), then
// greedy[r] = argmax_v lm_head[v] . n_r  (lower index first among equal values).
//
// Packed bf16 lm_head: the product of the node rows with lm_head is a dense
// contraction (64-256 rows share every lm_head byte), so it runs on MFMA with
// the argmax fused into the epilogue (skinny_mfma.hpp; the 32000-row
// vocabulary gives 250 8-wave workgroups).  RMSNorm with unit weight is a
// positive factor per row, so the product runs on the bf16 rows x themselves
// and the argmax is that of lm_head . x; the factor is applied only to the
// logits when they are asked for.  A 256-row node tile over a vocabulary too
// small to give that product 256 workgroups runs instead on the 32 x 32 x 16
// kernel with loader waves of lm_head_wide.hpp.  Each workgroup writes, per
// node, its best (value, index); a merge kernel reduces them.
// Row-major lm_head (float32 or bf16): the vector-ALU GEMV of the heads on the
// float32 normalised rows, one pass per 8 rows.
#include "common.hpp"
#include "lm_head_wide.hpp"
#include "skinny_mfma.hpp"

namespace medusa {

// One block per row; writes n = x * rsqrt(mean(x^2) + eps) in float32.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* __restrict__ x, int H, float eps,
                                                           float* __restrict__ n) {
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
    for (int j = threadIdx.x; j < H; j += 256) n[(size_t)r * H + j] = Elem<T>::load(xr, j) * rs;
}

// greedy[r] = best of the G workgroup candidates of row r
__global__ __launch_bounds__(64) void argmax_merge_kernel(const float* __restrict__ cand_val,
                                                          const int* __restrict__ cand_idx, int G,
                                                          int32_t* __restrict__ greedy) {
    const int r = blockIdx.x;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int g0 = threadIdx.x; g0 < G; g0 += 4 * 64) {  // four loads in flight per thread
        float v[4];
        int i[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g = g0 + u * 64;
            v[u] = g < G ? cand_val[(size_t)r * G + g] : -INFINITY;
            i[u] = g < G ? cand_idx[(size_t)r * G + g] : 0x7FFFFFFF;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (better(v[u], i[u], bv, bi)) { bv = v[u]; bi = i[u]; }
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



static size_t a256(size_t x) { return (x + 255) / 256 * 256; }

// greedy[r] = argmax_v lm_head[v] . n[r] for bf16 rows n already normalised
// (MFMA product with the fused argmax, then the merge of the workgroups'
// candidates).  Workspace: the candidates.
// Launch shape (measured, 4096-wide rows): up to 64 node rows, vocabularies
// of >= 8192 rows stream from 8-wave workgroups with one 16-row weight block
// per wave (64 x 32000: 45.6 us against 50.0 with 4 waves).  From 128 node
// rows on the products are bound by the LDS reads of the node fragments, so
// each wave takes two weight blocks (a fragment read feeds two products):
// 256 x 128256 in 280 us against 363, 512 x 128256 in 574 against 717; 8
// waves unless that leaves fewer than 256 workgroups (256 x 32000: 4 waves,
// 110 us against 126).  256-row node tiles that would get fewer than 256
// workgroups split the node blocks over two waves instead of dropping to 4
// waves (8 waves: 4 row groups x 2 node halves, 128 weight rows per
// workgroup): each wave then reads 8 node fragments a chunk, and two waves
// per SIMD hide each other's latencies (256 x 32000: 104 us against 125).
// With enough workgroups the unsplit 8-wave tile stays faster (512 x 128256:
// 620 us against 780): the split doubles the workgroups that stage each node
// row.
struct LmhShape {
    int waves, rb, ns;
};
static LmhShape lmh_shape(int R, int V) {
    const int nblk = lmh_nblk(R);
    if (nblk < 8) return {V >= 8192 ? 8 : 4, 1, 1};
    const int tiles = (R + nblk * 16 - 1) / (nblk * 16);
    const bool many = (V + 255) / 256 * tiles >= 256;
    if (nblk == 16) return {8, 2, many ? 1 : 2};
    return {many ? 8 : 4, 2, 1};
}
static int lmh_groups(int R, int V) {
    const LmhShape sh = lmh_shape(R, V);
    const int rows = 16 * sh.waves / sh.ns * sh.rb;
    return (V + rows - 1) / rows;
}

// Node tiles that would split their node blocks (too few workgroups), without
// logits: the 32 x 32 x 16 kernel of lm_head_wide.hpp with loader waves
// (register ring LMW_D chunks deep: measured at 256 x 4096 x 32000, 79 us
// with 1, 82 with 2, 85 with 4, against 90 for the 16 x 16 x 32 product).
constexpr int LMW_D = 1;
static bool lmw_use(int R, int H, int V, bool logits) {
    return lmh_nblk(R) == 16 && lmh_shape(R, V).ns == 2 && !logits && H % LMW_KC == 0;
}
// Node tiles with enough workgroups at 256 weight rows, without logits: the
// 256-row variant of lm_head_wide.hpp (512 x 4096 x 128256: 555 us against
// 628 for the 16 x 16 x 32 product; 256 x 4096 x 128256: 292 against 302).
static bool lmw256_use(int R, int H, int V, bool logits) {
    return lmh_nblk(R) == 16 && lmh_shape(R, V).ns == 1 && !logits && H % LMW_KC == 0;
}

size_t lm_head_greedy_workspace_bytes(int R, int H, int V) {
    const int G = lmh_groups(R, V) > lmw_groups(V) ? lmh_groups(R, V) : lmw_groups(V);
    (void)H;
    return a256((size_t)R * G * 4) * 2;
}

void launch_lm_head_greedy(const bf16_t* n, const bf16_t* lm_head, int R, int H, int V, int32_t* greedy,
                           float* logits, float rs_eps, void* ws, hipStream_t s) {
    if (lmw256_use(R, H, V, logits != nullptr)) {
        const int G = lmw256_groups(V), T = lmw_tiles(R);
        float* cv = (float*)ws;
        int* ci = (int*)((char*)ws + a256((size_t)R * G * 4));
        MEDUSA_LAUNCH("lm_head_argmax", lm_head_argmax_wide256_kernel, dim3((G + 7) / 8 * 8 * T), dim3(512), 0, s, n,
                      lm_head, R, H, V, T, G, cv, ci);
        MEDUSA_LAUNCH("argmax_merge", argmax_merge_kernel, dim3(R), dim3(64), 0, s, cv, ci, G, greedy);
        return;
    }
    if (lmw_use(R, H, V, logits != nullptr)) {
        const int G = lmw_groups(V), T = lmw_tiles(R);
        float* cv = (float*)ws;
        int* ci = (int*)((char*)ws + a256((size_t)R * G * 4));
        MEDUSA_LAUNCH("lm_head_argmax", lm_head_argmax_wide_kernel<LMW_D>, dim3((G + 7) / 8 * 8 * T), dim3(512), 0, s, n,
                      lm_head, R, H, V, T, G, cv, ci);
        MEDUSA_LAUNCH("argmax_merge", argmax_merge_kernel, dim3(R), dim3(64), 0, s, cv, ci, G, greedy);
        return;
    }
    const int G = lmh_groups(R, V);
    float* cv = (float*)ws;
    int* ci = (int*)((char*)ws + a256((size_t)R * G * 4));
    const int nblk = lmh_nblk(R);
    const dim3 grid(G, (R + nblk * 16 - 1) / (nblk * 16));
    const int nch = H / lmh_kc(nblk);
#define LMH_LAUNCH(NB, WV, RBL, NSP)                                                                   \
    MEDUSA_LAUNCH("lm_head_argmax", (skinny_mfma_kernel<NB, SKINNY_ARGMAX, WV, RBL, NSP>), grid, dim3(WV * 64), 0, \
                  s, n, lm_head, R, H, V, nch, cv, ci, logits, rs_eps)
    const LmhShape sh = lmh_shape(R, V);
    if (nblk == 16) {
        if (sh.ns == 2) LMH_LAUNCH(16, 8, 2, 2);
        else LMH_LAUNCH(16, 8, 2, 1);
    } else if (sh.waves == 8) {
        if (nblk == 4) LMH_LAUNCH(4, 8, 1, 1);
        else LMH_LAUNCH(8, 8, 2, 1);
    } else {
        if (nblk == 4) LMH_LAUNCH(4, 4, 1, 1);
        else LMH_LAUNCH(8, 4, 2, 1);
    }
#undef LMH_LAUNCH
    MEDUSA_LAUNCH("argmax_merge", argmax_merge_kernel, dim3(R), dim3(64), 0, s, cv, ci, G, greedy);
}

void launch_lm_head_greedy(const bf16_t* n, const bf16_t* lm_head, int R, int H, int V, int32_t* greedy, void* ws,
                           hipStream_t s) {
    launch_lm_head_greedy(n, lm_head, R, H, V, greedy, nullptr, -1.f, ws, s);
}

size_t greedy_workspace_bytes(int R, int H, int V, bool packed) {
    if (packed) return lm_head_greedy_workspace_bytes(R, H, V);
    const int G = gemv_groups_max(V);
    return a256((size_t)R * H * 4) + a256((size_t)8 * G * 4) * 2 + a256((size_t)R * 4);
}

// packed: bf16 x and packed bf16 lm_head (MFMA);  otherwise row-major lm_head
// of x's type (GEMV)
void launch_base_greedy(const void* x, const void* lm_head, bool packed, int R, int H, int V, float eps, bool bf16,
                        int32_t* greedy, float* logits, void* ws, hipStream_t s) {
    char* p = (char*)ws;
    if (packed) {
        // the logits are the scores of the normalised rows: the product
        // scales them by the RMSNorm factors it accumulates while staging x
        launch_lm_head_greedy((const bf16_t*)x, (const bf16_t*)lm_head, R, H, V, greedy, logits, eps, p, s);
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
        MEDUSA_LAUNCH("rmsnorm_rows", rmsnorm_rows_kernel<bf16_t>, dim3(R), dim3(256), 0, s, (const bf16_t*)x, H, eps,
                      n);
    else
        MEDUSA_LAUNCH("rmsnorm_rows", rmsnorm_rows_kernel<float>, dim3(R), dim3(256), 0, s, (const float*)x, H, eps,
                      n);
    for (int r0 = 0; r0 < R; r0 += 8) {
        const int nb = R - r0 < 8 ? R - r0 : 8;
        launch_vocab_topk_named(n + (size_t)r0 * H, lm_head, nb, H, V, 1, 1, bf16,
                                logits ? logits + (size_t)r0 * V : nullptr, greedy + r0, gval + r0, cv, ci, s,
                                "lm_head_gemv", "lm_head_gemv_merge");
    }
}

}  // namespace medusa
