// C ABI of the Medusa step library: argument validation, workspace carving,
// tree objects, kernel timing.  Every check runs on the host before anything
// is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/medusa.h"
#include "common.hpp"
#include "tree.hpp"

namespace medusa {

// launchers (kernel files)
void launch_resid_silu(const void* h, const void* w1, const void* b1, int B, int H, int K, bool bf16, float* z,
                       hipStream_t s);
void launch_vocab_topk(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                       float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s);
int vocab_topk_groups(int B, int V, int K);
size_t vocab_topk_lds_bytes(int B, int H, int V, int K);
int vocab_topk_packed_kc();
int resid_silu_packed_kc();
void launch_resid_silu_packed(const void* h, const void* w1p, const void* b1, int B, int H, int K, float* z,
                              hipStream_t s);
size_t vocab_topk_packed_ws_bytes(int B, int H, int V, int K, int topk);
void launch_vocab_topk_packed(const float* z, const void* w2p, int B, int H, int V, int K, int topk, float* logits,
                              int32_t* topk_idx, float* topk_val, void* ws, hipStream_t s);
void launch_vocab_topk_tree(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                            float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci,
                            const TreeBuild& tb, hipStream_t s);
void launch_vocab_topk_packed_tree(const float* z, const void* w2p, int B, int H, int V, int K, int topk,
                                   float* logits, int32_t* topk_idx, float* topk_val, void* ws, const TreeBuild& tb,
                                   hipStream_t s);
size_t resid_silu_lds_bytes(int B, int H);
void launch_build_tree(const TreeDev& t, const int32_t* topk_idx, int K, int topk, const int32_t* root_tok,
                       const int32_t* cache_len, int B, int32_t* node_tok, int32_t* node_pos, uint64_t* anc_mask,
                       hipStream_t s);
void launch_tree_attention(const void* q, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                           const int32_t* cache_len, int max_cache_len, const TreeDev& t, int B, int nH, int nKV,
                           int D, int Lmax, float scale, bool bf16, void* out, float* part_o, float* part_ml,
                           hipStream_t s, int target_wg = 0);
size_t attn_workspace_bytes(int B, int nH, int N, int D, int max_cache_len, bool bf16);
void attn_carve(int B, int nH, int N, int D, int max_cache_len, bool bf16, void* ws, float** part_o,
                float** part_ml);
size_t greedy_workspace_bytes(int R, int H, int V, bool packed);
void launch_base_greedy(const void* x, const void* lm_head, bool packed, int R, int H, int V, float eps, bool bf16,
                        int32_t* greedy, float* logits, void* ws, hipStream_t s);
void launch_accept(const TreeDev& t, const int32_t* node_tok, const int32_t* greedy, int B, int32_t* accept_len,
                   int32_t* accept_nodes, int32_t* out_tokens, const int32_t* cache_len, int32_t* new_cache_len,
                   void* k_cache, void* v_cache, int n_layers, int64_t layer_stride, int nKV, int D, int Lmax,
                   bool bf16, hipStream_t s);

struct LayerPtrs {
    const bf16_t *wqkv, *wo, *w_gate_up, *w_down;
};
void launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s);
bool read_mix_supported(int wp, int sp);
void launch_read_mix(const void* win, size_t win_bytes, const void* src, int wp, int sp, int rounds, uint32_t* sink,
                     int n_wg, hipStream_t s);
void launch_mfma_rate(int random_operands, int iters, float* out, int n_wg, hipStream_t s);
void launch_plant_greedy(const TreeDev& t, const int32_t* topk_idx, int B, int K, int topk,
                         const int32_t* cache_len, const PlantAlphas& pa, uint64_t seed, int V, int32_t* greedy,
                         hipStream_t s);
void launch_accept_stats(const TreeDev& t, const int32_t* accept_len, const int32_t* accept_nodes,
                         const int32_t* out_tokens, const int32_t* topk_idx, int B, int K, int topk, int32_t* counts,
                         hipStream_t s);
void launch_advance(const TreeDev& t, const int32_t* accept_len, const int32_t* accept_nodes,
                    const int32_t* out_tokens, const float* hidden, int B, int H, bool bf16, int32_t* root_tok,
                    void* h, int32_t* tokens, int32_t* n_tokens, int cap, const int32_t* new_cache_len,
                    int32_t* cache_len, hipStream_t s);
size_t typical_accept_workspace_bytes(int B, int N);
int typical_max_vocab();
void launch_speculative_sample(const float* p, const float* q, const int32_t* drafts, const float* u_accept,
                               const float* u_resample, int B, int gamma, int V, int32_t* n_accepted,
                               int32_t* out_tokens, hipStream_t s);
void launch_typical_accept(const TreeDev& t, const int32_t* node_tok, const float* logits, int B, int V,
                           float temperature, float eps, float delta, const float* uniform, int32_t* accept_len,
                           int32_t* accept_nodes, int32_t* out_tokens, const int32_t* cache_len,
                           int32_t* new_cache_len, void* k_cache, void* v_cache, int n_layers, int64_t layer_stride,
                           int nKV, int D, int Lmax, bool bf16, void* ws, hipStream_t s);
size_t packed_elems(int rows, int K);
void launch_pack_rows(const bf16_t* src, int rows, int K, bf16_t* dst, int dst_row0, int dst_rows, int inter,
                      hipStream_t s);
size_t decoder_workspace_bytes(int B, int N, int H, int nH, int nKV, int D, int F, int V, int max_cache_len);
size_t prefill_workspace_bytes(int B, int C, int H, int nH, int nKV, int D, int F, int V, int T, int max_cache_len);
void launch_prefill(const LayerPtrs* layers, int n_layers, const bf16_t* E, const bf16_t* lm_head, const TreeDev& chain,
                    const int32_t* tokens, int T, int32_t* cache_len, int max_cache_len, bf16_t* k_cache,
                    bf16_t* v_cache, int64_t layer_stride, int B, int H, int nH, int nKV, int D, int F, int V,
                    int Lmax, float eps, float rope_base, int32_t* next_tok, void* h_out, bool h_bf16, void* ws,
                    hipStream_t s);
void launch_decoder_verify(const LayerPtrs* layers, int n_layers, const bf16_t* E, const bf16_t* lm_head,
                           const TreeDev& t, const int32_t* node_tok, const int32_t* node_pos,
                           const int32_t* cache_len, int max_cache_len, bf16_t* k_cache, bf16_t* v_cache,
                           int64_t layer_stride, int B, int H, int nH, int nKV, int D, int F, int V, int Lmax,
                           float eps, float rope_base, int32_t* greedy, float* hidden, void* ws, hipStream_t s);
size_t skinny_gemm_workspace_bytes(int R, int K, int ncols);
void launch_skinny_gemm(const bf16_t* n, const bf16_t* w, int R, int K, int ncols, float* out, void* ws,
                        hipStream_t s);
void launch_embed(const int32_t* tok, const bf16_t* E, int R, int H, int V, float* x, hipStream_t s);
void launch_rmsnorm_f32_bf16(const float* x, int R, int H, float eps, bf16_t* n, hipStream_t s);
size_t rope_workspace_bytes(int R, int D);
void launch_rope(const float* qkv, const int32_t* pos, int R, int nH, int nKV, int D, float rope_base, bf16_t* q,
                 bf16_t* k, bf16_t* v, void* ws, hipStream_t s);
void launch_swiglu(const float* gate_up, int R, int F, bf16_t* a, hipStream_t s);

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }

struct Fail {
    medusa_status st;
};

static void failf(medusa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error(buf);
    throw Fail{st};
}
#define REQUIRE(cond, ...) \
    do {                   \
        if (!(cond)) failf(MEDUSA_EINVAL, __VA_ARGS__); \
    } while (0)
#define SUPPORT(cond, ...) \
    do {                   \
        if (!(cond)) failf(MEDUSA_EUNSUPPORTED, __VA_ARGS__); \
    } while (0)

static medusa_status finish_launches(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(std::string(what) + ": " + hipGetErrorString(e));
        return MEDUSA_EHIP;
    }
    return MEDUSA_OK;
}

template <typename F>
static medusa_status guarded(const char* what, F&& f) {
    g_err.clear();
    try {
        f();
    } catch (const Fail& x) {
        return x.st;
    }
    return finish_launches(what);
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct ProfRec {
    const char* name;
    hipEvent_t a, b;
};
struct ProfStat {
    int64_t calls = 0;
    double ms = 0.0;
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<ProfRec> g_prof_pending;
static std::vector<hipEvent_t> g_prof_pool;
static std::map<std::string, ProfStat> g_prof_stats;
static std::vector<std::pair<std::string, ProfStat>> g_prof_snapshot;
static thread_local const char* g_prof_name = nullptr;
static thread_local hipEvent_t g_prof_a = nullptr;
// the first HIP error of the timing events since the last collect; a launch
// whose events fail is left untimed and the next collect reports the error
static hipError_t g_prof_err = hipSuccess;

static void prof_fail(hipError_t e) {
    if (g_prof_err == hipSuccess) g_prof_err = e;
}

static hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
        prof_fail(err);
        return nullptr;
    }
    return e;
}

void prof_before(const char* name, hipStream_t s) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_name = name;
    hipEvent_t a = prof_event();
    if (a != nullptr) {
        const hipError_t err = hipEventRecord(a, s);
        if (err != hipSuccess) {
            prof_fail(err);
            g_prof_pool.push_back(a);
            a = nullptr;
        }
    }
    g_prof_a = a;
}

void prof_after(hipStream_t s) {
    if (!g_prof_on || g_prof_a == nullptr) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t b = prof_event();
    const hipError_t err = b != nullptr ? hipEventRecord(b, s) : hipErrorOutOfMemory;
    if (err != hipSuccess) {
        if (b != nullptr) {
            prof_fail(err);
            g_prof_pool.push_back(b);
        }
        g_prof_pool.push_back(g_prof_a);
    } else {
        g_prof_pending.push_back({g_prof_name, g_prof_a, b});
    }
    g_prof_a = nullptr;
}

}  // namespace medusa

using namespace medusa;

struct medusa_tree {
    TreeDev t;
};

extern "C" {

const char* medusa_last_error(void) { return g_err.c_str(); }
const char* medusa_version(void) { return "medusa-mi355x 0.1 (gfx950)"; }

// ---------------------------------------------------------------------------
// a1 / a2
// ---------------------------------------------------------------------------
static void check_heads_shape(int B, int H, int K, medusa_dtype dt) {
    REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
    REQUIRE(B >= 1 && K >= 1 && H >= 1, "B, H and K must be positive (B=%d H=%d K=%d)", B, H, K);
    SUPPORT(B <= MEDUSA_MAX_BATCH, "B=%d exceeds %d", B, MEDUSA_MAX_BATCH);
    SUPPORT(H % 8 == 0 && H <= 8192, "H=%d must be a multiple of 8 and <= 8192", H);
    SUPPORT(resid_silu_lds_bytes(B, H) <= 160 * 1024, "B*H too large for the LDS-staged right-hand sides");
}

static void check_w1_layout(int H, medusa_dtype dt, medusa_layout w1_layout) {
    REQUIRE(w1_layout == MEDUSA_ROW_MAJOR || w1_layout == MEDUSA_PACKED, "w1_layout must be ROW_MAJOR or PACKED");
    if (w1_layout == MEDUSA_PACKED) {
        SUPPORT(dt == MEDUSA_BF16, "a packed w1 must be bf16");
        SUPPORT(H % resid_silu_packed_kc() == 0, "packed w1: H=%d must be a multiple of %d", H,
                resid_silu_packed_kc());
    }
}

static void run_resid_silu(const void* h, const void* w1, medusa_layout w1_layout, const void* b1, int B, int H,
                           int K, medusa_dtype dt, float* z, hipStream_t s) {
    if (w1_layout == MEDUSA_PACKED)
        launch_resid_silu_packed(h, w1, b1, B, H, K, z, s);
    else
        launch_resid_silu(h, w1, b1, B, H, K, dt == MEDUSA_BF16, z, s);
}

medusa_status medusa_resid_silu(const void* h, const void* w1, medusa_layout w1_layout, const void* b1, int B,
                                int H, int K, medusa_dtype dt, float* z, void* stream) {
    return guarded("medusa_resid_silu", [&] {
        check_heads_shape(B, H, K, dt);
        check_w1_layout(H, dt, w1_layout);
        REQUIRE(h && w1 && b1 && z, "null pointer argument");
        run_resid_silu(h, w1, w1_layout, b1, B, H, K, dt, z, (hipStream_t)stream);
    });
}

size_t medusa_vocab_topk_workspace_size(int B, int H, int V, int K, int topk, medusa_dtype dt,
                                        medusa_layout w2_layout) {
    (void)dt;
    if (B < 1 || H < 1 || V < 1 || K < 1 || topk < 1) return 0;
    if (w2_layout == MEDUSA_PACKED) return vocab_topk_packed_ws_bytes(B, H, V, K, topk);
    const size_t G = (size_t)vocab_topk_groups(B, V, K);
    return align256((size_t)B * K * G * topk * 4) * 2;
}

static void carve_vocab_ws(void* ws, int B, int V, int K, int topk, float** cv, int** ci) {
    const size_t G = (size_t)vocab_topk_groups(B, V, K);
    const size_t one = align256((size_t)B * K * G * topk * 4);
    *cv = (float*)ws;
    *ci = (int*)((char*)ws + one);
}

static void check_vocab(int B, int H, int V, int K, int topk, medusa_dtype dt, medusa_layout w2_layout) {
    check_heads_shape(B, H, K, dt);
    REQUIRE(V >= 1, "V must be positive");
    REQUIRE(topk >= 1 && topk <= V, "topk=%d must be in [1, V]", topk);
    SUPPORT(topk <= MEDUSA_MAX_TOPK, "topk=%d exceeds %d", topk, MEDUSA_MAX_TOPK);
    REQUIRE(w2_layout == MEDUSA_ROW_MAJOR || w2_layout == MEDUSA_PACKED, "w2_layout must be ROW_MAJOR or PACKED");
    if (w2_layout == MEDUSA_PACKED) {
        SUPPORT(dt == MEDUSA_BF16, "a packed w2 must be bf16");
        SUPPORT(H % vocab_topk_packed_kc() == 0, "packed w2: H=%d must be a multiple of %d", H,
                vocab_topk_packed_kc());
    } else {
        SUPPORT(vocab_topk_lds_bytes(B, H, V, K) <= 160 * 1024, "B*H too large for the LDS-staged right-hand sides");
    }
}

// tb: build the candidate tree in the merge's launch (null: the merge alone)
static void run_vocab_topk(const float* z, const void* w2, medusa_layout w2_layout, int B, int H, int V, int K,
                           int topk, medusa_dtype dt, float* logits, int32_t* topk_idx, float* topk_val, void* ws,
                           hipStream_t s, const TreeBuild* tb = nullptr) {
    if (w2_layout == MEDUSA_PACKED) {
        if (tb) launch_vocab_topk_packed_tree(z, w2, B, H, V, K, topk, logits, topk_idx, topk_val, ws, *tb, s);
        else launch_vocab_topk_packed(z, w2, B, H, V, K, topk, logits, topk_idx, topk_val, ws, s);
        return;
    }
    float* cv;
    int* ci;
    carve_vocab_ws(ws, B, V, K, topk, &cv, &ci);
    if (tb)
        launch_vocab_topk_tree(z, w2, B, H, V, K, topk, dt == MEDUSA_BF16, logits, topk_idx, topk_val, cv, ci, *tb, s);
    else
        launch_vocab_topk(z, w2, B, H, V, K, topk, dt == MEDUSA_BF16, logits, topk_idx, topk_val, cv, ci, s);
}

medusa_status medusa_vocab_topk(const float* z, const void* w2, medusa_layout w2_layout, int B, int H, int V, int K,
                                int topk, medusa_dtype dt, float* logits, int32_t* topk_idx, float* topk_val,
                                void* ws, size_t ws_bytes, void* stream) {
    return guarded("medusa_vocab_topk", [&] {
        check_vocab(B, H, V, K, topk, dt, w2_layout);
        REQUIRE(z && w2 && topk_idx && topk_val && ws, "null pointer argument");
        const size_t need = medusa_vocab_topk_workspace_size(B, H, V, K, topk, dt, w2_layout);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        run_vocab_topk(z, w2, w2_layout, B, H, V, K, topk, dt, logits, topk_idx, topk_val, ws, (hipStream_t)stream);
    });
}

size_t medusa_heads_workspace_size(int B, int H, int V, int K, int topk, medusa_dtype dt, medusa_layout w2_layout) {
    if (B < 1 || H < 1 || V < 1 || K < 1 || topk < 1) return 0;
    return align256((size_t)B * K * H * 4) + medusa_vocab_topk_workspace_size(B, H, V, K, topk, dt, w2_layout);
}

// z = h for every head (lm_head mode)
__global__ void broadcast_h_kernel(const void* h, int B, int H, int K, int bf16, float* z) {
    const size_t n = (size_t)B * K * H;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t b = e / ((size_t)K * H), j = e % H;
        z[e] = bf16 ? bf16_to_f32(((const bf16_t*)h)[b * H + j]) : ((const float*)h)[b * H + j];
    }
}

medusa_status medusa_heads_forward(const void* h, const void* w1, const void* b1, const void* w2,
                                   medusa_layout layout, int B, int H, int V, int K, int topk, medusa_dtype dt,
                                   float* logits, int32_t* topk_idx, float* topk_val, void* ws, size_t ws_bytes,
                                   void* stream) {
    const medusa_layout w2_layout = layout;
    return guarded("medusa_heads_forward", [&] {
        check_vocab(B, H, V, K, topk, dt, w2_layout);
        if (w1) check_w1_layout(H, dt, layout);
        REQUIRE(h && w2 && topk_idx && topk_val && ws, "null pointer argument");
        REQUIRE((w1 == nullptr) == (b1 == nullptr), "w1 and b1 must both be given or both be NULL");
        const size_t need = medusa_heads_workspace_size(B, H, V, K, topk, dt, w2_layout);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        float* z = (float*)ws;
        void* vws = (char*)ws + align256((size_t)B * K * H * 4);
        hipStream_t s = (hipStream_t)stream;
        if (w1)
            run_resid_silu(h, w1, layout, b1, B, H, K, dt, z, s);
        else
            MEDUSA_LAUNCH("broadcast_h", broadcast_h_kernel, dim3(64), dim3(256), 0, s, h, B, H, K,
                          dt == MEDUSA_BF16 ? 1 : 0, z);
        run_vocab_topk(z, w2, w2_layout, B, H, V, K, topk, dt, logits, topk_idx, topk_val, vws, s);
    });
}

// the checks medusa_build_tree makes of a tree against K and topk
static void check_tree_for_heads(const medusa_tree* tree, int K, int topk) {
    REQUIRE(K >= tree->t.max_depth, "K=%d is smaller than the tree depth %d", K, tree->t.max_depth);
    REQUIRE(topk > tree->t.max_rank, "topk=%d does not cover rank %d", topk, tree->t.max_rank);
    SUPPORT(tree->t.max_depth * (tree->t.max_rank + 1) <= MEDUSA_MAX_DEPTH * MEDUSA_MAX_TOPK,
            "tree depth %d x ranks %d: more than %d candidates", tree->t.max_depth, tree->t.max_rank + 1,
            MEDUSA_MAX_DEPTH * MEDUSA_MAX_TOPK);
}

medusa_status medusa_heads_forward_tree(const void* h, const void* w1, const void* b1, const void* w2,
                                        medusa_layout layout, int B, int H, int V, int K, int topk, medusa_dtype dt,
                                        float* logits, int32_t* topk_idx, float* topk_val, const medusa_tree* tree,
                                        const int32_t* root_tok, const int32_t* cache_len, int32_t* node_tok,
                                        int32_t* node_pos, uint64_t* anc_mask, void* ws, size_t ws_bytes,
                                        void* stream) {
    const medusa_layout w2_layout = layout;
    return guarded("medusa_heads_forward_tree", [&] {
        check_vocab(B, H, V, K, topk, dt, w2_layout);
        if (w1) check_w1_layout(H, dt, layout);
        REQUIRE(h && w2 && topk_idx && topk_val && ws, "null pointer argument");
        REQUIRE(tree && root_tok && cache_len && node_tok && node_pos, "null pointer argument");
        REQUIRE((w1 == nullptr) == (b1 == nullptr), "w1 and b1 must both be given or both be NULL");
        check_tree_for_heads(tree, K, topk);
        const size_t need = medusa_heads_workspace_size(B, H, V, K, topk, dt, w2_layout);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        float* z = (float*)ws;
        void* vws = (char*)ws + align256((size_t)B * K * H * 4);
        hipStream_t s = (hipStream_t)stream;
        if (w1)
            run_resid_silu(h, w1, layout, b1, B, H, K, dt, z, s);
        else
            MEDUSA_LAUNCH("broadcast_h", broadcast_h_kernel, dim3(64), dim3(256), 0, s, h, B, H, K,
                          dt == MEDUSA_BF16 ? 1 : 0, z);
        TreeBuild tb;
        tb.t = &tree->t;
        tb.root_tok = root_tok;
        tb.cache_len = cache_len;
        tb.node_tok = node_tok;
        tb.node_pos = node_pos;
        tb.anc_mask = anc_mask;
        run_vocab_topk(z, w2, w2_layout, B, H, V, K, topk, dt, logits, topk_idx, topk_val, vws, s, &tb);
    });
}

// ---------------------------------------------------------------------------
// medusa_heads_forward without a caller workspace: z and the top-k partials
// go to `scratch`, a file-scope device array of MEDUSA_STATIC_SCRATCH_BYTES.
// In host code `scratch` names a host-side stand-in, not the device array, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
// ---------------------------------------------------------------------------
}  // extern "C"

static __device__ __align__(256) char scratch[MEDUSA_STATIC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_dev;  // per device: scratch's device address (null until looked up)

static void* scratch_on_current_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) failf(MEDUSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_dev.size() <= dev) g_scratch_dev.resize((size_t)dev + 1, nullptr);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            failf(MEDUSA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    return g_scratch_dev[dev];
}

extern "C" {

medusa_status medusa_heads_forward_static(const void* h, const void* w1, const void* b1, const void* w2,
                                          medusa_layout layout, int B, int H, int V, int K, int topk,
                                          medusa_dtype dt, float* logits, int32_t* topk_idx, float* topk_val,
                                          void* stream) {
    return guarded("medusa_heads_forward_static", [&] {
        // the same argument checks as medusa_heads_forward, then the size limit
        check_vocab(B, H, V, K, topk, dt, layout);
        if (w1) check_w1_layout(H, dt, layout);
        REQUIRE(h && w2 && topk_idx && topk_val, "null pointer argument");
        REQUIRE((w1 == nullptr) == (b1 == nullptr), "w1 and b1 must both be given or both be NULL");
        const size_t need = medusa_heads_workspace_size(B, H, V, K, topk, dt, layout);
        SUPPORT(need <= MEDUSA_STATIC_SCRATCH_BYTES,
                "these sizes need %zu bytes of scratch; the static array holds %zu (use medusa_heads_forward)",
                need, (size_t)MEDUSA_STATIC_SCRATCH_BYTES);
        void* ws = scratch_on_current_device();
        float* z = (float*)ws;
        void* vws = (char*)ws + align256((size_t)B * K * H * 4);
        hipStream_t s = (hipStream_t)stream;
        if (w1)
            run_resid_silu(h, w1, layout, b1, B, H, K, dt, z, s);
        else
            MEDUSA_LAUNCH("broadcast_h", broadcast_h_kernel, dim3(64), dim3(256), 0, s, h, B, H, K,
                          dt == MEDUSA_BF16 ? 1 : 0, z);
        run_vocab_topk(z, w2, layout, B, H, V, K, topk, dt, logits, topk_idx, topk_val, vws, s);
    });
}

// ---------------------------------------------------------------------------
// a3 tree
// ---------------------------------------------------------------------------
medusa_status medusa_tree_create(const int32_t* parent, const int32_t* rank, int N, int K, int topk,
                                 medusa_tree** out) {
    g_err.clear();
    try {
        REQUIRE(parent && rank && out, "null pointer argument");
        REQUIRE(N >= 1, "N must be >= 1");
        SUPPORT(N <= MEDUSA_MAX_TREE_NODES, "N=%d exceeds %d", N, MEDUSA_MAX_TREE_NODES);
        REQUIRE(K >= 1 && topk >= 1, "K and topk must be >= 1");
        SUPPORT(topk <= MEDUSA_MAX_TOPK, "topk=%d exceeds %d", topk, MEDUSA_MAX_TOPK);
        REQUIRE(parent[0] == -1, "parent[0] must be -1 (root)");
        TreeDev t;
        t.N = N;
        t.W = (N + 63) / 64;
        t.K = K;
        t.topk = topk;
        t.h_parent.assign(parent, parent + N);
        t.h_rank.assign(N, 0);
        t.h_depth.assign(N, 0);
        std::vector<uint32_t> seen((size_t)N * ((topk + 31) / 32), 0u);
        for (int i = 1; i < N; ++i) {
            const int p = parent[i];
            REQUIRE(p >= 0 && p < i, "parent[%d]=%d must satisfy 0 <= parent < index", i, p);
            REQUIRE(rank[i] >= 0 && rank[i] < topk, "rank[%d]=%d must be in [0, topk=%d)", i, rank[i], topk);
            t.h_depth[i] = t.h_depth[p] + 1;
            t.h_rank[i] = rank[i];
            REQUIRE(t.h_depth[i] <= K, "node %d has depth %d > K=%d", i, t.h_depth[i], K);
            uint32_t& w = seen[(size_t)p * ((topk + 31) / 32) + rank[i] / 32];
            REQUIRE(!(w & (1u << (rank[i] % 32))), "node %d repeats rank %d under parent %d", i, rank[i], p);
            w |= 1u << (rank[i] % 32);
            if (t.h_depth[i] > t.max_depth) t.max_depth = t.h_depth[i];
            if (rank[i] > t.max_rank) t.max_rank = rank[i];
        }
        t.h_mask.assign((size_t)N * t.W, 0ull);
        for (int i = 0; i < N; ++i)
            for (int j = i; j >= 0; j = j > 0 ? t.h_parent[j] : -1) t.h_mask[(size_t)i * t.W + j / 64] |= 1ull << (j % 64);
        // upload
        hipError_t e = hipSuccess;
        auto up = [&](void** dst, const void* src, size_t bytes) {
            if (e != hipSuccess) return;
            e = hipMalloc(dst, bytes);
            if (e == hipSuccess) e = hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice);
        };
        up((void**)&t.parent, t.h_parent.data(), N * sizeof(int));
        up((void**)&t.depth, t.h_depth.data(), N * sizeof(int));
        up((void**)&t.rank, t.h_rank.data(), N * sizeof(int));
        up((void**)&t.mask, t.h_mask.data(), t.h_mask.size() * sizeof(uint64_t));
        const int zero = 0;
        up((void**)&t.status, &zero, sizeof(int));
        if (e != hipSuccess) {
            // best-effort cleanup of what was allocated; the upload error is the one reported
            (void)hipFree(t.parent); (void)hipFree(t.depth); (void)hipFree(t.rank); (void)hipFree(t.mask);
            (void)hipFree(t.status);
            set_error(std::string("medusa_tree_create: ") + hipGetErrorString(e));
            return MEDUSA_EHIP;
        }
        medusa_tree* obj = new medusa_tree;
        obj->t = std::move(t);
        *out = obj;
    } catch (const Fail& x) {
        return x.st;
    }
    return MEDUSA_OK;
}

void medusa_tree_destroy(medusa_tree* tree) {
    if (!tree) return;
    // no status to return: a failed free (only after an earlier sticky
    // device error) leaks the five small arrays
    (void)hipFree(tree->t.parent);
    (void)hipFree(tree->t.depth);
    (void)hipFree(tree->t.rank);
    (void)hipFree(tree->t.mask);
    (void)hipFree(tree->t.status);
    delete tree;
}

static_assert(MEDUSA_STATUS_CACHE_LEN_CLAMPED == STATUS_CACHE_LEN_CLAMPED &&
                  MEDUSA_STATUS_CACHE_OVERFLOW == STATUS_CACHE_OVERFLOW,
              "status bits of the header and the kernels");

medusa_status medusa_tree_status(const medusa_tree* tree, int32_t* flags, int clear, void* stream) {
    return guarded("medusa_tree_status", [&] {
        REQUIRE(tree && flags, "null pointer argument");
        hipStream_t s = (hipStream_t)stream;
        hipError_t e = hipStreamSynchronize(s);
        int32_t v = 0;
        if (e == hipSuccess) e = hipMemcpy(&v, tree->t.status, sizeof(int32_t), hipMemcpyDeviceToHost);
        if (e == hipSuccess && clear) e = hipMemsetAsync(tree->t.status, 0, sizeof(int32_t), s);
        if (e == hipSuccess && clear) e = hipStreamSynchronize(s);
        if (e != hipSuccess) failf(MEDUSA_EHIP, "medusa_tree_status: %s", hipGetErrorString(e));
        *flags = v;
    });
}

int medusa_tree_num_nodes(const medusa_tree* tree) { return tree ? tree->t.N : 0; }
int medusa_tree_max_depth(const medusa_tree* tree) { return tree ? tree->t.max_depth : 0; }

medusa_status medusa_tree_mask_host(const medusa_tree* tree, uint64_t* mask, size_t words) {
    g_err.clear();
    if (!tree || !mask) { set_error("null pointer argument"); return MEDUSA_EINVAL; }
    if (words < tree->t.h_mask.size()) { set_error("mask buffer too small"); return MEDUSA_EINVAL; }
    memcpy(mask, tree->t.h_mask.data(), tree->t.h_mask.size() * sizeof(uint64_t));
    return MEDUSA_OK;
}

medusa_status medusa_build_tree(const medusa_tree* tree, const int32_t* topk_idx, const int32_t* root_tok,
                                const int32_t* cache_len, int B, int K, int topk, int32_t* node_tok,
                                int32_t* node_pos, uint64_t* anc_mask, void* stream) {
    return guarded("medusa_build_tree", [&] {
        REQUIRE(tree && topk_idx && root_tok && cache_len && node_tok && node_pos, "null pointer argument");
        REQUIRE(B >= 1, "B must be >= 1");
        check_tree_for_heads(tree, K, topk);
        launch_build_tree(tree->t, topk_idx, K, topk, root_tok, cache_len, B, node_tok, node_pos, anc_mask,
                          (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// a4 tree attention
// ---------------------------------------------------------------------------
size_t tree_attention_workspace_size(const medusa_tree* tree, int B, int nH, int D, int max_cache_len,
                                     medusa_dtype dt) {
    if (!tree || B < 1 || nH < 1 || D < 1 || max_cache_len < 0) return 0;
    return attn_workspace_bytes(B, nH, tree->t.N, D, max_cache_len, dt == MEDUSA_BF16);
}

medusa_status tree_attention_verify(const void* q, const void* k_tree, const void* v_tree, void* k_cache,
                                    void* v_cache, const int32_t* cache_len, int max_cache_len,
                                    const medusa_tree* tree, int B, int nH, int nKV, int D, int Lmax, float scale,
                                    medusa_dtype dt, void* out, void* ws, size_t ws_bytes, void* stream) {
    return guarded("tree_attention_verify", [&] {
        REQUIRE(tree && q && k_tree && v_tree && k_cache && v_cache && cache_len && out && ws,
                "null pointer argument");
        REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "bad dtype");
        REQUIRE(B >= 1 && nH >= 1 && nKV >= 1 && nH % nKV == 0, "need nH %% nKV == 0 (nH=%d nKV=%d)", nH, nKV);
        SUPPORT(D == 64 || D == 128, "D=%d not in {64, 128}", D);
        REQUIRE(max_cache_len >= 0 && max_cache_len + tree->t.N <= Lmax,
                "max_cache_len + N = %d exceeds Lmax = %d", max_cache_len + tree->t.N, Lmax);
        const size_t need = tree_attention_workspace_size(tree, B, nH, D, max_cache_len, dt);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        float* part_o;
        float* part_ml;
        attn_carve(B, nH, tree->t.N, D, max_cache_len, dt == MEDUSA_BF16, ws, &part_o, &part_ml);
        launch_tree_attention(q, k_tree, v_tree, k_cache, v_cache, cache_len, max_cache_len, tree->t, B, nH, nKV, D,
                              Lmax, scale, dt == MEDUSA_BF16, out, part_o, part_ml, (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// a5 base greedy
// ---------------------------------------------------------------------------
size_t medusa_base_greedy_workspace_size(int R, int H, int V, medusa_dtype dt, medusa_layout lm_layout) {
    if (R < 1 || H < 1 || V < 1) return 0;
    (void)dt;
    return greedy_workspace_bytes(R, H, V, lm_layout == MEDUSA_PACKED);
}

medusa_status medusa_base_greedy(const void* x, const void* lm_head, medusa_layout lm_layout, int R, int H, int V,
                                 float eps, medusa_dtype dt, int32_t* greedy, float* logits, void* ws,
                                 size_t ws_bytes, void* stream) {
    return guarded("medusa_base_greedy", [&] {
        REQUIRE(x && lm_head && greedy && ws, "null pointer argument");
        REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "bad dtype");
        REQUIRE(lm_layout == MEDUSA_ROW_MAJOR || lm_layout == MEDUSA_PACKED, "bad lm_head layout");
        REQUIRE(R >= 1 && V >= 1 && H >= 1, "R, H, V must be positive");
        SUPPORT(H % 8 == 0 && H <= 8192, "H=%d must be a multiple of 8 and <= 8192", H);
        if (lm_layout == MEDUSA_PACKED) {
            SUPPORT(dt == MEDUSA_BF16, "a packed lm_head must be bf16");
            SUPPORT(H % 64 == 0, "H=%d must be a multiple of 64 for a packed lm_head", H);
        }
        REQUIRE(eps >= 0.f, "eps must be >= 0");
        const size_t need = medusa_base_greedy_workspace_size(R, H, V, dt, lm_layout);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        launch_base_greedy(x, lm_head, lm_layout == MEDUSA_PACKED, R, H, V, eps, dt == MEDUSA_BF16, greedy, logits, ws,
                           (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// weight packing
// ---------------------------------------------------------------------------
size_t medusa_packed_size(int rows, int cols) {
    if (rows < 1 || cols < 1 || cols % 32 != 0) return 0;
    return packed_elems(rows, cols) * 2;
}

medusa_status medusa_pack_rows(const void* src, int rows, int cols, void* dst, int dst_row0, int dst_rows,
                               int interleave, void* stream) {
    return guarded("medusa_pack_rows", [&] {
        REQUIRE(src && dst, "null pointer argument");
        REQUIRE(rows >= 1 && cols >= 1, "rows and cols must be positive");
        SUPPORT(cols % 32 == 0, "cols=%d must be a multiple of 32", cols);
        REQUIRE(interleave >= 1, "interleave must be >= 1");
        if (interleave == 1) {
            REQUIRE(dst_row0 >= 0 && (int64_t)dst_row0 + rows <= dst_rows,
                    "rows [%d, %d) do not fit the %d packed rows", dst_row0, dst_row0 + rows, dst_rows);
        } else {
            REQUIRE(rows % 16 == 0 && dst_row0 % 16 == 0 && dst_row0 >= 0 && dst_row0 < 16 * interleave,
                    "interleaved packing needs rows and dst_row0 multiples of 16, dst_row0 < 16 * interleave");
            REQUIRE((int64_t)dst_row0 + (int64_t)(rows / 16 - 1) * 16 * interleave + 16 <= dst_rows,
                    "interleaved rows do not fit the %d packed rows", dst_rows);
        }
        launch_pack_rows((const bf16_t*)src, rows, cols, (bf16_t*)dst, dst_row0, dst_rows, interleave,
                         (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// a6 + a7 accept and compaction
// ---------------------------------------------------------------------------
medusa_status medusa_accept(const medusa_tree* tree, const int32_t* node_tok, const int32_t* greedy, int B,
                            int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                            const int32_t* cache_len, int32_t* new_cache_len, void* k_cache, void* v_cache,
                            int n_layers, int64_t layer_stride_elems, int nKV, int D, int Lmax, medusa_dtype dt,
                            void* stream) {
    return guarded("medusa_accept", [&] {
        REQUIRE(tree && node_tok && greedy && accept_len && accept_nodes && out_tokens && cache_len &&
                    new_cache_len,
                "null pointer argument");
        REQUIRE(B >= 1, "B must be >= 1");
        SUPPORT(tree->t.max_depth <= MEDUSA_MAX_DEPTH, "tree depth %d exceeds %d", tree->t.max_depth,
                MEDUSA_MAX_DEPTH);
        REQUIRE((k_cache == nullptr) == (v_cache == nullptr), "k_cache and v_cache must both be given or both NULL");
        if (k_cache) {
            REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "bad dtype");
            REQUIRE(n_layers >= 1 && nKV >= 1 && D >= 1 && Lmax >= tree->t.N, "bad cache shape");
            SUPPORT(D <= 128, "D=%d exceeds 128", D);
            REQUIRE(layer_stride_elems >= (int64_t)B * nKV * Lmax * D || n_layers == 1,
                    "layer stride smaller than one layer's cache");
        }
        launch_accept(tree->t, node_tok, greedy, B, accept_len, accept_nodes, out_tokens, cache_len, new_cache_len,
                      k_cache, v_cache, n_layers, layer_stride_elems, nKV, D, Lmax, dt == MEDUSA_BF16,
                      (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// typical acceptance (sampling mode)
// ---------------------------------------------------------------------------
size_t medusa_typical_accept_workspace_size(const medusa_tree* tree, int B) {
    if (!tree || B < 1) return 0;
    return typical_accept_workspace_bytes(B, tree->t.N);
}

medusa_status medusa_typical_accept(const medusa_tree* tree, const int32_t* node_tok, const float* logits, int B,
                                    int V, float temperature, float epsilon, float delta, const float* uniform,
                                    int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                                    const int32_t* cache_len, int32_t* new_cache_len, void* k_cache, void* v_cache,
                                    int n_layers, int64_t layer_stride_elems, int nKV, int D, int Lmax,
                                    medusa_dtype dt, void* ws, size_t ws_bytes, void* stream) {
    return guarded("medusa_typical_accept", [&] {
        REQUIRE(tree && node_tok && logits && uniform && accept_len && accept_nodes && out_tokens && cache_len &&
                    new_cache_len && ws,
                "null pointer argument");
        REQUIRE(B >= 1 && V >= 1, "B and V must be positive (B=%d V=%d)", B, V);
        SUPPORT(V <= typical_max_vocab(), "V=%d exceeds %d", V, typical_max_vocab());
        SUPPORT(tree->t.max_depth <= MEDUSA_MAX_DEPTH, "tree depth %d exceeds %d", tree->t.max_depth,
                MEDUSA_MAX_DEPTH);
        REQUIRE(temperature > 0.f && epsilon > 0.f && delta > 0.f,
                "temperature, epsilon and delta must be positive (%g %g %g)", temperature, epsilon, delta);
        REQUIRE(ws_bytes >= typical_accept_workspace_bytes(B, tree->t.N), "workspace too small");
        REQUIRE((k_cache == nullptr) == (v_cache == nullptr), "k_cache and v_cache must both be given or both NULL");
        if (k_cache) {
            REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "bad dtype");
            REQUIRE(n_layers >= 1 && nKV >= 1 && D >= 1 && Lmax >= tree->t.N, "bad cache shape");
            SUPPORT(D <= 128, "D=%d exceeds 128", D);
            REQUIRE(layer_stride_elems >= (int64_t)B * nKV * Lmax * D || n_layers == 1,
                    "layer stride smaller than one layer's cache");
        }
        launch_typical_accept(tree->t, node_tok, logits, B, V, temperature, epsilon, delta, uniform, accept_len,
                              accept_nodes, out_tokens, cache_len, new_cache_len, k_cache, v_cache, n_layers,
                              layer_stride_elems, nKV, D, Lmax, dt == MEDUSA_BF16, ws, (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// speculative sampling on a chain of drafts
// ---------------------------------------------------------------------------
medusa_status medusa_speculative_sample(const float* p, const float* q, const int32_t* drafts, const float* u_accept,
                                        const float* u_resample, int B, int gamma, int V, int32_t* n_accepted,
                                        int32_t* out_tokens, void* stream) {
    return guarded("medusa_speculative_sample", [&] {
        REQUIRE(p && u_resample && n_accepted && out_tokens, "null pointer argument");
        REQUIRE(gamma == 0 || (q && drafts && u_accept), "null draft argument");
        REQUIRE(B >= 1 && V >= 1 && gamma >= 0, "need B >= 1, V >= 1, gamma >= 0 (B=%d V=%d gamma=%d)", B, V,
                gamma);
        SUPPORT(gamma <= 64, "gamma=%d exceeds 64", gamma);
        SUPPORT(V <= typical_max_vocab(), "V=%d exceeds %d", V, typical_max_vocab());
        launch_speculative_sample(p, q, drafts, u_accept, u_resample, B, gamma, V, n_accepted, out_tokens,
                                  (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// hand-off to the next round
// ---------------------------------------------------------------------------
medusa_status medusa_advance(const medusa_tree* tree, const int32_t* accept_len, const int32_t* accept_nodes,
                             const int32_t* out_tokens, const float* hidden, int B, int H, medusa_dtype dt,
                             int32_t* root_tok, void* h, int32_t* tokens, int32_t* n_tokens, int cap,
                             const int32_t* new_cache_len, int32_t* cache_len, void* stream) {
    return guarded("medusa_advance", [&] {
        REQUIRE(tree && accept_len && accept_nodes && out_tokens && hidden && root_tok && h, "null pointer argument");
        REQUIRE(B >= 1 && H >= 1, "B and H must be positive (B=%d H=%d)", B, H);
        SUPPORT(tree->t.max_depth <= MEDUSA_MAX_DEPTH, "tree depth %d exceeds %d", tree->t.max_depth,
                MEDUSA_MAX_DEPTH);
        REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, "bad dtype");
        REQUIRE((tokens == nullptr) == (n_tokens == nullptr), "tokens and n_tokens must both be given or both NULL");
        REQUIRE(tokens == nullptr || cap >= 1, "cap=%d must be >= 1 when tokens are appended", cap);
        REQUIRE((new_cache_len == nullptr) == (cache_len == nullptr),
                "new_cache_len and cache_len must both be given or both NULL");
        launch_advance(tree->t, accept_len, accept_nodes, out_tokens, hidden, B, H, dt == MEDUSA_BF16, root_tok, h,
                       tokens, n_tokens, cap, new_cache_len, cache_len, (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// measurement aid: planted base-model choices
// ---------------------------------------------------------------------------
medusa_status medusa_plant_greedy(const medusa_tree* tree, const int32_t* topk_idx, const int32_t* cache_len, int B,
                                  int K, int topk, int V, const float* alpha, int n_alpha, uint64_t seed,
                                  int32_t* greedy, void* stream) {
    return guarded("medusa_plant_greedy", [&] {
        REQUIRE(alpha && n_alpha >= 1, "need at least one alpha");
        REQUIRE(tree && topk_idx && cache_len && greedy, "null pointer argument");
        REQUIRE(B >= 1 && V >= 1, "B and V must be positive (B=%d V=%d)", B, V);
        REQUIRE(K >= tree->t.max_depth, "K=%d is smaller than the tree depth %d", K, tree->t.max_depth);
        REQUIRE(topk >= 1 && topk > tree->t.max_rank, "topk=%d does not cover rank %d", topk, tree->t.max_rank);
        SUPPORT(tree->t.max_depth <= MEDUSA_MAX_DEPTH, "tree depth %d exceeds %d", tree->t.max_depth,
                MEDUSA_MAX_DEPTH);
        PlantAlphas pa;
        for (int d = 0; d < 16; ++d) {
            pa.a[d] = alpha[d < n_alpha ? d : n_alpha - 1];
            REQUIRE(pa.a[d] >= 0.f && pa.a[d] <= 1.f, "alpha=%g must be in [0, 1]", pa.a[d]);
        }
        launch_plant_greedy(tree->t, topk_idx, B, K, topk, cache_len, pa, seed, V, greedy, (hipStream_t)stream);
    });
}

medusa_status medusa_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, void* stream) {
    return guarded("medusa_stream_read", [&] {
        REQUIRE(src && sink, "null pointer argument");
        REQUIRE(bytes >= 16 && bytes % 16 == 0, "bytes=%zu must be a positive multiple of 16", bytes);
        REQUIRE(((uintptr_t)src & 15) == 0, "src must be 16-byte aligned");
        REQUIRE(n_wg >= 1 && n_wg <= (1 << 20), "n_wg=%d must be in [1, 2^20]", n_wg);
        launch_stream_read(src, bytes, sink, n_wg, (hipStream_t)stream);
    });
}

medusa_status medusa_read_mix(const void* window, size_t window_bytes, const void* src, size_t src_bytes,
                              int window_parts, int stream_parts, int rounds, uint32_t* sink, int n_wg, void* stream) {
    return guarded("medusa_read_mix", [&] {
        REQUIRE(sink, "null pointer argument");
        REQUIRE(read_mix_supported(window_parts, stream_parts),
                "(window_parts, stream_parts) = (%d, %d) must be (8, 0), (0, 8), (4, 2) or (8, 4)", window_parts,
                stream_parts);
        REQUIRE(rounds >= 1 && rounds <= (1 << 20), "rounds=%d must be in [1, 2^20]", rounds);
        REQUIRE(n_wg >= 1 && n_wg <= (1 << 16), "n_wg=%d must be in [1, 2^16]", n_wg);
        if (window_parts > 0) {
            REQUIRE(window, "null window");
            REQUIRE(window_bytes >= 1 && window_bytes % ((size_t)window_parts * 4096) == 0,
                    "window_bytes=%zu must be a positive multiple of window_parts x 4096", window_bytes);
            REQUIRE(((uintptr_t)window & 15) == 0, "window must be 16-byte aligned");
        }
        if (stream_parts > 0) {
            REQUIRE(src, "null src");
            REQUIRE(((uintptr_t)src & 15) == 0, "src must be 16-byte aligned");
            const size_t need = (size_t)rounds * stream_parts * 4096 * n_wg;
            REQUIRE(src_bytes >= need, "src_bytes=%zu < %zu (rounds x stream_parts x 4096 x n_wg)", src_bytes, need);
        }
        launch_read_mix(window, window_bytes, src, window_parts, stream_parts, rounds, sink, n_wg,
                        (hipStream_t)stream);
    });
}

medusa_status medusa_mfma_rate(int random_operands, int iters, float* out, int n_wg, void* stream) {
    return guarded("medusa_mfma_rate", [&] {
        REQUIRE(out, "null pointer argument");
        REQUIRE(random_operands == 0 || random_operands == 1, "random_operands must be 0 or 1");
        REQUIRE(iters >= 1 && iters <= (1 << 20), "iters=%d must be in [1, 2^20]", iters);
        REQUIRE(n_wg >= 1 && n_wg <= (1 << 16), "n_wg=%d must be in [1, 2^16]", n_wg);
        launch_mfma_rate(random_operands, iters, out, n_wg, (hipStream_t)stream);
    });
}

medusa_status medusa_accept_stats(const medusa_tree* tree, const int32_t* accept_len, const int32_t* accept_nodes,
                                  const int32_t* out_tokens, const int32_t* topk_idx, int B, int K, int topk,
                                  int32_t* counts, void* stream) {
    return guarded("medusa_accept_stats", [&] {
        REQUIRE(tree && accept_len && accept_nodes && out_tokens && topk_idx && counts, "null pointer argument");
        REQUIRE(B >= 1 && topk >= 1, "B and topk must be positive");
        REQUIRE(K >= tree->t.max_depth && K >= 1, "K=%d is smaller than the tree depth %d", K, tree->t.max_depth);
        SUPPORT(K <= 64 && tree->t.max_depth <= MEDUSA_MAX_DEPTH, "K=%d or the tree depth exceeds the limits", K);
        launch_accept_stats(tree->t, accept_len, accept_nodes, out_tokens, topk_idx, B, K, topk, counts,
                            (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// choosing a tree: the N rank tuples with the largest product of per-depth
// acceptance probabilities, best first
// ---------------------------------------------------------------------------
medusa_status medusa_tree_select(const double* acc, int K, int topk, int N, int32_t* parent, int32_t* rank) {
    g_err.clear();
    try {
        REQUIRE(acc && parent && rank, "null pointer argument");
        REQUIRE(K >= 1 && topk >= 1 && N >= 1, "K, topk and N must be positive");
        SUPPORT(N <= MEDUSA_MAX_TREE_NODES && topk <= MEDUSA_MAX_TOPK && K <= MEDUSA_MAX_DEPTH,
                "N=%d, topk=%d or K=%d exceeds the limits", N, topk, K);
        for (int i = 0; i < K * topk; ++i) REQUIRE(acc[i] >= 0.0 && acc[i] <= 1.0, "acc[%d]=%g not in [0, 1]", i, acc[i]);
        // a candidate: (product, rank tuple); best = larger product, then
        // shallower, then the lexicographically smaller tuple
        struct Cand {
            double prod;
            std::vector<int> path;
        };
        auto worse = [](const Cand& a, const Cand& b) {  // a ranks after b
            if (a.prod != b.prod) return a.prod < b.prod;
            if (a.path.size() != b.path.size()) return a.path.size() > b.path.size();
            return b.path < a.path;
        };
        std::vector<Cand> heap;
        auto push = [&](std::vector<int> p) {
            double prod = 1.0;
            for (size_t d = 0; d < p.size(); ++d) prod *= acc[d * topk + p[d]];
            heap.push_back(Cand{prod, std::move(p)});
            std::push_heap(heap.begin(), heap.end(), worse);
        };
        std::vector<std::vector<int>> chosen{{}};
        for (int r = 0; r < topk; ++r) push({r});
        while ((int)chosen.size() < N && !heap.empty()) {
            std::pop_heap(heap.begin(), heap.end(), worse);
            Cand c = std::move(heap.back());
            heap.pop_back();
            if ((int)c.path.size() < K)
                for (int r = 0; r < topk; ++r) {
                    std::vector<int> q = c.path;
                    q.push_back(r);
                    push(std::move(q));
                }
            chosen.push_back(std::move(c.path));
        }
        REQUIRE((int)chosen.size() == N, "only %zu candidates exist for N=%d", chosen.size(), N);
        // breadth-first order: by depth, then rank tuple
        std::sort(chosen.begin(), chosen.end(), [](const std::vector<int>& a, const std::vector<int>& b) {
            return a.size() != b.size() ? a.size() < b.size() : a < b;
        });
        std::map<std::vector<int>, int> index;
        for (int i = 0; i < N; ++i) index[chosen[i]] = i;
        parent[0] = -1;
        rank[0] = 0;
        for (int i = 1; i < N; ++i) {
            std::vector<int> up(chosen[i].begin(), chosen[i].end() - 1);
            auto it = index.find(up);
            // products of probabilities <= 1 never grow along a path, so the
            // best-first set is prefix-closed; equal products keep the order
            // above (a parent is shallower than its child)
            REQUIRE(it != index.end(), "internal: chosen set not prefix-closed");
            parent[i] = it->second;
            rank[i] = chosen[i].back();
        }
    } catch (const Fail& x) {
        return x.st;
    }
    return MEDUSA_OK;
}

// ---------------------------------------------------------------------------
// a8 decoder verify
// ---------------------------------------------------------------------------
size_t medusa_decoder_workspace_size(const medusa_tree* tree, int B, int H, int nH, int nKV, int D, int F, int V,
                                     int max_cache_len) {
    if (!tree || B < 1 || H < 1 || nH < 1 || nKV < 1 || D < 1 || F < 1 || V < 1 || max_cache_len < 0) return 0;
    return decoder_workspace_bytes(B, tree->t.N, H, nH, nKV, D, F, V, max_cache_len);
}

medusa_status medusa_decoder_verify(const medusa_layer_weights* layers, int n_layers, const void* embedding,
                                    const void* lm_head, const medusa_tree* tree, const int32_t* node_tok,
                                    const int32_t* node_pos, const int32_t* cache_len, int max_cache_len,
                                    void* k_cache, void* v_cache, int64_t layer_stride_elems, int B, int H, int nH,
                                    int nKV, int D, int F, int V, int Lmax, float rms_eps, float rope_base,
                                    int32_t* greedy, float* hidden, void* ws, size_t ws_bytes, void* stream) {
    return guarded("medusa_decoder_verify", [&] {
        REQUIRE(layers && embedding && lm_head && tree && node_tok && node_pos && cache_len && k_cache && v_cache &&
                    greedy && ws,
                "null pointer argument");
        REQUIRE(n_layers >= 1 && B >= 1 && H >= 1 && nH >= 1 && nKV >= 1 && D >= 1 && F >= 1 && V >= 1,
                "sizes must be positive");
        REQUIRE(nH % nKV == 0, "need nH %% nKV == 0 (nH=%d nKV=%d)", nH, nKV);
        SUPPORT(H == nH * D, "H=%d must equal nH*D=%d", H, nH * D);
        SUPPORT(D == 64 || D == 128, "D=%d not in {64, 128}", D);
        const int R = B * tree->t.N;
        SUPPORT(R <= MEDUSA_MAX_TREE_NODES, "B*N=%d exceeds %d", R, MEDUSA_MAX_TREE_NODES);
        SUPPORT(H % 64 == 0 && F % 64 == 0, "H=%d and F=%d must be multiples of 64", H, F);
        SUPPORT(H <= 16384, "H=%d exceeds 16384", H);
        REQUIRE(rms_eps >= 0.f && rope_base > 1.f, "need rms_eps >= 0 and rope_base > 1");
        REQUIRE(max_cache_len >= 0 && max_cache_len + tree->t.N <= Lmax,
                "max_cache_len + N = %d exceeds Lmax = %d", max_cache_len + tree->t.N, Lmax);
        REQUIRE(layer_stride_elems >= (int64_t)B * nKV * Lmax * D || n_layers == 1,
                "layer stride smaller than one layer's cache");
        std::vector<LayerPtrs> L((size_t)n_layers);
        for (int l = 0; l < n_layers; ++l) {
            const medusa_layer_weights& w = layers[l];
            REQUIRE(w.wqkv && w.wo && w.w_gate_up && w.w_down, "layer %d: null weight", l);
            L[l] = LayerPtrs{(const bf16_t*)w.wqkv, (const bf16_t*)w.wo, (const bf16_t*)w.w_gate_up,
                             (const bf16_t*)w.w_down};
        }
        const size_t need = medusa_decoder_workspace_size(tree, B, H, nH, nKV, D, F, V, max_cache_len);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        launch_decoder_verify(L.data(), n_layers, (const bf16_t*)embedding, (const bf16_t*)lm_head, tree->t, node_tok,
                              node_pos, cache_len, max_cache_len, (bf16_t*)k_cache, (bf16_t*)v_cache,
                              layer_stride_elems, B, H, nH, nKV, D, F, V, Lmax, rms_eps, rope_base, greedy, hidden, ws,
                              (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// prefill: a prompt through the decoder in chain-tree passes
// ---------------------------------------------------------------------------
static bool is_chain(const TreeDev& t) {
    for (int i = 1; i < t.N; ++i)
        if (t.h_parent[i] != i - 1) return false;
    return true;
}

size_t medusa_prefill_workspace_size(const medusa_tree* chain, int B, int H, int nH, int nKV, int D, int F, int V,
                                     int T, int max_cache_len) {
    if (!chain || B < 1 || H < 1 || nH < 1 || nKV < 1 || D < 1 || F < 1 || V < 1 || T < 1 || max_cache_len < 0)
        return 0;
    return prefill_workspace_bytes(B, chain->t.N, H, nH, nKV, D, F, V, T, max_cache_len);
}

medusa_status medusa_prefill(const medusa_layer_weights* layers, int n_layers, const void* embedding,
                             const void* lm_head, const medusa_tree* chain, const int32_t* tokens, int T,
                             int32_t* cache_len, int max_cache_len, void* k_cache, void* v_cache,
                             int64_t layer_stride_elems, int B, int H, int nH, int nKV, int D, int F, int V, int Lmax,
                             float rms_eps, float rope_base, int32_t* next_tok, void* hidden,
                             medusa_dtype hidden_dt, void* ws, size_t ws_bytes, void* stream) {
    return guarded("medusa_prefill", [&] {
        REQUIRE(hidden_dt == MEDUSA_F32 || hidden_dt == MEDUSA_BF16, "bad hidden dtype");
        REQUIRE(layers && embedding && lm_head && chain && tokens && cache_len && k_cache && v_cache && next_tok &&
                    hidden && ws,
                "null pointer argument");
        REQUIRE(is_chain(chain->t), "the tree handle must be a chain (parent[i] = i - 1)");
        REQUIRE(T >= 1, "T=%d must be positive", T);
        REQUIRE(n_layers >= 1 && B >= 1 && H >= 1 && nH >= 1 && nKV >= 1 && D >= 1 && F >= 1 && V >= 1,
                "sizes must be positive");
        REQUIRE(nH % nKV == 0, "need nH %% nKV == 0 (nH=%d nKV=%d)", nH, nKV);
        SUPPORT(H == nH * D, "H=%d must equal nH*D=%d", H, nH * D);
        SUPPORT(D == 64 || D == 128, "D=%d not in {64, 128}", D);
        const int C = chain->t.N;
        SUPPORT(B * C <= MEDUSA_MAX_TREE_NODES, "B*C=%d exceeds %d", B * C, MEDUSA_MAX_TREE_NODES);
        SUPPORT(H % 64 == 0 && F % 64 == 0, "H=%d and F=%d must be multiples of 64", H, F);
        SUPPORT(H <= 16384, "H=%d exceeds 16384", H);
        REQUIRE(rms_eps >= 0.f && rope_base > 1.f, "need rms_eps >= 0 and rope_base > 1");
        const int passes = (T + C - 1) / C;
        REQUIRE(max_cache_len >= 0 && (int64_t)max_cache_len + (int64_t)passes * C <= Lmax,
                "max_cache_len + %d passes x %d = %lld exceeds Lmax = %d", passes, C,
                (long long)max_cache_len + (long long)passes * C, Lmax);
        REQUIRE(layer_stride_elems >= (int64_t)B * nKV * Lmax * D || n_layers == 1,
                "layer stride smaller than one layer's cache");
        std::vector<LayerPtrs> L((size_t)n_layers);
        for (int l = 0; l < n_layers; ++l) {
            const medusa_layer_weights& w = layers[l];
            REQUIRE(w.wqkv && w.wo && w.w_gate_up && w.w_down, "layer %d: null weight", l);
            L[l] = LayerPtrs{(const bf16_t*)w.wqkv, (const bf16_t*)w.wo, (const bf16_t*)w.w_gate_up,
                             (const bf16_t*)w.w_down};
        }
        const size_t need = medusa_prefill_workspace_size(chain, B, H, nH, nKV, D, F, V, T, max_cache_len);
        REQUIRE(ws_bytes >= need, "workspace too small: %zu < %zu", ws_bytes, need);
        launch_prefill(L.data(), n_layers, (const bf16_t*)embedding, (const bf16_t*)lm_head, chain->t, tokens, T,
                       cache_len, max_cache_len, (bf16_t*)k_cache, (bf16_t*)v_cache, layer_stride_elems, B, H, nH,
                       nKV, D, F, V, Lmax, rms_eps, rope_base, next_tok, hidden, hidden_dt == MEDUSA_BF16, ws,
                       (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// the decoder layer's building blocks
// ---------------------------------------------------------------------------
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

size_t medusa_gemm_skinny_workspace_size(int R, int K, int ncols) {
    if (R < 1 || R > MEDUSA_MAX_TREE_NODES || K < 64 || K % 64 != 0 || ncols < 1) return 0;
    return skinny_gemm_workspace_bytes(R, K, ncols);
}

medusa_status medusa_gemm_skinny(const void* n, const void* w, int R, int K, int ncols, float* out, void* ws,
                                 size_t ws_bytes, void* stream) {
    return guarded("medusa_gemm_skinny", [&] {
        REQUIRE(n && w && out, "null pointer argument");
        REQUIRE(R >= 1 && K >= 1 && ncols >= 1, "sizes must be positive (R=%d K=%d ncols=%d)", R, K, ncols);
        SUPPORT(R <= MEDUSA_MAX_TREE_NODES, "R=%d exceeds %d", R, MEDUSA_MAX_TREE_NODES);
        SUPPORT(K % 64 == 0, "K=%d must be a multiple of 64", K);
        REQUIRE(aligned16(n) && aligned16(w) && aligned16(out), "n, w and out must be 16-byte aligned");
        const size_t need = skinny_gemm_workspace_bytes(R, K, ncols);
        REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), "workspace too small: %zu < %zu", ws_bytes, need);
        REQUIRE(need == 0 || aligned16(ws), "workspace must be 16-byte aligned");
        launch_skinny_gemm((const bf16_t*)n, (const bf16_t*)w, R, K, ncols, out, ws, (hipStream_t)stream);
    });
}

medusa_status medusa_embed(const int32_t* tok, const void* embedding, int R, int H, int V, float* x, void* stream) {
    return guarded("medusa_embed", [&] {
        REQUIRE(tok && embedding && x, "null pointer argument");
        REQUIRE(R >= 1 && H >= 1 && V >= 1, "sizes must be positive (R=%d H=%d V=%d)", R, H, V);
        SUPPORT(H % 8 == 0, "H=%d must be a multiple of 8", H);
        REQUIRE(aligned16(embedding) && aligned16(x), "embedding and x must be 16-byte aligned");
        launch_embed(tok, (const bf16_t*)embedding, R, H, V, x, (hipStream_t)stream);
    });
}

medusa_status medusa_rmsnorm(const float* x, int R, int H, float eps, void* n, void* stream) {
    return guarded("medusa_rmsnorm", [&] {
        REQUIRE(x && n, "null pointer argument");
        REQUIRE(R >= 1 && H >= 1, "sizes must be positive (R=%d H=%d)", R, H);
        REQUIRE(eps >= 0.f, "eps must be >= 0");
        SUPPORT(H % 4 == 0, "H=%d must be a multiple of 4", H);
        REQUIRE(aligned16(x) && ((uintptr_t)n & 7) == 0, "x must be 16-byte and n 8-byte aligned");
        launch_rmsnorm_f32_bf16(x, R, H, eps, (bf16_t*)n, (hipStream_t)stream);
    });
}

size_t medusa_rope_workspace_size(int R, int D) {
    if (R < 1 || D < 2 || D % 2 != 0 || D > 128) return 0;
    return rope_workspace_bytes(R, D);
}

medusa_status medusa_rope(const float* qkv, const int32_t* pos, int R, int nH, int nKV, int D, float rope_base,
                          void* q, void* k, void* v, void* ws, size_t ws_bytes, void* stream) {
    return guarded("medusa_rope", [&] {
        REQUIRE(qkv && pos && q && k && v && ws, "null pointer argument");
        REQUIRE(R >= 1 && nH >= 1 && nKV >= 1 && D >= 2, "sizes must be positive (R=%d nH=%d nKV=%d D=%d)", R, nH,
                nKV, D);
        SUPPORT(D % 2 == 0 && D <= 128, "D=%d must be even and at most 128", D);
        SUPPORT(R <= 65535 && nH + 2 * nKV <= 65535, "R=%d or nH + 2 nKV too large", R);
        REQUIRE(rope_base > 1.f, "rope_base must exceed 1");
        REQUIRE(ws_bytes >= rope_workspace_bytes(R, D), "workspace too small");
        REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
        launch_rope(qkv, pos, R, nH, nKV, D, rope_base, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v, ws, (hipStream_t)stream);
    });
}

medusa_status medusa_swiglu(const float* gate_up, int R, int F, void* a, void* stream) {
    return guarded("medusa_swiglu", [&] {
        REQUIRE(gate_up && a, "null pointer argument");
        REQUIRE(R >= 1 && F >= 1, "sizes must be positive (R=%d F=%d)", R, F);
        SUPPORT(F % 16 == 0, "F=%d must be a multiple of 16", F);
        SUPPORT(R <= 65535, "R=%d exceeds 65535", R);
        launch_swiglu(gate_up, R, F, (bf16_t*)a, (hipStream_t)stream);
    });
}

// ---------------------------------------------------------------------------
// profiler
// ---------------------------------------------------------------------------
medusa_status medusa_profiler_enable(int on) {
    g_prof_on = on != 0;
    return MEDUSA_OK;
}

medusa_status medusa_profiler_reset(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : g_prof_pending) {
        (void)hipEventSynchronize(r.b);  // discarded either way; only makes the events reusable
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_pending.clear();
    g_prof_stats.clear();
    g_prof_snapshot.clear();
    g_prof_err = hipSuccess;
    return MEDUSA_OK;
}

int medusa_profiler_collect(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : g_prof_pending) {
        float ms = 0.f;
        hipError_t err = hipEventSynchronize(r.b);
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.a, r.b);
        if (err == hipSuccess) {
            ProfStat& st = g_prof_stats[r.name];
            st.calls += 1;
            st.ms += ms;
        } else {
            prof_fail(err);
        }
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_pending.clear();
    g_prof_snapshot.assign(g_prof_stats.begin(), g_prof_stats.end());
    if (g_prof_err != hipSuccess) {
        set_error(std::string("medusa_profiler_collect: timing events failed: ") + hipGetErrorString(g_prof_err));
        g_prof_err = hipSuccess;
        return -1;
    }
    return (int)g_prof_snapshot.size();
}

medusa_status medusa_profiler_stat(int i, char* name, size_t name_len, int64_t* calls, double* total_ms) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (i < 0 || i >= (int)g_prof_snapshot.size()) {
        set_error("profiler index out of range");
        return MEDUSA_EINVAL;
    }
    if (name && name_len) {
        strncpy(name, g_prof_snapshot[i].first.c_str(), name_len - 1);
        name[name_len - 1] = 0;
    }
    if (calls) *calls = g_prof_snapshot[i].second.calls;
    if (total_ms) *total_ms = g_prof_snapshot[i].second.ms;
    return MEDUSA_OK;
}

}  // extern "C"
