/*
 * medusa.h -- C ABI of one Medusa decoding step on an AMD Instinct MI355X
 * (gfx950).
 *
 * The calls follow the method as the "Medusa Heads" glossary page
 * (Ultralytics; Arabic and Portuguese editions carry the same text) states it:
 *   - section on how the heads predict later tokens: K heads read the same last
 *     hidden state h; head k is one feed-forward layer with SiLU and a residual
 *     connection, then a projection to the vocabulary
 *     (medusa_resid_silu, medusa_vocab_topk, medusa_heads_forward);
 *   - section on tree attention and acceptance: the heads' top guesses form a
 *     Cartesian candidate tree (medusa_tree_create, medusa_build_tree); every
 *     candidate is verified in one pass in which each token sees only its tree
 *     ancestors (tree_attention_verify); under greedy decoding a candidate is
 *     accepted when it equals the base model's top choice
 *     (medusa_base_greedy), the longest accepted branch is kept and its state
 *     is handed to the next round (medusa_accept, which also compacts the
 *     accepted branch's keys/values in the cache).
 * The accepted-tokens-plus-one accounting (a correction or bonus token every
 * round) follows the speculative-decoding e-book "Giai ma dau co: doan truoc
 * roi kiem mot luot", section on why a round always yields k + 1 tokens.
 *
 * Conventions
 *   - Every pointer is a device pointer unless marked "host".
 *   - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream) and returns a medusa_status.  All
 *     arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and medusa_last_error() describes it.
 *   - The caller owns every buffer.  Scratch memory comes from a caller
 *     workspace `ws` of at least the size the matching *_workspace_size()
 *     returns; the compute calls never allocate.  The workspace must not be
 *     shared by calls that may run concurrently.
 *   - dtype MEDUSA_F32: float32 storage.  MEDUSA_BF16: bfloat16 storage
 *     (uint16 bit patterns).  Accumulation is always float32.
 *   - Row-major layouts; weights use the [out][in] layout of a linear layer.
 *   - Top-k and argmax order: larger value first, lower index first among
 *     equal values; decisions are taken on the float32 accumulators.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MEDUSA_OK = 0,
    MEDUSA_EINVAL = 1,        /* null pointer, bad shape, bad tree spec, sizes too small */
    MEDUSA_EUNSUPPORTED = 2,  /* valid request outside the implemented envelope */
    MEDUSA_EHIP = 3           /* a HIP runtime call or kernel launch failed */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

/* Layout of a weight matrix [rows][cols]: row-major, or packed by
 * medusa_pack_rows into the fragment order of the MFMA products. */
typedef enum { MEDUSA_ROW_MAJOR = 0, MEDUSA_PACKED = 1 } medusa_layout;

/* Opaque candidate-tree topology (library-owned; device copy inside). */
typedef struct medusa_tree medusa_tree;

/* Thread-local description of the last error on this thread ("" if none). */
const char* medusa_last_error(void);
const char* medusa_version(void);

/* Implementation limits. */
#define MEDUSA_MAX_TREE_NODES 256
#define MEDUSA_MAX_TOPK 16
#define MEDUSA_MAX_DEPTH 16
#define MEDUSA_MAX_BATCH 8

/* ---------------------------------------------------------------------------
 * Step a1 -- residual-SiLU block of every head (heads page, section on how the
 * heads predict later tokens):  z[b][k][:] = h[b] + SiLU(W1_k h[b] + b1_k).
 *   h  [B][H] (dt), b1 [K][H] (dt)
 *   w1 head k's square matrix ([out][in]), laid out as w1_layout says:
 *      MEDUSA_ROW_MAJOR: [K][H][H] (dt), streamed by a vector-ALU GEMV;
 *      MEDUSA_PACKED (bf16 only, H a multiple of 64): K packed H x H
 *      matrices back to back (head k at byte offset k * medusa_packed_size(H,
 *      H)), streamed through MFMA with the bf16 h rows as exact operands;
 *      the faster choice from B = 4 on.
 *   z  [B][K][H] float32 (output)
 * Limits: 1 <= B <= 8, H % 8 == 0, H <= 8192.
 * ------------------------------------------------------------------------- */
medusa_status medusa_resid_silu(const void* h, const void* w1, medusa_layout w1_layout, const void* b1,
                                int B, int H, int K, medusa_dtype dt,
                                float* z, void* stream);

/* ---------------------------------------------------------------------------
 * Step a2 -- vocabulary projection and per-head top-k (heads page: projection
 * to the vocabulary; tree section: the heads' top guesses).
 *   z        [B][K][H] float32: head k's input for sequence b
 *   w2       head k's projection (no bias), laid out as w2_layout says:
 *            MEDUSA_ROW_MAJOR: [K][V][H] (dt), streamed by a vector-ALU GEMV
 *            (every weight byte meets B <= 8 inputs);
 *            MEDUSA_PACKED (bf16 only, H a multiple of 128): K packed
 *            matrices of V rows x H columns back to back, each
 *            medusa_packed_size(V, H) bytes (medusa_pack_rows of head k at
 *            byte offset k * medusa_packed_size(V, H)), streamed through
 *            MFMA with z entering as a bf16 head plus a bf16 remainder (17
 *            significant bits); the faster choice from B = 4 on.
 *   logits   [B][K][V] float32, optional (NULL: not written)
 *   topk_idx [B][K][topk] int32, topk_val [B][K][topk] float32 (outputs);
 *            ties keep the lower index.
 * Limits: 1 <= topk <= min(16, V), 1 <= B <= 8, H % 8 == 0, H <= 8192.
 * ------------------------------------------------------------------------- */
size_t medusa_vocab_topk_workspace_size(int B, int H, int V, int K, int topk, medusa_dtype dt,
                                        medusa_layout w2_layout);
medusa_status medusa_vocab_topk(const float* z, const void* w2, medusa_layout w2_layout,
                                int B, int H, int V, int K, int topk, medusa_dtype dt,
                                float* logits, int32_t* topk_idx, float* topk_val,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Steps a1 + a2 in one call: the K Medusa heads on the last hidden state.
 *   w1 == NULL and b1 == NULL: z_k = h for every head (plain projection, e.g.
 *   the base model's lm_head with K = 1).  `layout` applies to w1 and w2
 *   alike.  Workspace holds z and the top-k partials.  Other arguments as
 *   above.
 * ------------------------------------------------------------------------- */
size_t medusa_heads_workspace_size(int B, int H, int V, int K, int topk, medusa_dtype dt,
                                   medusa_layout w2_layout);
medusa_status medusa_heads_forward(const void* h, const void* w1, const void* b1, const void* w2,
                                   medusa_layout layout,
                                   int B, int H, int V, int K, int topk, medusa_dtype dt,
                                   float* logits, int32_t* topk_idx, float* topk_val,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_heads_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments without a workspace.  z
 * and the top-k partials live in a library-owned device array of
 * MEDUSA_STATIC_SCRATCH_BYTES on each GPU the library runs on (held until the
 * process ends).  Nothing in it needs to start at zero: every call writes what
 * it reads.  Calls that overlap on one GPU (several streams or threads) race
 * on the array; serialise them.  The first call on each device looks up the
 * array's device address (make it outside a graph capture).  Returns
 * MEDUSA_EUNSUPPORTED, enqueuing nothing, when
 * medusa_heads_workspace_size(...) exceeds MEDUSA_STATIC_SCRATCH_BYTES
 * (8 sequences x 5 heads x hidden 4096 x vocabulary 128256 need about 2.0
 * MB).  Allocates nothing: no hipMalloc, no allocating library call.
 * ------------------------------------------------------------------------- */
#define MEDUSA_STATIC_SCRATCH_BYTES (8u << 20)
medusa_status medusa_heads_forward_static(const void* h, const void* w1, const void* b1, const void* w2,
                                          medusa_layout layout,
                                          int B, int H, int V, int K, int topk, medusa_dtype dt,
                                          float* logits, int32_t* topk_idx, float* topk_val, void* stream);

/* ---------------------------------------------------------------------------
 * Step a3 -- candidate tree (tree section: Cartesian product of the heads'
 * top guesses, sharing prefixes).
 *
 * medusa_tree_create: host arrays parent[N], rank[N] in breadth-first order.
 *   Node 0 is the root (parent[0] = -1, the token the base model already
 *   chose); node i > 0 has 0 <= parent[i] < i and carries the rank[i]-th token
 *   (0 <= rank[i] < topk) of head depth(i) (1 <= depth(i) <= K).  Siblings
 *   must have distinct ranks.  1 <= N <= 256.  Uploads the spec and the
 *   ancestor bitmask to the current device (allocates; not for hot loops).
 *   Candidate trees are at most 16 deep (medusa_build_tree, medusa_accept,
 *   medusa_typical_accept, medusa_advance and medusa_plant_greedy refuse
 *   deeper ones with MEDUSA_EUNSUPPORTED; medusa_build_tree also needs depth x
 *   (largest rank + 1) <= 256); a deeper chain (parent[i] = i - 1, rank 0,
 *   K = N - 1) serves the verify pass and medusa_prefill.
 * medusa_build_tree: node_tok[b][i] = root_tok[b] for i = 0, else
 *   topk_idx[b][depth(i)-1][rank[i]];  node_pos[b][i] = cache_len[b] + depth(i);
 *   anc_mask (optional) [N][W] uint64, W = ceil(N/64): bit j of word j/64 of
 *   row i is set iff node j is node i or an ancestor of i.
 * ------------------------------------------------------------------------- */
medusa_status medusa_tree_create(const int32_t* parent, const int32_t* rank, int N, int K, int topk,
                                 medusa_tree** out);
void medusa_tree_destroy(medusa_tree* tree);

/* ---------------------------------------------------------------------------
 * Device-side status of a tree handle.  Sizes that live in device memory
 * (cache_len[]) cannot be validated on the host before launch; when a kernel
 * meets an invalid one it keeps every access in bounds, does what the call
 * documents for that case, and sets a bit of the tree's status word (atomic
 * OR; every call that takes the tree shares the word):
 *   MEDUSA_STATUS_CACHE_LEN_CLAMPED: tree_attention_verify (or the decoder
 *     pass) read a cache_len[b] outside [0, max_cache_len] and used the
 *     clamped value;
 *   MEDUSA_STATUS_CACHE_OVERFLOW: medusa_accept / medusa_typical_accept were
 *     given caches and a cache_len[b] < 0 or cache_len[b] + N > Lmax: that
 *     sequence's caches were not compacted and new_cache_len[b] = cache_len[b].
 * medusa_tree_status waits for `stream`, copies the word into *flags (host)
 * and, if clear != 0, resets it to 0.  Work of the tree on other streams must
 * have finished (the caller synchronises them).  Not for use inside a graph
 * capture.  Created trees start at 0.
 * ------------------------------------------------------------------------- */
#define MEDUSA_STATUS_CACHE_LEN_CLAMPED 1
#define MEDUSA_STATUS_CACHE_OVERFLOW 2
medusa_status medusa_tree_status(const medusa_tree* tree, int32_t* flags, int clear, void* stream);
int medusa_tree_num_nodes(const medusa_tree* tree);
int medusa_tree_max_depth(const medusa_tree* tree);
/* host copy of the ancestor bitmask, [N][ceil(N/64)] */
medusa_status medusa_tree_mask_host(const medusa_tree* tree, uint64_t* mask, size_t words);

medusa_status medusa_build_tree(const medusa_tree* tree, const int32_t* topk_idx,
                                const int32_t* root_tok, const int32_t* cache_len, int B, int K, int topk,
                                int32_t* node_tok, int32_t* node_pos, uint64_t* anc_mask, void* stream);

/* ---------------------------------------------------------------------------
 * Steps a1 + a2 + a3 in one call (heads page; tree section: the tree is the
 * Cartesian product of the heads' top guesses): medusa_heads_forward, then
 * medusa_build_tree on the top-k it chose, without the tree build's own
 * launch: the merge workgroup of head k (one per sequence and head) also
 * writes the tree nodes at depth k + 1, whose tokens are that head's
 * choices, and head 0's the root.  Arguments as medusa_heads_forward (the
 * same workspace size) and as medusa_build_tree (the tree, root_tok,
 * cache_len, node_tok, node_pos and the optional anc_mask); every output
 * equals what those two calls write.  Errors: those of either call; on
 * error nothing is enqueued.
 * ------------------------------------------------------------------------- */
medusa_status medusa_heads_forward_tree(const void* h, const void* w1, const void* b1, const void* w2,
                                        medusa_layout layout,
                                        int B, int H, int V, int K, int topk, medusa_dtype dt,
                                        float* logits, int32_t* topk_idx, float* topk_val,
                                        const medusa_tree* tree, const int32_t* root_tok,
                                        const int32_t* cache_len, int32_t* node_tok, int32_t* node_pos,
                                        uint64_t* anc_mask, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Step a4 -- tree-masked attention (tree section: all candidates appended in
 * one pass; each token sees only its ancestors -- and itself).
 *   q [B][N][nH][D], k_tree / v_tree [B][N][nKV][D] (dt)
 *   k_cache / v_cache [B][nKV][Lmax][D] (dt): slots < cache_len[b] are the
 *     prefix; this call also writes the tree keys/values to slots
 *     cache_len[b] .. cache_len[b]+N-1.
 *   out [B][N][nH][D] (dt): o = sum_j softmax_j(scale * q.k_j) v_j over the
 *     prefix and the node's ancestors-or-self; query head h reads KV head
 *     h / (nH / nKV).
 *   max_cache_len (host): an upper bound of cache_len[] (sizes the launch);
 *     a cache_len[b] outside [0, max_cache_len] is clamped into it and
 *     MEDUSA_STATUS_CACHE_LEN_CLAMPED is set in the tree's status word.
 *   Cache slots at and past cache_len[b] are never part of the result,
 *     whatever they hold (NaN included).
 * Limits: D in {64, 128}; nH % nKV == 0; max_cache_len + N <= Lmax.
 * ------------------------------------------------------------------------- */
size_t tree_attention_workspace_size(const medusa_tree* tree, int B, int nH, int D,
                                     int max_cache_len, medusa_dtype dt);
medusa_status tree_attention_verify(const void* q, const void* k_tree, const void* v_tree,
                                    void* k_cache, void* v_cache, const int32_t* cache_len,
                                    int max_cache_len, const medusa_tree* tree,
                                    int B, int nH, int nKV, int D, int Lmax, float scale,
                                    medusa_dtype dt, void* out, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Weight packing for the MFMA products (base greedy's lm_head, the decoder's
 * projections).  Not a step of the method: a layout, applied once when the
 * weights are loaded.  A packed matrix of `rows` rows and `cols` columns
 * (bf16), NRB = ceil(rows / 16) blocks of 16 rows, stores row r, column k at
 * element
 *   ((k / 32) * NRB + r / 16) * 512 + ((k % 32) / 8 * 16 + r % 16) * 8 + k % 8
 * (every 16 x 32 tile is one contiguous 1 KB fragment; the fragments of one
 * 32-wide k-step are contiguous over all row blocks) and occupies
 * medusa_packed_size(rows, cols) bytes (rows rounded up to 16).
 *   medusa_pack_rows: src [rows][cols] row-major bf16 (device) -> rows of dst,
 *   a packed matrix of dst_rows rows.  interleave == 1: source row i goes to
 *   packed row dst_row0 + i, so several matrices stack into one by packing
 *   each at its row offset (the decoder's q|k|v); the call that ends at
 *   dst_rows also zeroes the padding rows.  interleave == n > 1: source row i
 *   goes to packed row dst_row0 + (i / 16) * 16 n + i % 16, so n matrices
 *   packed with dst_row0 = 0, 16, .. 16 (n - 1) alternate in blocks of 16
 *   rows (the decoder's gate|up; rows and dst_row0 multiples of 16).
 *   Asynchronous on `stream`; src must stay valid until the copy has run.
 * Limits: cols % 32 == 0.  medusa_packed_size returns 0 for invalid sizes.
 * ------------------------------------------------------------------------- */
size_t medusa_packed_size(int rows, int cols);
medusa_status medusa_pack_rows(const void* src, int rows, int cols, void* dst, int dst_row0, int dst_rows,
                               int interleave, void* stream);

/* ---------------------------------------------------------------------------
 * Step a5 -- the base model's greedy choice after every tree node (tree
 * section: greedy acceptance compares with the model's top choice).
 *   x [R][H] (dt): one row per node; n = x * rsqrt(mean(x^2) + eps) (unit
 *   weight); greedy[r] = argmax_v (lm_head[v] . n_r), lower index first among
 *   equal values; logits [R][V] = lm_head . n (float32, optional).
 *   lm_head [V][H] (dt) in lm_layout: MEDUSA_PACKED (bf16 only) runs the MFMA
 *   product on the bf16 rows x and applies the positive factor
 *   rsqrt(mean(x^2) + eps) to the float32 scores (it does not move the
 *   argmax); MEDUSA_ROW_MAJOR (any dt) forms n in float32 for the vector GEMV.
 *   greedy [R] int32.
 * Limits: H % 8 == 0, H <= 8192, R >= 1; packed: H % 64 == 0.
 * ------------------------------------------------------------------------- */
size_t medusa_base_greedy_workspace_size(int R, int H, int V, medusa_dtype dt, medusa_layout lm_layout);
medusa_status medusa_base_greedy(const void* x, const void* lm_head, medusa_layout lm_layout, int R, int H, int V,
                                 float eps, medusa_dtype dt, int32_t* greedy, float* logits,
                                 void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Steps a6 + a7 -- longest accepted branch and its KV hand-off (tree section:
 * keep the longest branch the model accepts; its final state feeds the heads
 * next round; e-book: a round yields the accepted tokens plus one).
 *   node_tok, greedy [B][N] int32 (greedy[b][i]: base choice after node i)
 *   accept_len [B]: L = depth of the deepest node whose whole chain matches
 *   accept_nodes [B][Dmax+1]: node ids of the accepted path (root first),
 *     -1 after position L;  Dmax = the tree's maximum depth
 *   out_tokens [B][Dmax+1]: the L accepted tokens then greedy[path[L]]
 *     (the correction/bonus token, next round's root), -1 after position L
 *   cache_len [B] (in) / new_cache_len [B] (out) = cache_len + L + 1
 *   k_cache / v_cache (optional, both or neither): n_layers caches, layer l
 *     at base + l * layer_stride_elems, each [B][nKV][Lmax][D] (dt); for
 *     d = 1..L slot cache_len+d receives slot cache_len+path[d] (all sources
 *     read before any write).  A sequence whose cache_len[b] is negative or
 *     whose tree slots would pass Lmax (cache_len[b] + N > Lmax) is not
 *     compacted, gets new_cache_len[b] = cache_len[b], and sets
 *     MEDUSA_STATUS_CACHE_OVERFLOW in the tree's status word.
 * ------------------------------------------------------------------------- */
medusa_status medusa_accept(const medusa_tree* tree, const int32_t* node_tok, const int32_t* greedy,
                            int B, int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                            const int32_t* cache_len, int32_t* new_cache_len,
                            void* k_cache, void* v_cache, int n_layers, int64_t layer_stride_elems,
                            int nKV, int D, int Lmax, medusa_dtype dt, void* stream);

/* ---------------------------------------------------------------------------
 * Typical acceptance, the sampling-mode rule in place of steps a5 + a6 (tree
 * section: under sampling a candidate is kept when its probability under the
 * base model exceeds a threshold tied to the entropy of the distribution,
 * accepting more tokens without matching the distribution exactly).  The
 * page names the rule, not its form; the form taken:
 *   p(. | node) = softmax(logits[b][node] / temperature), H its entropy (nats);
 *   node i (depth >= 1) passes when p(node_tok[b][i] | parent(i)) >
 *   min(epsilon, delta * exp(-H(parent(i)))), and is accepted when it and
 *   every ancestor pass; L and the path as in medusa_accept (deepest accepted
 *   node, lowest index among equally deep ones);
 *   out_tokens[b][L] (the round's extra token) is drawn from p(. | path[L])
 *   by inverse transform sampling with uniform[b] in [0, 1): the smallest
 *   token index whose cumulative probability (index order) exceeds it.
 *   logits [B][N][V] float32: the base model's scores after every node
 *     (medusa_base_greedy's optional logits output);
 *   the other arguments, the outputs and the compaction as medusa_accept;
 *   workspace: medusa_typical_accept_workspace_size(tree, B) bytes.
 * Limits: V <= 262144.  Three kernels: the per-node softmax statistics,
 * acceptance with the compaction, then the draw of the extra token.
 * ------------------------------------------------------------------------- */
size_t medusa_typical_accept_workspace_size(const medusa_tree* tree, int B);
medusa_status medusa_typical_accept(const medusa_tree* tree, const int32_t* node_tok, const float* logits, int B,
                                    int V, float temperature, float epsilon, float delta, const float* uniform,
                                    int32_t* accept_len, int32_t* accept_nodes, int32_t* out_tokens,
                                    const int32_t* cache_len, int32_t* new_cache_len, void* k_cache, void* v_cache,
                                    int n_layers, int64_t layer_stride_elems, int nKV, int D, int Lmax,
                                    medusa_dtype dt, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Speculative sampling on a chain of drafts (draft-model speculative
 * decoding; the speculative-decoding e-book, section on being faster with an
 * unchanged output): draft i, drawn from q_i, is accepted with probability
 * min(1, p_i(x) / q_i(x)); the round stops at the first rejection n and draws
 * its token from max(0, p_n - q_n) normalised; if every draft passes, the
 * extra token is drawn from p_gamma.  The output is then distributed exactly
 * as p.  The random draws are inputs:
 *   p [B][gamma+1][V], q [B][gamma][V] float32 probability rows (row i: after
 *     the first i drafts); drafts [B][gamma] int32;
 *   u_accept [B][gamma]: draft i passes when u_accept * q_i(x) < p_i(x);
 *   u_resample [B][gamma+1] in [0, 1): the draw at the stopping position, by
 *     inverse transform sampling (the smallest token index whose cumulative
 *     weight, index order, exceeds u times the total);
 *   n_accepted [B] (out); out_tokens [B][gamma+1] (out): the n accepted
 *     drafts, the drawn token, then -1.
 * Limits: gamma <= 64, V <= 262144.  One kernel; no workspace.
 * ------------------------------------------------------------------------- */
medusa_status medusa_speculative_sample(const float* p, const float* q, const int32_t* drafts, const float* u_accept,
                                        const float* u_resample, int B, int gamma, int V, int32_t* n_accepted,
                                        int32_t* out_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * The loop around the step -- hand-off of the accepted branch to the next
 * round (tree section: the final state of the longest accepted branch feeds
 * the heads next round; e-book, section on why a round always yields k + 1
 * tokens: the extra token the base model chose after the last accepted one).
 * With L = accept_len[b] and the node path accept_nodes[b] from medusa_accept
 * (Dmax = the tree's maximum depth):
 *   root_tok [B] (out) = out_tokens[b][L]: the bonus token, next tree's root;
 *   h [B][H] (out, dt; bf16 rounds to nearest even) = hidden[b][accept_nodes[b][L]]:
 *     the final normalised state at the deepest accepted node, which the
 *     heads read next round (hidden [B][N][H] float32: medusa_decoder_verify's
 *     optional output);
 *   tokens [B][cap], n_tokens [B] (optional, both or neither): the round's
 *     L + 1 tokens out_tokens[b][0..L] are written at tokens[b][n_tokens[b] ..]
 *     (indices >= cap are dropped) and n_tokens[b] grows by L + 1;
 *   new_cache_len, cache_len [B] (optional, both or neither): cache_len[b] =
 *     new_cache_len[b], so the next round reads its prefix length from the
 *     buffer this round's medusa_accept read (the two may not alias there).
 * A sequence whose L is outside [0, Dmax] or whose node is outside [0, N) is
 * left unchanged.  One kernel; no workspace.
 * ------------------------------------------------------------------------- */
medusa_status medusa_advance(const medusa_tree* tree, const int32_t* accept_len, const int32_t* accept_nodes,
                             const int32_t* out_tokens, const float* hidden, int B, int H, medusa_dtype dt,
                             int32_t* root_tok, void* h, int32_t* tokens, int32_t* n_tokens, int cap,
                             const int32_t* new_cache_len, int32_t* cache_len, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid, not a step of the method.  With random weights the base
 * model's choices never match the heads' guesses, so every round accepts
 * nothing.  medusa_plant_greedy overwrites greedy [B][N] (the base model's
 * choice after every node, as medusa_base_greedy or medusa_decoder_verify
 * wrote it) with a planted continuation: for sequence b and depth d, the
 * token after every depth-d node is head (d + 1)'s rank-r guess
 * topk_idx[b][d][r] with probability a (1 - a)^r (r < topk), a =
 * alpha[min(d, n_alpha - 1)] (host array: one alpha, or one per depth), else a
 * token outside that head's top-k (at depth K: any token), drawn with the
 * counter hash of (seed, b, cache_len[b], d) -- a new prefix length draws a new
 * continuation, so a captured loop draws anew every round.  A round then
 * accepts the ranks drawn as far as the tree holds them: 1 + sum over nodes of
 * the product of alpha (1 - alpha)^rank along their path tokens per round on
 * average (the rank prior the sparse tree was chosen under, with alpha =
 * 0.8).  One kernel; no workspace.  Limits: tree depth <= 16, K >= depth.
 * ------------------------------------------------------------------------- */
medusa_status medusa_plant_greedy(const medusa_tree* tree, const int32_t* topk_idx, const int32_t* cache_len, int B,
                                  int K, int topk, int V, const float* alpha, int n_alpha, uint64_t seed,
                                  int32_t* greedy, void* stream);

/* ---------------------------------------------------------------------------
 * Choosing the candidate tree from measured acceptance (tree section: the
 * sparse tree is built from the combinations of head guesses most likely to
 * be accepted).
 *
 * medusa_accept_stats adds what one round of medusa_accept revealed to
 * counts [K][topk + 1] (int32, device, accumulated with atomic adds): for
 * sequence b with L = accept_len[b], the base model's choice at depth
 * d <= L was the rank-rank[path[d]] candidate (counts[d - 1][rank]++), and
 * at depth L + 1 <= K it was the extra token out_tokens[b][L], found at rank
 * r of head L + 1's top-k topk_idx[b][L] (counts[L][r]++) or among none of
 * them (counts[L][topk]++); deeper depths are not observed.  One kernel.
 *
 * medusa_tree_select (host only, no device work): the N-node tree with the
 * largest expected tokens per round, 1 + sum over nodes of the product along
 * the node's path of acc[d][r] -- the probability that head d + 1's rank-r
 * guess is the base model's choice given the path so far (host [K][topk]
 * doubles) -- chosen best-first: larger product, then shallower, then the
 * lexicographically smaller rank tuple.  Writes parent[N], rank[N] (host) in
 * breadth-first order, ready for medusa_tree_create.
 * ------------------------------------------------------------------------- */
medusa_status medusa_accept_stats(const medusa_tree* tree, const int32_t* accept_len, const int32_t* accept_nodes,
                                  const int32_t* out_tokens, const int32_t* topk_idx, int B, int K, int topk,
                                  int32_t* counts, void* stream);
medusa_status medusa_tree_select(const double* acc, int K, int topk, int N, int32_t* parent, int32_t* rank);

/* ---------------------------------------------------------------------------
 * Step a8 -- the tree-verify forward pass through a Llama-shaped decoder
 * ("Medusa Heads" glossary, section on tree attention and acceptance: every
 * candidate is appended to the input of one forward pass of the base model,
 * each token attending only to its tree ancestors).  The decoder internals are
 * not on the pages; this is the standard pre-norm Llama layer:
 *   n = RMSNorm(x); q, k = RoPE(W_q n), RoPE(W_k n) at position node_pos;
 *   v = W_v n; o = tree attention of q over the layer's cache prefix plus the
 *   node's ancestors-or-self (the tree keys/values are written to cache slots
 *   cache_len .. cache_len + N - 1 of the layer, as tree_attention_verify
 *   does); x += W_o o; n' = RMSNorm(x); x += W_down (SiLU(W_gate n') *
 *   (W_up n')); after the last layer greedy = argmax_v lm_head[v] .
 *   RMSNorm(x), lower index first among equal values.
 *   RMSNorm: unit weight, x * rsqrt(mean(x^2) + rms_eps).  RoPE rotates the
 *   pair (i, i + D/2) of every head by node_pos * rope_base^(-2i/D).
 *   x starts as embedding[node_tok] and is kept in float32; the normalised
 *   rows, q/k/v, the attention output and the SwiGLU product are rounded to
 *   bf16 (nearest even) before they enter the next product.
 * Arguments (bf16 only; device pointers unless noted):
 *   layers (host array [n_layers]): each layer's weights, [out][in] matrices
 *     packed by medusa_pack_rows: wqkv = W_q [nH*D][H], W_k and W_v
 *     [nKV*D][H] stacked in that order ((nH + 2 nKV) D rows); wo [H][nH*D];
 *     w_gate_up = W_gate and W_up [F][H] interleaved in blocks of 16 rows
 *     (interleave 2: gate rows 16j.. at packed block 2j, up rows at 2j + 1);
 *     w_down [H][F];
 *   embedding [V][H] row-major;  lm_head [V][H] packed;
 *   node_tok, node_pos [B][N] int32 (medusa_build_tree's outputs; token ids
 *     outside [0, V) read row 0 of the embedding);  cache_len [B];
 *   k_cache / v_cache: n_layers caches, layer l at base + l * layer_stride_elems,
 *     each [B][nKV][Lmax][D];
 *   greedy [B][N] int32 (output); hidden [B][N][H] float32, optional: the
 *     final normalised rows (bf16 values) that lm_head scores.
 * Limits: H == nH * D, D in {64, 128}, H and F multiples of 64,
 *   B*N <= 256, H <= 16384.
 *   The workspace must not be shared by calls that may run concurrently.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void* wqkv;
    const void* wo;
    const void* w_gate_up;
    const void* w_down;
} medusa_layer_weights;

size_t medusa_decoder_workspace_size(const medusa_tree* tree, int B, int H, int nH, int nKV, int D, int F, int V,
                                     int max_cache_len);
medusa_status medusa_decoder_verify(const medusa_layer_weights* layers, int n_layers, const void* embedding,
                                    const void* lm_head, const medusa_tree* tree, const int32_t* node_tok,
                                    const int32_t* node_pos, const int32_t* cache_len, int max_cache_len,
                                    void* k_cache, void* v_cache, int64_t layer_stride_elems, int B, int H, int nH,
                                    int nKV, int D, int F, int V, int Lmax, float rms_eps, float rope_base,
                                    int32_t* greedy, float* hidden, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill of a prompt before the first round (the state a round starts from:
 * the prompt's keys/values in every layer's cache, the base model's greedy
 * choice after the prompt -- the first root token -- and the final
 * normalised row that chose it -- the heads' first input).  The prompt goes
 * through the same decoder pass as medusa_decoder_verify, C tokens at a time
 * with `chain` a chain tree of C nodes (parent[i] = i - 1, rank 0, created
 * with K = C - 1): every token sees the cache prefix and the chunk's earlier
 * tokens, i.e. causal attention, and writes its keys/values at slot
 * cache_len[b] + its index.  The last pass is padded with copies of the last
 * token, whose keys/values land in slots past the new length that no prompt
 * token sees (they are overwritten later).
 *   tokens [B][T] int32 (ids outside [0, V) read row 0 of the embedding);
 *   cache_len [B] (in: the prefix before the prompt; out: + T);
 *   max_cache_len (host): an upper bound of cache_len[] on entry;
 *   next_tok [B] (out): greedy choice after the last prompt token;
 *   hidden [B][H] (out, hidden_dt: MEDUSA_F32 or MEDUSA_BF16, exact either way:
 *     the values are bf16): that token's final normalised row, the heads'
 *     first input;
 *   the other arguments as medusa_decoder_verify.
 * Limits: max_cache_len + ceil(T / C) * C <= Lmax; B * C <= 256; the
 * decoder's limits.  Workspace: medusa_prefill_workspace_size bytes.
 * ------------------------------------------------------------------------- */
size_t medusa_prefill_workspace_size(const medusa_tree* chain, int B, int H, int nH, int nKV, int D, int F, int V,
                                     int T, int max_cache_len);
medusa_status medusa_prefill(const medusa_layer_weights* layers, int n_layers, const void* embedding,
                             const void* lm_head, const medusa_tree* chain, const int32_t* tokens, int T,
                             int32_t* cache_len, int max_cache_len, void* k_cache, void* v_cache,
                             int64_t layer_stride_elems, int B, int H, int nH, int nKV, int D, int F, int V, int Lmax,
                             float rms_eps, float rope_base, int32_t* next_tok, void* hidden,
                             medusa_dtype hidden_dt, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The decoder layer's building blocks as calls of their own: the products,
 * norms, rotations, gating and embedding that medusa_decoder_verify chains
 * (the standard pre-norm Llama layer described above; the pages give no
 * decoder internals), run by the same kernels.  Rows are the R = B*N tree
 * tokens; the fp32 arrays are row-major and dense.  bf16 only.
 *
 * medusa_gemm_skinny: out [R][ncols] fp32 = n [R][K] (bf16) times the
 *   transposed weight W [ncols][K], W packed by medusa_pack_rows
 *   (dst_rows = ncols), fp32 accumulation.  The contraction is split over
 *   whole rounds of workgroups as in the layer; the partial sums go to the
 *   workspace (medusa_gemm_skinny_workspace_size bytes, 0 when unsplit: then
 *   ws may be NULL) and are added in split order.  1 <= R <= 256, K a
 *   multiple of 64; n, W, out and ws 16-byte aligned.
 * medusa_rmsnorm: n [R][H] bf16 = x * rsqrt(mean(x^2) + eps) per row of the
 *   fp32 x [R][H] (unit weight; bf16 rounding to nearest even).  H a
 *   multiple of 4; x 16-byte, n 8-byte aligned.
 * medusa_rope: from the fp32 product qkv [R][(nH + 2 nKV) D] (heads: nH of
 *   q, nKV of k, nKV of v, D columns each), q [R][nH][D] and k [R][nKV][D]
 *   rotated (pair (i, i + D/2) by the angle pos[r] * rope_base^(-2i/D),
 *   angles in double, applied in fp32) and v [R][nKV][D], all bf16.
 *   D even, <= 128; workspace medusa_rope_workspace_size(R, D) bytes
 *   (the (cos, sin) table), 16-byte aligned.
 * medusa_swiglu: a [R][F] bf16 = SiLU(g) * u from the fp32 product of a
 *   gate|up matrix packed with interleave 2 ([R][2F]: column blocks of 16
 *   alternate gate and up, gate column c at 32 (c / 16) + c % 16, its up
 *   column 16 later).  F a multiple of 16.
 * medusa_embed: x [R][H] fp32 = embedding [tok[r]] (bf16 [V][H], exact
 *   widening); ids outside [0, V) read row 0.  H a multiple of 8; embedding
 *   and x 16-byte aligned.
 * ------------------------------------------------------------------------- */
size_t medusa_gemm_skinny_workspace_size(int R, int K, int ncols);
medusa_status medusa_gemm_skinny(const void* n, const void* w, int R, int K, int ncols, float* out, void* ws,
                                 size_t ws_bytes, void* stream);
medusa_status medusa_rmsnorm(const float* x, int R, int H, float eps, void* n, void* stream);
size_t medusa_rope_workspace_size(int R, int D);
medusa_status medusa_rope(const float* qkv, const int32_t* pos, int R, int nH, int nKV, int D, float rope_base,
                          void* q, void* k, void* v, void* ws, size_t ws_bytes, void* stream);
medusa_status medusa_swiglu(const float* gate_up, int R, int F, void* a, void* stream);
medusa_status medusa_embed(const int32_t* tok, const void* embedding, int R, int H, int V, float* x, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid: reads `bytes` (a multiple of 16; src 16-byte aligned) once
 * with 16-byte non-temporal loads, 4 in flight per thread, n_wg workgroups of
 * 256 threads each taking a contiguous slice, and writes the XOR of what
 * each workgroup read to sink[n_wg] (uint32).  Its rate is the achievable
 * HBM read ceiling for the weight streams' access pattern (bench.py times it
 * over 1 GiB with 16,384 workgroups).
 * ------------------------------------------------------------------------- */
medusa_status medusa_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid: the rate at which one workgroup per CU pulls data through
 * its vector-memory path.  n_wg workgroups of 256 threads run `rounds`
 * rounds; in each, every thread issues window_parts 16-byte loads of the
 * shared `window` (plain loads, so the window stays in L2: 4 KB blocks read
 * consecutively from offset 0, wrapping at window_bytes, which must be a
 * multiple of window_parts x 4096) and stream_parts
 * 16-byte non-temporal loads of its workgroup's own slice of `src`
 * (workgroup g reads bytes [g, g + 1) x rounds x stream_parts x 4096, in
 * order), all in flight together, then XORs them.  (window_parts, stream_parts) is one of (8, 0)
 * (window only), (0, 8) (HBM only), (4, 2) and (8, 4) (2 : 1 mixes, the
 * wide lm_head's ratio of node-row to weight bytes).  sink[g] (uint32) =
 * the XOR of every word workgroup g loaded.  Pointers of a part that is 0
 * are not read.  Errors: EINVAL for another pair, rounds or n_wg outside
 * [1, 2^20] / [1, 2^16], misaligned or null pointers, a window size that is
 * not a whole number of rounds, or src_bytes below
 * rounds x stream_parts x 4096 x n_wg.
 * ------------------------------------------------------------------------- */
medusa_status medusa_read_mix(const void* window, size_t window_bytes, const void* src, size_t src_bytes,
                              int window_parts, int stream_parts, int rounds, uint32_t* sink, int n_wg,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid: the matrix-wave loop of the wide lm_head product on its
 * own.  n_wg workgroups of 4 waves (one per SIMD); each wave keeps 8
 * independent 32 x 32 x 16 bf16 accumulators and runs `iters` iterations of
 * 4 k-steps, each reading the 8 node fragments of the next k-step from a
 * 64 KB LDS tile (the lm_head's swizzled layout) while the current 8
 * products run, and one workgroup barrier per iteration: 32 products (1 MFLOP
 * a wave) per iteration.  random_operands = 0: every operand element is 1.0,
 * so out[g * 256 + t] = iters x 64 x 128 exactly; 1: bf16 values of random
 * sign and magnitude in [0.25, 2) (the data-dependent power of real
 * operands).  out: n_wg x 256 floats, the sum of each thread's accumulator
 * elements.  Errors: EINVAL for random_operands not 0 / 1, iters outside
 * [1, 2^20], n_wg outside [1, 2^16] or a null out.
 * ------------------------------------------------------------------------- */
medusa_status medusa_mfma_rate(int random_operands, int iters, float* out, int n_wg, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timing: while enabled, every kernel launch of the library is
 * bracketed by HIP events on its stream.  medusa_profiler_collect waits for
 * the recorded events and folds them into per-kernel totals and returns their
 * count; ..._stat reads entry i (0 <= i < count) of those totals.  If creating,
 * recording or reading a timing event failed since the last reset or collect,
 * the launches concerned are missing from the totals and collect returns -1
 * (medusa_last_error() names the HIP error); the totals stay readable.
 * ------------------------------------------------------------------------- */
medusa_status medusa_profiler_enable(int on);
medusa_status medusa_profiler_reset(void);
int medusa_profiler_collect(void);
medusa_status medusa_profiler_stat(int i, char* name, size_t name_len, int64_t* calls, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
