// Tree-masked attention (step a4): every tree node attends to the cache
// prefix plus its own ancestors-or-self.
//
// Both variants split the key space "prefix (cache_len[b] keys) followed by
// the N tree keys" into ranges; tree keys come straight from k_tree / v_tree
// and are visible to query i only where bit j of its ancestor row is set.
// Each range keeps an online-softmax state (reference m, sum l, unnormalised
// output) in base-2 exponent form, written as a partial, and
// tree_attn_merge_kernel rescales and sums the partials.  One workgroup per
// KV head also copies the tree keys/values into cache slots
// cache_len .. cache_len + N - 1.
//
// First the vector-ALU variant (float32 storage): grid (B * nH, S, query
// blocks of 16); range s covers keys [s * KPS, (s+1) * KPS) of the key space;
// split 0 / query block 0 writes the cache slots.  The bf16 MFMA variant
// follows the merge kernel.
#include <type_traits>

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
    float scale_log2, int KPS, float* __restrict__ part_o, float* __restrict__ part_ml, int* __restrict__ status) {
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
    // cache lengths outside [0, max_cache_len] are clamped (never read past
    // Lmax) and reported in the tree's status word
    const int P_in = cache_len[b];
    const int P = max(0, min(P_in, max_cache_len));
    const int total = P + N;

    // tree K/V -> cache slots P..P+N-1 (one writer per KV head)
    if (s == 0 && blockIdx.z == 0 && h % grp == 0) {
        if (tid == 0 && P != P_in && status != nullptr) atomicOr(status, STATUS_CACHE_LEN_CLAMPED);
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

// out[b][i][h][:] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s; a split with m_s = -inf saw no key of query i and adds
// nothing (its partial row is never summed, so its contents do not matter).
// One thread per 4 columns of an output row; the partials of 8 splits are
// loaded together (one memory round trip per 8 splits).
constexpr int ATT_MERGE_THREADS = 256;
constexpr int ATT_MERGE_SPLITS = 8;

template <typename T, int D>
__global__ __launch_bounds__(ATT_MERGE_THREADS) void tree_attn_merge_kernel(const float* __restrict__ part_o,
                                                                             const float* __restrict__ part_ml,
                                                                             int S, int N, int nH,
                                                                             T* __restrict__ out) {
    constexpr int TPR = D / 4;                       // threads per output row
    constexpr int RPB = ATT_MERGE_THREADS / TPR;     // rows per workgroup
    constexpr int SU = ATT_MERGE_SPLITS;
    const int bh = blockIdx.y;
    const int i = blockIdx.x * RPB + threadIdx.x / TPR;
    if (i >= N) return;
    const int c = (threadIdx.x % TPR) * 4;
    const size_t row0 = (size_t)bh * S * N + i;      // partial row of split s: row0 + s * N
    float M = -INFINITY, L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += SU) {
        float2 ml[SU];
        f32x4 o[SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const size_t r = row0 + (size_t)min(s0 + u, S - 1) * N;
            ml[u] = *(const float2*)(part_ml + r * 2);
            o[u] = *(const f32x4*)(part_o + r * D + c);
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < SU; ++u)
            if (s0 + u < S) mx = fmaxf(mx, ml[u].x);
        if (mx == -INFINITY) continue;
        const float r = exp2f(M - mx);  // 0 while nothing has been summed
        L *= r;
        acc *= r;
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            if (s0 + u < S && ml[u].x != -INFINITY) {
                const float f = exp2f(ml[u].x - mx);
                L += f * ml[u].y;
                acc += f * o[u];
            }
        }
        M = mx;
    }
    const float inv = 1.f / L;
    const size_t dst = (((size_t)(bh / nH) * N + i) * nH + (bh % nH)) * D + c;
    if constexpr (sizeof(T) == 2) {
        *(uint2*)(out + dst) = (uint2){pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    } else {
        *(f32x4*)(out + dst) = acc * inv;
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA variant.
//
// Work split: a workgroup holds the tree queries of one head (a block of QW =
// 32 QG of them) against one key range.  Ranges 0..S-2 each cover KPS
// consecutive prefix keys (cache slots); range S-1 is the N tree keys, read
// from k_tree / v_tree under the ancestor mask.  The tree range's workgroup of
// query block 0 also copies the tree keys/values into cache slots P..P+N-1.
// The last tile of a prefix range may load slots at and past P (its rows are
// clamped to the host bound max_cache_len, not to P, since the tiles are
// requested before P is read), racing with that copy; those keys' scores are
// masked and their V values zeroed (per key pair in masked tiles with one
// query block a wave; with two, the V rows in LDS once the tile has landed,
// one extra barrier on that tile alone), so whatever the slots hold (old
// data, the new tree keys, NaN) never reaches the output.
// With several query blocks per head
// the blocks of one key range get linear workgroup ids 8 apart: workgroups are
// dealt to the 8 XCDs round-robin, so the blocks land on one XCD and read the
// range's K/V through the same L2.
//
// Inside the workgroup, 8 waves = QG query groups x KG = 8 / QG key groups:
// wave w takes QBW blocks of 16 queries, 16 QBW (w % QG) .., against the
// KW = 64 / KG keys 16 (w / QG) NKB .. of every 64-key tile (NKB = KW / 16
// blocks of 16 keys), keeps its own online-softmax state, and the key groups
// are merged through LDS at the end.  Up to 64 tree nodes 4 x 2 with one
// query block per wave: a single merge step of half-size states (2 query
// groups of two blocks x 4 key groups read the tiles from LDS half as often,
// but their two merge steps measured 2 us, more than the LDS reads save while
// the loop waits on HBM anyway); up to 128 nodes 4 x 2 with two blocks; up to
// 256 QG = 8 (every wave against the whole tile, no merge): a wide tree then
// shares each K/V tile, its barrier and its loads among all its queries
// instead of re-streaming the range once per 64 queries, and each wave has
// 4x the independent products per tile.
//
// Contractions, in transposed form so that no register data moves between
// lanes:
//   S^T[key][q]  = K . Q^T  (v_mfma_f32_16x16x32_bf16; A = the wave's 16 keys
//                            x 32 dims from the LDS K tile, B = the query
//                            block's Q fragment, held in registers);
//   O^T[d][q]   += V^T . P^T (v_mfma_f32_16x16x32_bf16 over the wave's 16
//                            keys twice: each probability is split into a
//                            bf16 head and a bf16 remainder, so the product
//                            carries 17 significant bits of P; the lane's B
//                            fragment is the heads and remainders of exactly
//                            the 4 keys its S^T output holds; A = V^T of
//                            those keys, repeated, read from the row-major
//                            LDS V tile by ds_read_b64_tr_b16, which
//                            transposes 4 x 4 blocks of 16-bit values across
//                            lanes).
// Softmax in base 2 against a lazily raised reference M: a query's M (and so
// O and l) changes only when a key block's score exceeds it by more than 2^8, so
// probabilities stay <= 256 and almost every tile skips the rescale; O / l is
// the same for any reference.  The state of query q lives in the 4 lanes that
// hold its column.
//
// Pipeline: K/V tiles of 64 keys go from HBM straight into a ring of
// MF_STAGES LDS stages with global_load_lds_dwordx4 (lane l of a wave writes
// bytes 16 l .. 16 l + 15 of a 1 KB block), three tiles ahead of the one
// being computed.  Each wave waits only for its own loads of the current
// tile (an explicit vmcnt that leaves the loads of the younger requested
// tiles in flight), then one barrier per tile publishes the tile and frees
// the stage the next load overwrites.  No tile past the range is requested;
// rows of the last tile past the range are clamped to its last row (their
// scores are masked and their V values zeroed).  Within a
// stage a row's 16-byte chunks are XOR-swizzled by a function of the row, so
// the K fragment reads (16 rows, one chunk) and the transposing V reads (4
// rows, two chunks) hit distinct LDS banks.  The first tiles are requested
// before the sequence's cache length is read (clamped to the host bound
// max_cache_len, so they stay in bounds).  The 64-query variant stages its
// queries in LDS with the same loads; the wider ones load each wave's query
// fragments straight into registers right after tile 0 is requested and
// wait for both before requesting tiles 1 and 2.
// ---------------------------------------------------------------------------
constexpr int MF_TK = 64;       // keys per tile
// query groups of a workgroup and 16-query blocks per wave for an N-node
// tree: up to 64 nodes 4 groups of one block (two key groups), up to 128 4
// groups of two blocks (two key groups), up to 256 8 groups of two blocks
// (one key group)
__host__ __device__ constexpr int mf_qg(int N) { return N <= 128 ? 4 : 8; }
__host__ __device__ constexpr int mf_qbw(int N) { return N <= 64 ? 1 : 2; }
constexpr int MF_THREADS = 512;
constexpr int MF_STAGES = 4;
constexpr float MF_LAZY = 8.f;  // log2 of the largest probability before a rescale

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte global -> LDS load per lane: lane l writes LDS bytes
// lds_addr + 16 l .. + 15 (lds_addr wave-uniform).  Issued from asm, so the
// compiler does not model these loads: the explicit vmcnt waits below alone
// order them with the LDS reads, and no load the compiler does model is in
// flight while they are (the compiler would otherwise count its own waits
// without them, which only over-waits, but could not place the tile waits).
// M0 is saved and restored around the load.
__device__ __forceinline__ void mf_dma16(const void* src, const void* lds_dst) {
    const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_dst);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(a)
        : "memory");
}

// 4 bf16 values of V^T from the row-major V tile (see the lane layout above).
__device__ __forceinline__ i16x4 ds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// XOR swizzle of the 16-byte chunks of LDS row r (DC chunks per row).
template <int DC> __device__ __forceinline__ int mf_swz(int r) {
    if constexpr (DC == 16) return ((r << 1) & 14) | ((r >> 3) & 1);
    else return ((r << 1) & 6) | ((r >> 2) & 1);
}

// This wave's loads of the current tile are done (the `younger` loads
// issued after them may still be in flight) and its LDS reads of the
// previous tile too; then the workgroup barrier.  s_waitcnt immediate:
// vmcnt = younger, expcnt = 7 (no wait), lgkmcnt = 0.  The compiler fences
// keep every memory access on its side of the barrier.
template <int younger> __device__ __forceinline__ void mf_tile_barrier() {
    static_assert(younger < 16, "vmcnt field");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x70 | younger);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// This wave's LDS accesses are done (lgkmcnt = 0; loads into LDS still in
// flight are not waited for: vmcnt = 63), then the workgroup barrier.
__device__ __forceinline__ void mf_lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Every load of this wave into LDS has landed (vmcnt = 0, lgkmcnt = 15).
__device__ __forceinline__ void mf_loads_landed() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, int QG, int QBW>
__global__ __launch_bounds__(MF_THREADS) void tree_attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_tree, const bf16_t* __restrict__ v_tree,
    bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    const uint64_t* __restrict__ mask, int N, int W, int nH, int nKV, int Lmax, int max_cache_len,
    float scale_log2, int KPS, int S, int QB, int BH, float* __restrict__ part_o, float* __restrict__ part_ml,
    int* __restrict__ status) {
    constexpr int TK = MF_TK;
    constexpr int KG = 8 / QG;                   // key groups
    constexpr int KW = TK / KG;                  // keys per wave per tile
    constexpr int NKB = KW / 16;                 // 16-key blocks per wave per tile
    constexpr int QW = 16 * QBW * QG;            // queries per workgroup
    constexpr bool QLDS = QW <= 64;              // queries staged in LDS (else straight into registers)
    constexpr int DK = D / 32;                   // k-steps of S^T over the head dimension
    constexpr int DB = D / 16;                   // 16-row blocks of O^T
    constexpr int DC = D / 8;                    // 16-byte chunks per key row
    constexpr int ROWB = D * 2;                  // bytes per key row
    constexpr int TILE_B = TK * ROWB;            // bytes of one K (or V) tile
    constexpr int STAGE_B = 2 * TILE_B;          // K tile, then V tile
    constexpr int BLKS = 2 * TILE_B / 1024;      // 1 KB load blocks per stage
    constexpr int NLD = BLKS / (MF_THREADS / 64);  // loads per wave per tile
    static_assert((QG == 2 || QG == 4 || QG == 8) && (QBW == 1 || QBW == 2), "query groups");
    static_assert(NLD >= 1 && NLD * (MF_THREADS / 64) == BLKS && (BLKS / 2) % NLD == 0, "load split");
    constexpr int QBLKS = QLDS ? QW * ROWB / 1024 : 8;  // 1 KB load blocks of the query block
    constexpr int NQLD = QBLKS / (MF_THREADS / 64);     // query loads per wave
    static_assert(NQLD >= 1 && NQLD * (MF_THREADS / 64) == QBLKS, "query load split");
    // after the key loop the stages hold the states of the key groups' waves
    // for their merge: O^T fragments + (M, l) per lane, one wave per stage
    constexpr int MERGE_WAVE_F = QBW * DB * 64 * 4 + QBW * 64 * 2;
    static_assert(MERGE_WAVE_F * 4 <= STAGE_B && MF_STAGES == 4 && (KG / 2) * QG <= MF_STAGES,
                  "merge area: one wave state per stage");
    // four separate arrays, so the compiler can tell a stage being read from
    // the stages the loads in flight write to
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_B];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_B];
    __shared__ __attribute__((aligned(1024))) char lds2[STAGE_B];
    __shared__ __attribute__((aligned(1024))) char lds3[STAGE_B];
    auto stage_ptr = [&](int u) -> char* { return u == 0 ? lds0 : u == 1 ? lds1 : u == 2 ? lds2 : lds3; };
    __shared__ __attribute__((aligned(1024))) char qlds[QLDS ? QW * ROWB : 1024];  // the block's queries (swizzled rows)

    const int Lid = blockIdx.x;
    const int qblk = (Lid >> 3) % QB;
    const int unit = (Lid & 7) + 8 * (Lid / (8 * QB));
    if (unit >= BH * S) return;
    const int bh = unit % BH, s = unit / BH;
    const int b = bh / nH, h = bh - b * nH;
    const int grp = nH / nKV;
    const int kvh = h / grp;
    const bool tree = s == S - 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int kq = wave / QG, qh = wave % QG;  // key group, query group
    const size_t cache_row0 = ((size_t)b * nKV + kvh) * Lmax;
    const size_t prow = ((size_t)bh * S + s) * N;  // partial rows of this (head, range)

    // key range: rows j = 0 .. at kbase / vbase + j * stride elements; rows
    // up to nspec - 1 are always in bounds, the first nkeys are the range
    const bf16_t* kbase;
    const bf16_t* vbase;
    int nspec, stride, k0 = 0;
    if (tree) {
        const size_t o = (size_t)b * N * nKV * D + (size_t)kvh * D;
        kbase = k_tree + o;
        vbase = v_tree + o;
        nspec = N;
        stride = nKV * D;
    } else {
        k0 = s * KPS;
        const size_t o = (cache_row0 + k0) * D;
        kbase = k_cache + o;
        vbase = v_cache + o;
        nspec = max(1, min(KPS, max_cache_len - k0));
        stride = D;
    }

    // the lane's queries (a padded query, qi >= N, computes with the last
    // query's data and is never written)
    int qidx[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) qidx[qb] = qblk * QW + qh * 16 * QBW + qb * 16 + lr;
    u32x4 qf[QBW][DK];  // QLDS: read from LDS after the first tile barrier; else loaded below
    // in the tree range, the block's ancestor rows in LDS (row r: query
    // min(qblk * QW + r, N - 1); words past W are never used: the range has W
    // tiles), loaded and waited for before any load into LDS is issued, read
    // after the first tile's barrier
    __shared__ uint64_t mlds[QW][4];
    if (tree) {
        for (int t = tid; t < QW * 4; t += MF_THREADS) {
            const int r = t >> 2, w = t & 3;
            mlds[r][w] = mask[(size_t)min(qblk * QW + r, N - 1) * W + min(w, W - 1)];
        }
        mf_loads_landed();
    }
    // the lane's row of the block's ancestor rows for its query block qb
    auto mword = [&](int qb, int i) -> uint64_t { return mlds[qh * 16 * QBW + qb * 16 + lr][i]; };
    // the query block -> LDS: row r is query min(qblk * QW + r, N - 1)
    if constexpr (QLDS) {
#pragma unroll
        for (int j = 0; j < NQLD; ++j) {
            const int unit16 = (wave * NQLD + j) * 64 + lane;
            const int r = unit16 / DC;
            const int c = (unit16 % DC) ^ mf_swz<DC>(r);
            const int qc = min(qblk * QW + r, N - 1);
            mf_dma16(q + (((size_t)b * N + qc) * nH + h) * D + c * 8, qlds + (wave * NQLD + j) * 1024);
        }
    }

    // tile loads: wave w moves 1 KB blocks w * NLD .. w * NLD + NLD - 1 of a
    // stage (the first half of the blocks is the K tile); lane l writes the
    // 16-byte unit (block, l): row lrow[j], physical chunk -> logical chunk
    const bool ld_v = wave * NLD >= BLKS / 2;
    const char* gsrc = (const char*)(ld_v ? vbase : kbase);
    int lrow[NLD];
    uint32_t lcol[NLD];  // byte offset of the logical chunk within the row
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
        const int unit16 = ((wave * NLD + j) % (BLKS / 2)) * 64 + lane;  // 16-byte unit within the tile
        lrow[j] = unit16 / DC;
        lcol[j] = (uint32_t)(((unit16 % DC) ^ mf_swz<DC>(lrow[j])) * 16);
    }
    auto issue = [&](int stage, int i) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int row = min(i * TK + lrow[j], nspec - 1);
            const char* src = gsrc + (size_t)row * stride * 2 + lcol[j];
            mf_dma16(src, stage_ptr(stage) + (wave * NLD + j) * 1024);
        }
    };
    // the first three tiles of the range as far as it can reach (the true
    // size is known only after the cache length is read)
    const int nt_spec = (nspec + TK - 1) / TK;
    issue(0, 0);
    if constexpr (!QLDS) {
        // the wave's query fragments straight into registers, right behind
        // tile 0's loads: one full wait covers both, and tile 0 is needed
        // first anyway; tiles 1 and 2 are requested after it, so the wait
        // leaves them in flight (and no compiler-placed wait for these
        // loads remains after it)
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
            const bf16_t* qrow = q + (((size_t)b * N + min(qidx[qb], N - 1)) * nH + h) * D;
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) qf[qb][ks] = *(const u32x4*)(qrow + (ks * 4 + lk) * 8);
        }
        mf_loads_landed();
    }
    if (nt_spec > 1) issue(1, 1);
    if (nt_spec > 2) issue(2, 2);

    // the sequence's prefix length decides the range's true size; a length
    // outside [0, max_cache_len] is clamped and reported in the status word
    const int P_in = cache_len[b];
    const int P = max(0, min(P_in, max_cache_len));
    if (tree && qblk == 0 && h % grp == 0 && tid == 0 && P != P_in && status != nullptr)
        atomicOr(status, STATUS_CACHE_LEN_CLAMPED);
    const int nkeys = tree ? N : min(KPS, P - k0);
    if (nkeys <= 0) {  // a range past this sequence's prefix: empty partials
        if (tid < QW) {
            const int i = qblk * QW + tid;
            if (i < N) {
                part_ml[(prow + i) * 2] = -INFINITY;
                part_ml[(prow + i) * 2 + 1] = 0.f;
            }
        }
        mf_loads_landed();  // no load into LDS outlives the workgroup
        return;
    }
    const int ntiles = (nkeys + TK - 1) / TK;
    // tile t has been requested iff t < ntiles, or t < 3 and t < nt_spec
    auto requested = [&](int t) { return t < ntiles || (t < 3 && t < nt_spec); };

    // per-lane LDS byte offsets (within a stage) of the K and V^T fragments
    // of key block 0; block kb is kb * 16 rows further (the swizzle of a row
    // depends only on its row within 16)
    const int krow = kq * KW + lr;
    uint32_t koff[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) koff[ks] = krow * ROWB + (((ks * 4 + lk) ^ mf_swz<DC>(krow)) * 16);
    const int vrow = kq * KW + lk * 4 + (lr >> 2);
    uint32_t voff[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        voff[db] = TILE_B + vrow * ROWB + (((db * 2 + ((lr & 3) >> 1)) ^ mf_swz<DC>(vrow)) * 16) + (lr & 1) * 8;

    f32x4 o[QBW][DB];
    float Mq[QBW], l[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        Mq[qb] = -3.402823466e38f;  // reference (scaled, base 2); finite so that M - M' never is inf - inf
        l[qb] = 0.f;                // this lane's share of the query's sum
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    // Keys kb * 16 .. kb * 16 + 31 of the wave's share of tile i (stage st):
    // S^T of each 16-key block (the lane holds keys 4 lk .. 4 lk + 3 of both
    // blocks), the mask, the reference, then O^T += V^T . P^T with the lane's
    // 8 keys of the pair as one 32-deep contraction, once over the
    // probabilities' bf16 heads and once over their bf16 remainders (17
    // significant bits together); A = those 8 keys' V^T values, 4 from each
    // block's transposing read, so no register is copied to build it.
    auto key_pair = [&](auto masked_tag, const char* st, int i, int kb) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        static_assert(NKB % 2 == 0, "16-key blocks are taken in pairs");
        f32x4 sc[QBW][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 ka[DK];
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) ka[ks] = *(const u32x4*)(st + koff[ks] + (kb + h) * 16 * ROWB);
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb) {
                f32x4 a = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK; ++ks)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[ks]),
                                                                __builtin_bit_cast(bf16x8, qf[qb][ks]), a, 0, 0, 0);
                sc[qb][h] = a;
            }
        }
        const int kk0 = kq * KW + kb * 16 + lk * 4;  // the lane's first key of block kb (block kb + 1: 16 on)
        u32x4 ph[QBW], pr[QBW];  // the probabilities' bf16 heads and remainders
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
            if constexpr (MASKED) {
                // keys past the range; in the tree range, non-ancestors
                const uint64_t word = !tree ? ~0ull : mword(qb, i);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = kk0 + h * 16 + r;
                        const bool vis = i * TK + kk < nkeys && ((word >> kk) & 1ull);
                        sc[qb][h][r] = vis ? sc[qb][h][r] : -INFINITY;
                    }
            }
            const float lm = fmaxf(fmaxf(fmaxf(sc[qb][0][0], sc[qb][0][1]), fmaxf(sc[qb][0][2], sc[qb][0][3])),
                                   fmaxf(fmaxf(sc[qb][1][0], sc[qb][1][1]), fmaxf(sc[qb][1][2], sc[qb][1][3])));
            if (__any(lm * scale_log2 > Mq[qb] + MF_LAZY)) {
                // raise the reference of the queries that need it (the pair's
                // max over the query's 4 lanes decides, so they agree)
                float t = fmaxf(lm, __shfl_xor(lm, 16, 64));
                t = fmaxf(t, __shfl_xor(t, 32, 64));
                const float tc = t * scale_log2;
                const float Mn = tc > Mq[qb] + MF_LAZY ? tc : Mq[qb];
                const float alpha = __builtin_amdgcn_exp2f(Mq[qb] - Mn);  // exactly 1 when unchanged
                Mq[qb] = Mn;
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
            }
            // probabilities (bare v_exp_f32: arguments <= 8, masked ones
            // -inf); k-slots 4 h .. 4 h + 3 of the lane's B fragments are
            // keys 4 lk .. 4 lk + 3 of block kb + h
            const float nm = -Mq[qb];
            float pv[8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[h * 4 + r] = __builtin_amdgcn_exp2f(fmaf(sc[qb][h][r], scale_log2, nm));
                    l[qb] += pv[h * 4 + r];
                }
            uint32_t hw[4], rw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                hw[w] = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
                rw[w] = pack_bf16x2(pv[2 * w] - bf16_lo(hw[w]), pv[2 * w + 1] - bf16_hi(hw[w]));
            }
            ph[qb] = (u32x4){hw[0], hw[1], hw[2], hw[3]};
            pr[qb] = (u32x4){rw[0], rw[1], rw[2], rw[3]};
        }
        // rows past the prefix in the last tile of a prefix range hold
        // whatever the cache slots hold (they were requested before the
        // prefix length was known): their probability is 0, but 0 times a
        // NaN or infinite V is NaN, so the lane's V elements of keys past the
        // range are zeroed (element e of a transposed read is key 4 lk + e of
        // its block); only masked pairs pay for this
        uint32_t keep[2][2] = {{~0u, ~0u}, {~0u, ~0u}};
        if constexpr (MASKED) {
            if (!tree) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int nv = nkeys - (i * TK + kk0 + h * 16);  // the lane's keys of block kb + h in range
                    keep[h][0] = nv >= 2 ? ~0u : nv == 1 ? 0x0000FFFFu : 0u;
                    keep[h][1] = nv >= 4 ? ~0u : nv == 3 ? 0x0000FFFFu : 0u;
                }
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            uint2 v0 = __builtin_bit_cast(uint2, ds_read_tr16(st + voff[db] + kb * 16 * ROWB));
            uint2 v1 = __builtin_bit_cast(uint2, ds_read_tr16(st + voff[db] + (kb + 1) * 16 * ROWB));
            if constexpr (MASKED) {
                v0.x &= keep[0][0];
                v0.y &= keep[0][1];
                v1.x &= keep[1][0];
                v1.y &= keep[1][1];
            }
            const u32x4 va = (u32x4){v0.x, v0.y, v1.x, v1.y};
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb)
                o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, ph[qb]), o[qb][db], 0,
                                                                    0, 0);
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb)
                o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, pr[qb]), o[qb][db], 0,
                                                                    0, 0);
        }
    };

    for (int tb = 0; tb < ntiles; tb += MF_STAGES) {
#pragma unroll
        for (int u = 0; u < MF_STAGES; ++u) {
            const int i = tb + u;
            if (i < ntiles) {
                // wait for tile i: the younger requests are those of tiles i+1, i+2
                if (requested(i + 2)) mf_tile_barrier<2 * NLD>();
                else if (requested(i + 1)) mf_tile_barrier<NLD>();
                else mf_tile_barrier<0>();
                if (i + 3 < ntiles) issue((u + 3) % MF_STAGES, i + 3);
                if constexpr (QLDS) {
                    if (i == 0) {
#pragma unroll
                        for (int qb = 0; qb < QBW; ++qb) {
                            const int r = qh * 16 * QBW + qb * 16 + lr;
#pragma unroll
                            for (int ks = 0; ks < DK; ++ks)
                                qf[qb][ks] = *(const u32x4*)(qlds + r * ROWB + (((ks * 4 + lk) ^ mf_swz<DC>(r)) * 16));
                        }
                    }
                }
                const char* st = stage_ptr(u);
                const bool masked = tree || (i + 1) * TK > nkeys;
                if (QBW == 2 && !tree && masked) {
                    // two query blocks a wave (no separate body for full
                    // tiles): the last tile of a prefix range that ends inside
                    // it has rows past the range that hold whatever the cache
                    // slots hold (requested before the prefix length was
                    // known, or slots the tree range is writing); their scores
                    // are masked, but 0 times a NaN or infinite V is NaN, so
                    // those V rows are zeroed here, once, instead of masking V
                    // in every key block of every tile
                    const int r0 = nkeys - i * TK;  // the first row past the range, 1 .. TK - 1
                    for (int e = tid; e < (TK - r0) * DC; e += MF_THREADS)
                        *(u32x4*)(stage_ptr(u) + TILE_B + (r0 + e / DC) * ROWB + (e % DC) * 16) =
                            (u32x4){0u, 0u, 0u, 0u};
                    mf_lds_barrier();
                }
                if constexpr (QBW == 1) {
                    // two 16-key blocks at a time; a tile whose keys are all
                    // visible runs the body compiled without mask work; not
                    // unrolled, so the pairs do not compete for registers
#pragma unroll 1
                    for (int kb = 0; kb < NKB; kb += 2) {
                        if (masked) key_pair(std::true_type{}, st, i, kb);
                        else key_pair(std::false_type{}, st, i, kb);
                    }
                } else {
                // one 16-key block at a time: S^T, mask, reference, then O^T
                // (the online softmax takes its keys in any grouping); not
                // unrolled, so the blocks do not compete for registers (two
                // query blocks per wave leave no room for the pairs)
#pragma unroll 1
                for (int kb = 0; kb < NKB; ++kb) {
                    u32x4 ka[DK];
#pragma unroll
                    for (int ks = 0; ks < DK; ++ks) ka[ks] = *(const u32x4*)(st + koff[ks] + kb * 16 * ROWB);
                    const int kk0 = kq * KW + kb * 16 + lk * 4;  // the lane's first key of the block
                    u32x4 pb[QBW];
#pragma unroll
                    for (int qb = 0; qb < QBW; ++qb) {
                        f32x4 sc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < DK; ++ks)
                            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[ks]),
                                                                         __builtin_bit_cast(bf16x8, qf[qb][ks]), sc, 0,
                                                                         0, 0);
                        // mask: keys past the range; in the tree range, non-ancestors
                        if (masked) {
                            const uint64_t word = !tree ? ~0ull : mword(qb, i);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const bool vis = i * TK + kk0 + r < nkeys && ((word >> (kk0 + r)) & 1ull);
                                sc[r] = vis ? sc[r] : -INFINITY;
                            }
                        }
                        const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                        if (__any(lm * scale_log2 > Mq[qb] + MF_LAZY)) {
                            // raise the reference of the queries that need it (the
                            // block max over the query's 4 lanes decides, so they agree)
                            float t = fmaxf(lm, __shfl_xor(lm, 16, 64));
                            t = fmaxf(t, __shfl_xor(t, 32, 64));
                            const float tc = t * scale_log2;
                            const float Mn = tc > Mq[qb] + MF_LAZY ? tc : Mq[qb];
                            const float alpha = __builtin_amdgcn_exp2f(Mq[qb] - Mn);  // exactly 1 when unchanged
                            Mq[qb] = Mn;
                            l[qb] *= alpha;
#pragma unroll
                            for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
                        }
                        // probabilities (bare v_exp_f32: arguments <= 8, masked
                        // ones -inf) as head + remainder, both bf16 (17 significant
                        // bits together): k-slots 0..3 of the lane's B fragment
                        // carry the heads of its 4 keys, slots 4..7 the remainders,
                        // and the A fragment repeats the 4 keys' V^T values in both
                        // halves
                        const float nm = -Mq[qb];
                        float p4[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            p4[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], scale_log2, nm));
                            l[qb] += p4[r];
                        }
                        const uint32_t h01 = pack_bf16x2(p4[0], p4[1]), h23 = pack_bf16x2(p4[2], p4[3]);
                        const uint32_t r01 = pack_bf16x2(p4[0] - bf16_lo(h01), p4[1] - bf16_hi(h01));
                        const uint32_t r23 = pack_bf16x2(p4[2] - bf16_lo(h23), p4[3] - bf16_hi(h23));
                        pb[qb] = (u32x4){h01, h23, r01, r23};
                    }
                    // O^T += V^T . P^T over the block's 16 keys (V rows past a
                    // prefix range were zeroed in LDS when the tile landed)
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const uint2 v = __builtin_bit_cast(uint2, ds_read_tr16(st + voff[db] + kb * 16 * ROWB));
                        const u32x4 va = (u32x4){v.x, v.y, v.x, v.y};  // the 4 keys' V^T values, twice
#pragma unroll
                        for (int qb = 0; qb < QBW; ++qb)
                            o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                                __builtin_bit_cast(bf16x8, pb[qb]),
                                                                                o[qb][db], 0, 0, 0);
                    }
                }
                }
            }
        }
    }

    // per-query sums over the 4 lanes of the query
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        l[qb] += __shfl_xor(l[qb], 16, 64);
        l[qb] += __shfl_xor(l[qb], 32, 64);
    }
    // the stages become the merge area once no tile load is in flight
    mf_loads_landed();
    // merge the key groups: groups lo .. 2 lo - 1 into 0 .. lo - 1 for lo =
    // KG / 2, .., 1 (the state of source slot k sits in stage k)
#pragma unroll
    for (int lo = KG / 2; lo >= 1; lo /= 2) {
        __syncthreads();                     // the stages (or the previous step's area) are free
        if (kq >= lo && kq < 2 * lo) {
            float* w = (float*)stage_ptr((kq - lo) * QG + qh);
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
                for (int db = 0; db < DB; ++db) *(f32x4*)(w + ((qb * DB + db) * 64 + lane) * 4) = o[qb][db];
                *(float2*)(w + QBW * DB * 64 * 4 + (qb * 64 + lane) * 2) = (float2){Mq[qb], l[qb]};
            }
        }
        __syncthreads();
        if (kq < lo) {
            const float* w = (const float*)stage_ptr(kq * QG + qh);
#pragma unroll
            for (int qb = 0; qb < QBW; ++qb) {
                const float2 ml = *(const float2*)(w + QBW * DB * 64 * 4 + (qb * 64 + lane) * 2);
                const float Mn = fmaxf(Mq[qb], ml.x);
                const float fa = __builtin_amdgcn_exp2f(Mq[qb] - Mn), fb = __builtin_amdgcn_exp2f(ml.x - Mn);
                Mq[qb] = Mn;
                l[qb] = l[qb] * fa + ml.y * fb;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[qb][db] = o[qb][db] * fa + *(const f32x4*)(w + ((qb * DB + db) * 64 + lane) * 4) * fb;
            }
        }
    }
    // key group 0 writes the partial: O^T block db, lane holds
    // d = db * 16 + 4 * lk + r of query column lr
    if (kq == 0) {
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
            if (qidx[qb] < N) {
                const size_t r = prow + qidx[qb];
#pragma unroll
                for (int db = 0; db < DB; ++db) *(f32x4*)(part_o + r * D + db * 16 + lk * 4) = o[qb][db];
                if (lk == 0) {
                    part_ml[r * 2] = l[qb] > 0.f ? Mq[qb] : -INFINITY;
                    part_ml[r * 2 + 1] = l[qb];
                }
            }
        }
    }
    // tree keys/values -> cache slots P..P+N-1 (one writer per KV head)
    if (tree && qblk == 0 && h % grp == 0) {
        for (int e = tid; e < N * DC; e += MF_THREADS) {
            const int t = e / DC, c = e - t * DC;
            const size_t src = (size_t)t * stride + c * 8;
            const size_t dst = (cache_row0 + P + t) * D + c * 8;
            *(u32x4*)(k_cache + dst) = *(const u32x4*)(kbase + src);
            *(u32x4*)(v_cache + dst) = *(const u32x4*)(vbase + src);
        }
    }
}

struct AttnPlan {
    bool mfma;
    int S;    // partial slots per (head, query): key ranges
    int KPS;  // keys per range (MFMA: prefix keys per range; the tree keys are one more range)
    int QB;   // query blocks per head (MFMA)
};

// Workgroups the key-range split aims at: the MFMA path fills one round of
// the 256 CUs (one 8-wave workgroup per CU), the vector-ALU path several.
constexpr int ATT_MFMA_TARGET_WG = 256;
constexpr int ATT_MFMA_MAX_RANGE = 2816;
constexpr int ATT_VALU_TARGET_WG = 1024;

static AttnPlan attn_plan(bool bf16, int B, int nH, int N, int max_cache_len, int target_wg = 0) {
    AttnPlan p;
    p.mfma = bf16 && N <= MEDUSA_MAX_NODES_DEV;
    if (p.mfma) {
        // as many prefix ranges as fit beside the tree range in the target,
        // but no range longer than ATT_MFMA_MAX_RANGE keys (a longer chain of
        // tiles in one workgroup costs more than the extra partials), each a
        // whole number of 64-key tiles (measured: 7 ranges of 320 keys for
        // 32 heads x 2048 keys, 2 of 2048 for 4 query blocks x 32 heads x
        // 4096 keys, 3 of 2752 for 8 x 32 heads up to 8192 keys)
        const int QW = 16 * mf_qbw(N) * mf_qg(N);
        p.QB = (N + QW - 1) / QW;
        const int target = target_wg > 0 ? target_wg : ATT_MFMA_TARGET_WG;
        const int units = B * nH * p.QB;
        int Sp = target / units - 1;
        const int by_len = (max_cache_len + ATT_MFMA_MAX_RANGE - 1) / ATT_MFMA_MAX_RANGE;
        if (Sp < by_len) Sp = by_len;
        if (Sp < 1) Sp = 1;
        long long kps = ((long long)max_cache_len + Sp - 1) / Sp;
        if (kps < MF_TK) kps = MF_TK;
        kps = (kps + MF_TK - 1) / MF_TK * MF_TK;
        p.KPS = (int)kps;
        p.S = (int)((max_cache_len + kps - 1) / kps) + 1;
        return p;
    }
    const int max_total = max_cache_len + N;
    const int base = B * nH * ((N + ATT_QB - 1) / ATT_QB);
    const int target = target_wg > 0 ? target_wg : ATT_VALU_TARGET_WG;
    int S = (target + base - 1) / base;
    const int max_s = (max_total + ATT_TK - 1) / ATT_TK;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    int kps = (max_total + S - 1) / S;
    kps = ((kps + ATT_TK - 1) / ATT_TK) * ATT_TK;
    p.KPS = kps;
    p.S = (max_total + kps - 1) / kps;
    p.QB = 1;
    return p;
}

void launch_tree_attention(const void* q, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                           const int32_t* cache_len, int max_cache_len, const TreeDev& t, int B, int nH,
                           int nKV, int D, int Lmax, float scale, bool bf16, void* out, float* part_o,
                           float* part_ml, hipStream_t s, int target_wg) {
    const int N = t.N;
    const AttnPlan pl = attn_plan(bf16, B, nH, N, max_cache_len, target_wg);
    const float scale_log2 = scale * 1.4426950408889634f;
    if (pl.mfma) {
        const bf16_t *Q = (const bf16_t*)q, *KT = (const bf16_t*)k_tree, *VT = (const bf16_t*)v_tree;
        bf16_t *KC = (bf16_t*)k_cache, *VC = (bf16_t*)v_cache;
        const int units = B * nH * pl.S;
        const dim3 grid((unsigned)(((units + 7) / 8) * 8 * pl.QB));
#define MEDUSA_MF(DD, QG, QBW)                                                                                \
    MEDUSA_LAUNCH("tree_attn_mfma", (tree_attn_mfma_kernel<DD, QG, QBW>), grid, dim3(MF_THREADS), 0, s, Q, KT,  \
                  VT, KC, VC, cache_len, t.mask, N, t.W, nH, nKV, Lmax, max_cache_len, scale_log2, pl.KPS, pl.S, \
                  pl.QB, B * nH, part_o, part_ml, t.status)
        const int qg = mf_qg(N), qbw = mf_qbw(N);
        if (D == 64) {
            if (qbw == 1) MEDUSA_MF(64, 4, 1); else if (qg == 4) MEDUSA_MF(64, 4, 2); else MEDUSA_MF(64, 8, 2);
        } else {
            if (qbw == 1) MEDUSA_MF(128, 4, 1); else if (qg == 4) MEDUSA_MF(128, 4, 2); else MEDUSA_MF(128, 8, 2);
        }
#undef MEDUSA_MF
    } else {
        const dim3 grid(B * nH, pl.S, (N + ATT_QB - 1) / ATT_QB);
#define MEDUSA_ATT(T, DD)                                                                                   \
    MEDUSA_LAUNCH("tree_attn_split", (tree_attn_valu_kernel<T, DD>), grid, dim3(ATT_THREADS), 0, s,         \
                  (const T*)q, (const T*)k_tree, (const T*)v_tree, (T*)k_cache, (T*)v_cache, cache_len,     \
                  t.mask, N, t.W, nH, nKV, Lmax, max_cache_len, scale_log2, pl.KPS, part_o, part_ml, t.status)
        if (bf16) {
            if (D == 64) MEDUSA_ATT(bf16_t, 64); else MEDUSA_ATT(bf16_t, 128);
        } else {
            if (D == 64) MEDUSA_ATT(float, 64); else MEDUSA_ATT(float, 128);
        }
#undef MEDUSA_ATT
    }
#define MEDUSA_MERGE(T, DD)                                                                                  \
    MEDUSA_LAUNCH("tree_attn_merge", (tree_attn_merge_kernel<T, DD>),                                        \
                  dim3((N + ATT_MERGE_THREADS / (DD / 4) - 1) / (ATT_MERGE_THREADS / (DD / 4)), B * nH),     \
                  dim3(ATT_MERGE_THREADS), 0, s, part_o, part_ml, pl.S, N, nH, (T*)out)
    if (bf16) {
        if (D == 64) MEDUSA_MERGE(bf16_t, 64); else MEDUSA_MERGE(bf16_t, 128);
    } else {
        if (D == 64) MEDUSA_MERGE(float, 64); else MEDUSA_MERGE(float, 128);
    }
#undef MEDUSA_MERGE
}

size_t attn_workspace_bytes(int B, int nH, int N, int D, int max_cache_len, bool bf16) {
    const int S = attn_plan(bf16, B, nH, N, max_cache_len).S;
    const size_t rows = (size_t)B * nH * S * N;
    return (rows * D * sizeof(float) + 255) / 256 * 256 + rows * 2 * sizeof(float);
}

void attn_carve(int B, int nH, int N, int D, int max_cache_len, bool bf16, void* ws, float** part_o,
                float** part_ml) {
    const int S = attn_plan(bf16, B, nH, N, max_cache_len).S;
    const size_t rows = (size_t)B * nH * S * N;
    *part_o = (float*)ws;
    *part_ml = (float*)((char*)ws + (rows * D * sizeof(float) + 255) / 256 * 256);
}

}  // namespace medusa
