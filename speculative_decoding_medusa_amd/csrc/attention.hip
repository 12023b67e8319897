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
// The S (m, l) pairs are read in parallel into LDS first; the partial rows are
// then summed four splits at a time (independent loads in flight).
constexpr int ATT_MAX_SPLITS = 1024;

template <typename T, int D>
__global__ __launch_bounds__(D) void tree_attn_combine_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml, int S, int N,
                                                              int nH, T* __restrict__ out) {
    __shared__ float ms[ATT_MAX_SPLITS];
    __shared__ float ls[ATT_MAX_SPLITS];
    __shared__ float red[D / 64];
    const int i = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / nH, h = bh - b * nH;
    const int c = threadIdx.x;
    float mloc = -INFINITY;
    for (int s = c; s < S; s += D) {
        const size_t pr = ((size_t)bh * S + s) * N + i;
        ms[s] = part_ml[pr * 2];
        ls[s] = part_ml[pr * 2 + 1];
        mloc = fmaxf(mloc, ms[s]);
    }
    mloc = wave_max(mloc);
    if ((c & 63) == 0) red[c >> 6] = mloc;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) M = fmaxf(M, red[w]);
    float L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + u;
            v[u] = (s < S && ms[s] != -INFINITY) ? part_o[(((size_t)bh * S + s) * N + i) * D + c] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int s = s0 + u;
            if (s < S && ms[s] != -INFINITY) {
                const float f = exp2f(ms[s] - M);
                L += f * ls[s];
                acc += f * v[u];
            }
        }
    }
    Elem<T>::store(out, (((size_t)b * N + i) * nH + h) * D + c, acc / L);
}

// ---------------------------------------------------------------------------
// bf16 MFMA variant.  The same split-KV decomposition, with the contractions
// on MFMA in transposed form so that no register data has to move between
// lanes:
//   S^T[key][q] = K . Q^T   (v_mfma_f32_16x16x32_bf16; A = K tile rows from
//                            LDS, B = the wave's Q rows held in registers for
//                            the whole kernel);
//   the output layout gives each lane 4 consecutive keys of one query per
//   16-key block, exactly the 8 values the next product needs as its B
//   operand, so P^T never leaves the lane;
//   O^T[d][q] += V^T . P^T (v_mfma_f32_16x16x32_f16; A = V^T from an LDS tile
//                            stored transposed, [d][key], widened to fp16; B =
//                            the probabilities rounded to fp16, whose 11-bit
//                            significand keeps the weighted sum 8x closer to
//                            the exact one than bf16 would; the contraction
//                            runs over the keys in a fixed permuted order, the
//                            same for both operands).
// The online-softmax state of query q lives in the 4 lanes that hold column q.
// Tiles of 64 keys are staged in LDS by the whole workgroup, up to three tiles
// in flight in a register ring.
// ---------------------------------------------------------------------------
constexpr int MF_TK = 64;

template <int D, int WAVES, int QBW>
__global__ __launch_bounds__(WAVES * 64) void tree_attn_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_tree, const bf16_t* __restrict__ v_tree,
    bf16_t* __restrict__ k_cache, bf16_t* __restrict__ v_cache, const int32_t* __restrict__ cache_len,
    const uint64_t* __restrict__ mask, int N, int W, int nH, int nKV, int Lmax, int max_cache_len,
    float scale_log2, int KPS, float* __restrict__ part_o, float* __restrict__ part_ml) {
    constexpr int NT = WAVES * 64;
    constexpr int TK = MF_TK;
    constexpr int KB = TK / 16;     // 16-key blocks per tile
    constexpr int DK = D / 32;      // k-steps of S over the head dimension
    constexpr int DB = D / 16;      // 16-row blocks of O^T
    constexpr int CH = TK * D / 8;  // 16-byte chunks per tile per tensor
    constexpr int PT = CH / NT;     // chunks per thread
    constexpr int DC = D / 8;       // chunks per key row
    __shared__ __attribute__((aligned(16))) bf16_t Ks[TK][D + 8];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D][TK + 4];  // fp16 bits; 136-byte rows: 4-way write conflicts at most

    const int bh = blockIdx.x;
    const int b = bh / nH, h = bh - b * nH;
    const int grp = nH / nKV;
    const int kvh = h / grp;
    const int S = gridDim.y;
    const int s = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int P = max(0, min(cache_len[b], max_cache_len));
    const int total = P + N;

    if (s == 0 && h % grp == 0) {
        for (int e = tid; e < N * DC; e += NT) {
            const int t = e / DC, c = e - t * DC;
            const size_t src = (((size_t)b * N + t) * nKV + kvh) * D + c * 8;
            const size_t dst = (((size_t)b * nKV + kvh) * Lmax + P + t) * D + c * 8;
            *(u32x4*)(k_cache + dst) = *(const u32x4*)(k_tree + src);
            *(u32x4*)(v_cache + dst) = *(const u32x4*)(v_tree + src);
        }
    }

    // this lane's queries (column lr of each of its 16-query blocks)
    u32x4 qf[QBW][DK];
    uint64_t mrow[QBW][4];
    int qidx[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int qi = (wave * QBW + qb) * 16 + lr;
        qidx[qb] = qi;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
            qf[qb][ks] = qi < N ? *(const u32x4*)(q + (((size_t)b * N + qi) * nH + h) * D + ks * 32 + lk * 8)
                                : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int w = 0; w < 4; ++w) mrow[qb][w] = (qi < N && w < W) ? mask[(size_t)qi * W + w] : 0ull;
    }

    f32x4 o[QBW][DB];
    float m[QBW], l[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    const int k_begin = s * KPS;
    const int k_end = min(total, k_begin + KPS);
    const size_t cache_row0 = ((size_t)b * nKV + kvh) * Lmax;

    // Tile loads: thread t owns KPT consecutive keys (group t / DC) and the
    // 16-byte column chunk t % DC of each, so 16 lanes read one 256-byte key
    // row contiguously.  K goes to LDS row-major; V is transposed in
    // registers (v_perm_b32 pairs the same column of two keys) and written as
    // KPT-key runs of each column row of Vt.
    constexpr int KPT = PT;  // keys per thread per tile
    const int kg = tid / DC, dc = tid - (tid / DC) * DC;
    // Register ring of RING tiles: a workgroup's first RING tiles are all in
    // flight before the first is consumed, and each consumed slot is refilled
    // with the tile RING ahead.  Loads complete in issue order, so waiting for
    // the oldest slot never waits for a younger one.
    constexpr int RING = QBW == 1 ? 3 : 1;
    u32x4 kreg[RING][KPT], vreg[RING][KPT];
    auto load_tile = [&](u32x4(&kr)[KPT], u32x4(&vr)[KPT], int t0) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int j = t0 + kg * KPT + e;
            if (j < k_end) {
                if (j < P) {
                    const size_t off = (cache_row0 + j) * D + dc * 8;
                    kr[e] = ld_stream(k_cache + off);
                    vr[e] = ld_stream(v_cache + off);
                } else {
                    const size_t off = (((size_t)b * N + (j - P)) * nKV + kvh) * D + dc * 8;
                    kr[e] = *(const u32x4*)(k_tree + off);
                    vr[e] = *(const u32x4*)(v_tree + off);
                }
            } else {
                kr[e] = (u32x4){0u, 0u, 0u, 0u};
                vr[e] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };
    // K -> LDS row-major (bf16); V widened to fp16 (exact for every bf16 value
    // of magnitude >= 2^-14; smaller ones move by < 2^-25), transposed in
    // registers and written as KPT-key runs of each row of Vt.
    auto store_tile = [&](const u32x4(&kr)[KPT], const u32x4(&vr)[KPT]) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) *(u32x4*)(&Ks[kg * KPT + e][dc * 8]) = kr[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // column dc * 8 + i
            float f[KPT];
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                f[e] = (i & 1) ? bf16_hi(vr[e][i >> 1]) : bf16_lo(vr[e][i >> 1]);
            uint16_t* dst = &Vt[dc * 8 + i][kg * KPT];
            if (KPT == 4) {
                *(uint2*)dst = (uint2){pack_f16x2(f[0], f[1]), pack_f16x2(f[2 % KPT], f[3 % KPT])};
            } else if (KPT == 2) {
                *(uint32_t*)dst = pack_f16x2(f[0], f[1 % KPT]);
            } else {
                *dst = (uint16_t)(pack_f16x2(f[0], 0.f) & 0xFFFFu);
            }
        }
    };
#pragma unroll
    for (int u = 0; u < RING; ++u)
        if (k_begin + u * TK < k_end) load_tile(kreg[u], vreg[u], k_begin + u * TK);
    for (int tb = k_begin; tb < k_end; tb += RING * TK) {
#pragma unroll
        for (int u = 0; u < RING; ++u) {
            const int t0 = tb + u * TK;
            if (t0 < k_end) {
                __syncthreads();
                store_tile(kreg[u], vreg[u]);
                __syncthreads();
                if (t0 + RING * TK < k_end) load_tile(kreg[u], vreg[u], t0 + RING * TK);
                {  // compute tile t0 (written inline: a lambda here made the compiler spill)
        // tiles entirely inside the prefix and the split need no masking
        // (padded query columns are never written out)
        const bool plain = QBW == 1 && t0 + TK <= P && t0 + TK <= k_end;
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
            f32x4 st[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                st[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK; ++ks) {
                    const u32x4 a = *(const u32x4*)(&Ks[kb * 16 + lr][ks * 32 + lk * 8]);
                    st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                     __builtin_bit_cast(bf16x8, qf[qb][ks]), st[kb],
                                                                     0, 0, 0);
                }
            }
            // scale, mask (prefix: visible; tree key t: ancestor bit), tile max
            const int qi = qidx[qb];
            float tmax = -INFINITY;
            if (plain) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        st[kb][r] *= scale_log2;
                        tmax = fmaxf(tmax, st[kb][r]);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = t0 + kb * 16 + lk * 4 + r;
                        bool vis = j < k_end && qi < N;
                        if (vis && j >= P) {
                            const int t = j - P;
                            const int w = t >> 6;
                            const uint64_t word = w == 0 ? mrow[qb][0] : w == 1 ? mrow[qb][1]
                                                                      : w == 2 ? mrow[qb][2] : mrow[qb][3];
                            vis = (word >> (t & 63)) & 1ull;
                        }
                        const float x = vis ? st[kb][r] * scale_log2 : -INFINITY;
                        st[kb][r] = x;
                        tmax = fmaxf(tmax, x);
                    }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m[qb], tmax);
            const bool live = m_new != -INFINITY;
            // exponents are <= 0: the bare v_exp_f32 (no denormal range fix-up;
            // results below 2^-126 vanish in the fp16 probabilities anyway)
            const float alpha = live ? __builtin_amdgcn_exp2f(m[qb] - m_new) : 1.f;
            float psum = 0.f;
            uint32_t pk[KB][2];  // fp16 pairs of P^T (round to nearest even)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float p4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p4[r] = live ? __builtin_amdgcn_exp2f(st[kb][r] - m_new) : 0.f;
                    psum += p4[r];
                }
                pk[kb][0] = pack_f16x2(p4[0], p4[1]);
                pk[kb][1] = pack_f16x2(p4[2], p4[3]);
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            l[qb] = l[qb] * alpha + psum;
            m[qb] = m_new;
            // the accumulators live in AGPRs, so a rescale costs three instructions
            // per element: skip it when no query of the wave raised its max
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
            }
#pragma unroll
            for (int k2 = 0; k2 < TK / 32; ++k2) {
                const u32x4 bp = (u32x4){pk[2 * k2][0], pk[2 * k2][1], pk[2 * k2 + 1][0], pk[2 * k2 + 1][1]};
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint2 lo = *(const uint2*)(&Vt[db * 16 + lr][k2 * 32 + lk * 4]);
                    const uint2 hi = *(const uint2*)(&Vt[db * 16 + lr][k2 * 32 + 16 + lk * 4]);
                    const u32x4 av = (u32x4){lo.x, lo.y, hi.x, hi.y};
                    o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                                       __builtin_bit_cast(f16x8, bp), o[qb][db], 0,
                                                                       0, 0);
                }
            }
        }
                    }
            }
        }
    }

    // O^T block db: lane holds d = db*16 + 4*lk + r of query column lr
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
        const int qi = qidx[qb];
        if (qi < N) {
            const size_t pr = ((size_t)bh * S + s) * N + qi;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *(f32x4*)(part_o + pr * D + db * 16 + lk * 4) = o[qb][db];
            if (lk == 0) { part_ml[pr * 2] = m[qb]; part_ml[pr * 2 + 1] = l[qb]; }
        }
    }
}

struct AttnPlan {
    bool mfma;
    int S;    // splits of the key range
    int KPS;  // keys per split
};

// Workgroups the split of the key range aims at (MFMA path / vector-ALU path).
constexpr int ATT_MFMA_TARGET_WG = 256;
constexpr int ATT_VALU_TARGET_WG = 1024;

static AttnPlan attn_plan(bool bf16, int B, int nH, int N, int max_total, int target_wg = 0) {
    AttnPlan p;
    p.mfma = bf16 && N <= MEDUSA_MAX_NODES_DEV;
    const int unit = p.mfma ? 32 : ATT_TK;
    const int qblocks = p.mfma ? 1 : (N + ATT_QB - 1) / ATT_QB;
    const int base = B * nH * qblocks;
    const int target = target_wg > 0 ? target_wg : p.mfma ? ATT_MFMA_TARGET_WG : ATT_VALU_TARGET_WG;
    int S = (target + base - 1) / base;
    const int max_s = (max_total + unit - 1) / unit;
    if (S > max_s) S = max_s;
    if (S > ATT_MAX_SPLITS) S = ATT_MAX_SPLITS;
    if (S < 1) S = 1;
    int kps = (max_total + S - 1) / S;
    kps = ((kps + unit - 1) / unit) * unit;
    p.KPS = kps;
    p.S = (max_total + kps - 1) / kps;
    return p;
}

void launch_tree_attention(const void* q, const void* k_tree, const void* v_tree, void* k_cache, void* v_cache,
                           const int32_t* cache_len, int max_cache_len, const TreeDev& t, int B, int nH,
                           int nKV, int D, int Lmax, float scale, bool bf16, void* out, float* part_o,
                           float* part_ml, hipStream_t s, int target_wg) {
    const int N = t.N;
    const AttnPlan pl = attn_plan(bf16, B, nH, N, max_cache_len + N, target_wg);
    const float scale_log2 = scale * 1.4426950408889634f;
    if (pl.mfma) {
        const bf16_t *Q = (const bf16_t*)q, *KT = (const bf16_t*)k_tree, *VT = (const bf16_t*)v_tree;
        bf16_t *KC = (bf16_t*)k_cache, *VC = (bf16_t*)v_cache;
#define MEDUSA_MF(DD, WV, QB)                                                                                   \
    MEDUSA_LAUNCH("tree_attn_mfma", (tree_attn_mfma_kernel<DD, WV, QB>), dim3(B * nH, pl.S), dim3(WV * 64), 0, s, \
                  Q, KT, VT, KC, VC, cache_len, t.mask, N, t.W, nH, nKV, Lmax, max_cache_len, scale_log2, pl.KPS,   \
                  part_o, part_ml)
        if (D == 64) {
            if (N <= 64) MEDUSA_MF(64, 4, 1); else if (N <= 128) MEDUSA_MF(64, 4, 2); else MEDUSA_MF(64, 8, 2);
        } else {
            if (N <= 64) MEDUSA_MF(128, 4, 1); else if (N <= 128) MEDUSA_MF(128, 4, 2); else MEDUSA_MF(128, 8, 2);
        }
#undef MEDUSA_MF
        if (D == 64)
            MEDUSA_LAUNCH("tree_attn_combine", (tree_attn_combine_kernel<bf16_t, 64>), dim3(N, B * nH), dim3(64), 0,
                          s, part_o, part_ml, pl.S, N, nH, (bf16_t*)out);
        else
            MEDUSA_LAUNCH("tree_attn_combine", (tree_attn_combine_kernel<bf16_t, 128>), dim3(N, B * nH), dim3(128),
                          0, s, part_o, part_ml, pl.S, N, nH, (bf16_t*)out);
        return;
    }
    const dim3 grid(B * nH, pl.S, (N + ATT_QB - 1) / ATT_QB);
    const int S = pl.S, KPS = pl.KPS;
#define MEDUSA_ATT(T, DD)                                                                                   \
    do {                                                                                                    \
        MEDUSA_LAUNCH("tree_attn_split", (tree_attn_valu_kernel<T, DD>), grid, dim3(ATT_THREADS), 0, s,     \
                      (const T*)q, (const T*)k_tree, (const T*)v_tree, (T*)k_cache, (T*)v_cache, cache_len, \
                      t.mask, N, t.W, nH, nKV, Lmax, max_cache_len, scale_log2, KPS, part_o, part_ml);      \
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

size_t attn_workspace_bytes(int B, int nH, int N, int D, int max_cache_len, bool bf16) {
    const int S = attn_plan(bf16, B, nH, N, max_cache_len + N).S;
    const size_t rows = (size_t)B * nH * S * N;
    return (rows * D * sizeof(float) + 255) / 256 * 256 + rows * 2 * sizeof(float);
}

void attn_carve(int B, int nH, int N, int D, int max_cache_len, bool bf16, void* ws, float** part_o,
                float** part_ml) {
    const int S = attn_plan(bf16, B, nH, N, max_cache_len + N).S;
    const size_t rows = (size_t)B * nH * S * N;
    *part_o = (float*)ws;
    *part_ml = (float*)((char*)ws + (rows * D * sizeof(float) + 255) / 256 * 256);
}

}  // namespace medusa
