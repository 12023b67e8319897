// Measurement aids.  stream_read: the achievable HBM read rate with the
// access pattern the weight streams use (16-byte non-temporal loads, several
// in flight per thread, all workgroups busy); the streaming kernels' rates
// are compared with it next to the HBM peak.  read_mix: what one workgroup
// per CU can pull through its vector-memory path from a shared L2-resident
// window, from its own HBM slice, or from both mixed in the same waves (the
// wide lm_head's node rows and weights).  mfma_rate: the wide lm_head's
// matrix loop (32 x 32 x 16 bf16 products with node fragments from LDS, one
// barrier per 32 products) on constant or random operands.
#include "common.hpp"

namespace medusa {

constexpr int READ_THREADS = 256;
constexpr int READ_INFLIGHT = 4;  // 16-byte loads in flight per thread (measured: 4 ahead of 8 and 16)

// Each workgroup reads a contiguous slice; the XOR of every loaded word goes
// to one value per workgroup, so no load can be dropped.
__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const size_t per_wg = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per_wg;
    const size_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
    uint32_t acc = 0;
    for (size_t i0 = lo + threadIdx.x; i0 < hi; i0 += (size_t)READ_THREADS * READ_INFLIGHT) {
        u32x4 v[READ_INFLIGHT];
#pragma unroll
        for (int u = 0; u < READ_INFLIGHT; ++u) {
            const size_t i = i0 + (size_t)u * READ_THREADS;
            v[u] = i < hi ? ld_stream(src + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < READ_INFLIGHT; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    __shared__ uint32_t red[READ_THREADS / 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < READ_THREADS / 64; ++w) t ^= red[w];
        sink[blockIdx.x] = t;
    }
}

void launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s) {
    MEDUSA_LAUNCH("stream_read", stream_read_kernel, dim3(n_wg), dim3(READ_THREADS), 0, s, (const u32x4*)src,
                  bytes / 16, sink);
}

// One round: every thread issues WP window loads (plain: the window stays in
// L2) and SP loads of its workgroup's slice of `src` (non-temporal), all in
// flight together, then XORs them.  The window is read in 4 KB blocks (256 threads x 16 bytes),
// consecutive per round and wrapping at its end; the slice of workgroup g is
// rounds x SP x 4 KB starting at g times that.
template <int WP, int SP>
__global__ __launch_bounds__(READ_THREADS) void read_mix_kernel(const u32x4* __restrict__ win, size_t w16,
                                                                const u32x4* __restrict__ src, int rounds,
                                                                uint32_t* __restrict__ sink) {
    const int tid = threadIdx.x;
    const u32x4* slice = src + (size_t)blockIdx.x * rounds * SP * READ_THREADS;
    size_t wpos = 0;  // window position of this round's first block, in 16-byte units
    uint32_t acc = 0;
    for (int r = 0; r < rounds; ++r) {
        u32x4 v[WP + SP];
#pragma unroll
        for (int u = 0; u < WP; ++u) v[u] = win[wpos + (size_t)u * READ_THREADS + tid];
#pragma unroll
        for (int u = 0; u < SP; ++u) v[WP + u] = ld_stream(slice + ((size_t)r * SP + u) * READ_THREADS + tid);
        // every load of the round is issued before the first is consumed (left
        // to itself the compiler interleaves the XORs and waits after three)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < WP + SP; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        if constexpr (WP > 0) {
            wpos += (size_t)WP * READ_THREADS;
            if (wpos == w16) wpos = 0;  // the window is a whole number of rounds
        }
    }
    __shared__ uint32_t red[READ_THREADS / 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < READ_THREADS / 64; ++w) t ^= red[w];
        sink[blockIdx.x] = t;
    }
}

// (window parts, stream parts) pairs with a compiled kernel
bool read_mix_supported(int wp, int sp) {
    return (wp == 8 && sp == 0) || (wp == 0 && sp == 8) || (wp == 4 && sp == 2) || (wp == 8 && sp == 4);
}

void launch_read_mix(const void* win, size_t win_bytes, const void* src, int wp, int sp, int rounds,
                     uint32_t* sink, int n_wg, hipStream_t s) {
    const u32x4* W = (const u32x4*)win;
    const u32x4* S = (const u32x4*)src;
    const size_t w16 = win_bytes / 16;
#define MEDUSA_MIX(A, B)                                                                                   \
    MEDUSA_LAUNCH("read_mix", (read_mix_kernel<A, B>), dim3(n_wg), dim3(READ_THREADS), 0, s, W, w16, S, rounds, \
                  sink)
    if (wp == 8 && sp == 0) MEDUSA_MIX(8, 0);
    else if (wp == 0 && sp == 8) MEDUSA_MIX(0, 8);
    else if (wp == 4 && sp == 2) MEDUSA_MIX(4, 2);
    else MEDUSA_MIX(8, 4);
#undef MEDUSA_MIX
}

// The wide lm_head's matrix-wave loop: 4 waves (one per SIMD), each with 8
// independent 32 x 32 x 16 accumulators; per iteration 4 k-steps, each
// reading the 8 node fragments of the next k-step from LDS (128-byte rows,
// 16-byte column c of row r at c ^ ((r >> 1) & 7)) while the current 8
// products run, then a barrier.  The A operand stays in registers.
// Operands: RND = 0 every bf16 element 1.0 (A and B), so every accumulator
// element ends at iters x 64; RND = 1 bf16 values of random sign and
// magnitude in [0.25, 2) from a hash of the element's position.
// out[blockIdx.x * 256 + thread] = the sum of the thread's 128 accumulator
// elements.
__device__ __forceinline__ uint32_t mr_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
__device__ __forceinline__ bf16_t mr_value(uint32_t i, int rnd) {
    if (!rnd) return 0x3f80;  // 1.0
    const uint32_t h = mr_hash(i * 2654435761u + 12345u);
    return (bf16_t)(((h & 1u) << 15) | ((125u + (h >> 1) % 4u) << 7) | ((h >> 8) & 0x7fu));
}

template <int RND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) bf16_t ns[2][256][64];
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5, rsw = (l32 >> 1) & 7;
    for (int i = tid; i < 2 * 256 * 64; i += 256) (&ns[0][0][0])[i] = mr_value((uint32_t)(blockIdx.x * 32768 + i), RND);
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = __builtin_bit_cast(__bf16, mr_value((uint32_t)(tid * 8 + e + 999999), RND));
    __syncthreads();
    auto read_b = [&](int st, int s, int t) {
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(&ns[st][t * 32 + l32][((2 * s + hi) ^ rsw) * 8]));
    };
    f32x16 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = (f32x16){};
    bf16x8 bc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) bc[t] = read_b(0, 0, t);
    for (int it = 0; it < iters; ++it) {
        const int st = it & 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 bn[8];
            const int sn = s + 1 < 4 ? s + 1 : 0, stn = s + 1 < 4 ? st : st ^ 1;
#pragma unroll
            for (int t = 0; t < 8; ++t) bn[t] = read_b(stn, sn, t);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bc[t], acc[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 8; ++t) bc[t] = bn[t];
        }
        __syncthreads();
    }
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[t][r];
    out[(size_t)blockIdx.x * 256 + tid] = sum;
}

void launch_mfma_rate(int random_operands, int iters, float* out, int n_wg, hipStream_t s) {
    if (random_operands)
        MEDUSA_LAUNCH("mfma_rate", mfma_rate_kernel<1>, dim3(n_wg), dim3(256), 0, s, iters, out);
    else
        MEDUSA_LAUNCH("mfma_rate", mfma_rate_kernel<0>, dim3(n_wg), dim3(256), 0, s, iters, out);
}

}  // namespace medusa
