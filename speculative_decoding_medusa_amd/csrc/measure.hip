// Measurement aid: the achievable HBM read rate with the access pattern the
// weight streams use (16-byte non-temporal loads, several in flight per
// thread, all workgroups busy).  The streaming kernels' rates are compared
// with it next to the HBM peak.
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

}  // namespace medusa
