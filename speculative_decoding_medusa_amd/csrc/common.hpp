// Shared device/host helpers of the Medusa step library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace medusa {

constexpr int MEDUSA_MAX_TOPK_DEV = 16;
constexpr int MEDUSA_MAX_DEPTH_DEV = 16;
constexpr int MEDUSA_MAX_NODES_DEV = 256;

// Bits of a tree handle's status word (the MEDUSA_STATUS_* values of the C
// header): an invalid device-side length was clamped or an operation skipped.
constexpr int STATUS_CACHE_LEN_CLAMPED = 1;
constexpr int STATUS_CACHE_OVERFLOW = 2;

// ---------------------------------------------------------------------------
// Storage types
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// One 16-byte load of data that is streamed once per call (weights, KV
// cache): non-temporal, so it does not displace reused lines from the caches.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Two floats -> packed bf16 pair (low half = lo), round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Two floats -> packed fp16 pair (low half = lo), round to nearest even, in
// one v_cvt_pk_f16_f32.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int PER16 = 4;  // elements per 16-byte chunk
    __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
    // expand one 16-byte chunk into floats
    __device__ __forceinline__ static void expand(const u32x4& c, float* out) {
        out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
        out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
    }
};
template <> struct Elem<bf16_t> {
    static constexpr int PER16 = 8;
    __device__ __forceinline__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
    __device__ __forceinline__ static void expand(const u32x4& c, float* out) {
        out[0] = bf16_lo(c.x); out[1] = bf16_hi(c.x); out[2] = bf16_lo(c.y); out[3] = bf16_hi(c.y);
        out[4] = bf16_lo(c.z); out[5] = bf16_hi(c.z); out[6] = bf16_lo(c.w); out[7] = bf16_hi(c.w);
    }
};

// ---------------------------------------------------------------------------
// Wavefront (64-lane) reductions.  The xor butterfly leaves the bitwise same
// result in every lane (each step adds the same two operands in both lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// (value, index) ordering of top-k / argmax: larger value first, then lower index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Wave-wide argmax of (v, i) pairs; every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        float ov = __shfl_xor(v, m, 64);
        int oi = __shfl_xor(i, m, 64);
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Sorted register list of the best TK (value, index) pairs, best first.
template <int TK>
__device__ __forceinline__ void sorted_insert(float (&lv)[TK], int (&li)[TK], float v, int i) {
    if (!better(v, i, lv[TK - 1], li[TK - 1])) return;
    lv[TK - 1] = v;
    li[TK - 1] = i;
#pragma unroll
    for (int t = TK - 1; t > 0; --t) {
        if (better(lv[t], li[t], lv[t - 1], li[t - 1])) {
            const float tv = lv[t]; lv[t] = lv[t - 1]; lv[t - 1] = tv;
            const int ti = li[t]; li[t] = li[t - 1]; li[t - 1] = ti;
        }
    }
}
template <int TK>
__device__ __forceinline__ void sorted_pop(float (&lv)[TK], int (&li)[TK]) {
#pragma unroll
    for (int u = 0; u < TK - 1; ++u) { lv[u] = lv[u + 1]; li[u] = li[u + 1]; }
    lv[TK - 1] = -INFINITY;
    li[TK - 1] = 0x7FFFFFFF;
}

}  // namespace medusa

// ---------------------------------------------------------------------------
// Host-side launch plumbing (profiler hooks, error text).
// ---------------------------------------------------------------------------
namespace medusa {
void set_error(const std::string& msg);
void prof_before(const char* name, hipStream_t s);
void prof_after(hipStream_t s);
}  // namespace medusa

#define MEDUSA_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                   \
    do {                                                                               \
        ::medusa::prof_before(name, stream);                                           \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);           \
        ::medusa::prof_after(stream);                                                  \
    } while (0)
