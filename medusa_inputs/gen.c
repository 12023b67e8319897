/*
 * Seeded synthetic-input generator shared by the CPU oracle's tests and the
 * GPU path's tests and benchmark.  It holds none of the Medusa method's
 * arithmetic: it only turns (seed, stream, element index) into numbers.
 *
 * Counter-based, so any element of any tensor can be regenerated on its own:
 *   words = Philox4x32-10(counter = {lo32(e), hi32(e), stream, 0x6d656475},
 *                         key     = {lo32(seed), hi32(seed)})
 * Philox4x32-10 is the generator published by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds of two
 * 32x32->64-bit multiplies with a Weyl-sequence key schedule.
 *
 * Normal variates use an Irwin-Hall sum of the eight 16-bit halves u_j of the
 * four output words:  x = sum_j (2 u_j - 65535), an even integer with
 * |x| <= 524280, mean 0 and variance (8/3)(65536^2 - 1).  The float32 value
 * is float(x) * s with s = float32(sigma / sqrt((8/3)(65536^2 - 1))): one
 * correctly rounded multiply, so every IEEE-754 implementation produces the
 * same bits.  bf16 values are the float32 value rounded to nearest-even.
 * The sum of eight uniforms has excess kurtosis -0.15 and tails cut at
 * +-4.9 sigma; it stands in for N(0, sigma^2).
 *
 * Uniform integers in [lo, hi] use the first word w: lo + (w * (hi-lo+1)) >> 32.
 *
 * Build: gcc -O3 -fopenmp -shared -fPIC gen.c -o libmedusa_inputs.so
 */
#include <stdint.h>
#include <math.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u
#define STREAM_TAG 0x6d656475u

static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
        uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k0;
        uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
}

/* Raw block, exported for known-answer tests. */
void mi_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    philox4x32_10(c, key[0], key[1]);
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

static inline void block(uint64_t seed, uint32_t stream, uint64_t e, uint32_t w[4]) {
    w[0] = (uint32_t)e; w[1] = (uint32_t)(e >> 32); w[2] = stream; w[3] = STREAM_TAG;
    philox4x32_10(w, (uint32_t)seed, (uint32_t)(seed >> 32));
}

static inline int32_t irwin_hall8(const uint32_t w[4]) {
    int32_t x = 0;
    for (int j = 0; j < 4; ++j) {
        x += 2 * (int32_t)(w[j] & 0xFFFFu) - 65535;
        x += 2 * (int32_t)(w[j] >> 16) - 65535;
    }
    return x;
}

static float normal_scale(double sigma) {
    return (float)(sigma / sqrt((8.0 / 3.0) * (65536.0 * 65536.0 - 1.0)));
}

static inline uint16_t f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v; v.f = f;
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void mi_normal_f32(float* out, uint64_t n, uint64_t seed, uint32_t stream,
                   uint64_t offset, double sigma) {
    const float s = normal_scale(sigma);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t w[4];
        block(seed, stream, offset + (uint64_t)i, w);
        out[i] = (float)irwin_hall8(w) * s;
    }
}

void mi_normal_bf16(uint16_t* out, uint64_t n, uint64_t seed, uint32_t stream,
                    uint64_t offset, double sigma) {
    const float s = normal_scale(sigma);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t w[4];
        block(seed, stream, offset + (uint64_t)i, w);
        out[i] = f32_to_bf16_rne((float)irwin_hall8(w) * s);
    }
}

void mi_uniform_i32(int32_t* out, uint64_t n, uint64_t seed, uint32_t stream,
                    uint64_t offset, int32_t lo, int32_t hi) {
    const uint64_t span = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t w[4];
        block(seed, stream, offset + (uint64_t)i, w);
        out[i] = (int32_t)((int64_t)lo + (int64_t)(((uint64_t)w[0] * span) >> 32));
    }
}

/* Uniform float32 in [0, 1): (w >> 8) * 2^-24, exact. */
void mi_uniform_f32(float* out, uint64_t n, uint64_t seed, uint32_t stream, uint64_t offset) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        uint32_t w[4];
        block(seed, stream, offset + (uint64_t)i, w);
        out[i] = (float)(w[0] >> 8) * (1.0f / 16777216.0f);
    }
}
