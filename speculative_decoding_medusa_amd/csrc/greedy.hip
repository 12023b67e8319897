// Base model's greedy choice after every tree node (step a5):
// n_r = x_r * rsqrt(mean(x_r^2) + eps) (bf16-rounded for bf16 weights), then
// greedy[r] = argmax_v lm_head[v] . n_r.
#include "common.hpp"

namespace medusa {

// One block per row; writes n as float32 (holding bf16-representable values
// when round_bf16 is set).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* __restrict__ x, int H, float eps,
                                                           int round_bf16, float* __restrict__ n) {
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
    for (int j = threadIdx.x; j < H; j += 256) {
        float v = Elem<T>::load(xr, j) * rs;
        if (round_bf16) v = bf16_to_f32(f32_to_bf16(v));
        n[(size_t)r * H + j] = v;
    }
}

void launch_vocab_topk(const float* z, const void* w2, int B, int H, int V, int K, int topk, bool bf16,
                       float* logits, int32_t* topk_idx, float* topk_val, float* cv, int* ci, hipStream_t s);
int vocab_topk_groups(int V, int K);

size_t greedy_workspace_bytes(int R, int H, int V) {
    const int G = vocab_topk_groups(V, 1);
    return (size_t)R * H * 4 + 256 + (size_t)8 * G * 8 + 256 + (size_t)R * 4 + 256;
}

void launch_base_greedy(const void* x, const void* lm_head, int R, int H, int V, float eps, bool bf16,
                        int32_t* greedy, float* logits, void* ws, hipStream_t s) {
    char* p = (char*)ws;
    float* n = (float*)p;
    p += ((size_t)R * H * 4 + 255) / 256 * 256;
    const int G = vocab_topk_groups(V, 1);
    float* cv = (float*)p;
    int* ci = (int*)(p + (size_t)8 * G * 4);
    p += ((size_t)8 * G * 8 + 255) / 256 * 256;
    float* gval = (float*)p;
    if (bf16)
        MEDUSA_LAUNCH("rmsnorm_rows", rmsnorm_rows_kernel<bf16_t>, dim3(R), dim3(256), 0, s, (const bf16_t*)x, H,
                      eps, 1, n);
    else
        MEDUSA_LAUNCH("rmsnorm_rows", rmsnorm_rows_kernel<float>, dim3(R), dim3(256), 0, s, (const float*)x, H,
                      eps, 0, n);
    for (int r0 = 0; r0 < R; r0 += 8) {
        const int nb = R - r0 < 8 ? R - r0 : 8;
        launch_vocab_topk(n + (size_t)r0 * H, lm_head, nb, H, V, 1, 1, bf16, logits ? logits + (size_t)r0 * V : nullptr,
                          greedy + r0, gval + r0, cv, ci, s);
    }
}

}  // namespace medusa
