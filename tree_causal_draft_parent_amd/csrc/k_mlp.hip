// k_mlp.hip -- gated MLP activation of the draft layer.
//
// The Qwen3 models the pages draft for (abstract) gate their MLP with SiLU:
//     y[m][c] = silu(gu[m][c]) * gu[m][I + c],  silu(g) = g / (1 + exp(-g)),
// with the gate projection in the first I columns of gu and the up
// projection in the last I (one projection call with the two weights
// stacked).  Elementwise and HBM-bound: a grid-stride loop over 16-byte
// groups of outputs (8 bf16 or 4 fp32) when the shapes allow it, else over
// single elements; fp32 arithmetic, bf16 storage rounded to nearest even.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kMlpThreads = 256;

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__device__ __forceinline__ float ldm(const float *p) { return *p; }
__device__ __forceinline__ float ldm(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void stm(float *p, float v) { *p = v; }
__device__ __forceinline__ void stm(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }

template <typename T> struct MPack;
template <> struct MPack<uint16_t> {
    static constexpr int n = 8;
    static __device__ __forceinline__ void load(const uint16_t *p, float *x) {
        const u32x4 v = *(const u32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(v[i] << 16);
            x[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float *x) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        *(u32x4 *)p = v;
    }
};
template <> struct MPack<float> {
    static constexpr int n = 4;
    static __device__ __forceinline__ void load(const float *p, float *x) {
        const f32x4 v = *(const f32x4 *)p;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = v[i];
    }
    static __device__ __forceinline__ void store(float *p, const float *x) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = x[i];
        *(f32x4 *)p = v;
    }
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kMlpThreads) void k_swiglu(const T *__restrict__ gu, int64_t M, int64_t I,
                                                        int64_t ld, T *__restrict__ y) {
    constexpr int G = VEC ? MPack<T>::n : 1;
    const int64_t per_row = I / G;
    const int64_t total = M * per_row;
    for (int64_t t = (int64_t)blockIdx.x * kMlpThreads + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kMlpThreads) {
        const int64_t m = t / per_row, c = (t % per_row) * G;
        const T *row = gu + m * ld;
        if constexpr (VEC) {
            float g[G], u[G];
            MPack<T>::load(row + c, g);
            MPack<T>::load(row + I + c, u);
#pragma unroll
            for (int e = 0; e < G; ++e) g[e] = silu_mul(g[e], u[e]);
            MPack<T>::store(y + m * I + c, g);
        } else {
            stm(y + m * I + c, silu_mul(ldm(row + c), ldm(row + I + c)));
        }
    }
}

template <typename T, bool VEC>
void launch_swiglu_t(const T *gu, int64_t M, int64_t I, int64_t ld, T *y, hipStream_t s) {
    constexpr int G = VEC ? MPack<T>::n : 1;
    const int64_t total = M * (I / G);
    int64_t blocks = (total + kMlpThreads - 1) / kMlpThreads;
    const int64_t cap = (int64_t)num_cus() * 16;           // grid-stride beyond this
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL((k_swiglu<T, VEC>), dim3((unsigned)blocks), dim3(kMlpThreads), 0, s, gu, M, I,
                       ld, y);
}

}  // namespace

hipError_t launch_swiglu(const void *gu, int64_t M, int64_t I, int64_t ld, jf_dtype dtype, void *y,
                         hipStream_t s) {
    const int G = dtype == JF_BF16 ? 8 : 4;
    const bool vec = I % G == 0 && ld % G == 0 && (uintptr_t)gu % 16 == 0 && (uintptr_t)y % 16 == 0;
    if (dtype == JF_BF16) {
        if (vec) launch_swiglu_t<uint16_t, true>((const uint16_t *)gu, M, I, ld, (uint16_t *)y, s);
        else launch_swiglu_t<uint16_t, false>((const uint16_t *)gu, M, I, ld, (uint16_t *)y, s);
    } else {
        if (vec) launch_swiglu_t<float, true>((const float *)gu, M, I, ld, (float *)y, s);
        else launch_swiglu_t<float, false>((const float *)gu, M, I, ld, (float *)y, s);
    }
    return hipGetLastError();
}

}  // namespace jf
