// k_norm.hip -- root-mean-square normalisation of rows.
//
// The Qwen3 models the pages draft for (abstract) normalise the hidden state
// of a layer, and per head its queries and keys, by the root mean square:
//     y[r][c] = x[r][c] / sqrt(mean_c(x[r][c]^2) + eps) * w[c].
// One wavefront per row: the sum of squares is accumulated in fp64 (so the
// result does not depend on the row length's rounding), the inverse root is
// rounded once to fp32, and a second pass over the row (a cache hit) writes
// x * inv * w in fp32, rounded to the storage type.  16-byte loads when the
// row length, stride and pointers allow them.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRowsPerBlock = kNormThreads / kWave;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void st1(float *p, float v) { *p = v; }
__device__ __forceinline__ void st1(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }

template <typename T> struct NPack;
template <> struct NPack<uint16_t> {
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
template <> struct NPack<float> {
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

template <typename T>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const T *__restrict__ x, int64_t rows,
                                                          int H, int64_t ldx, const T *__restrict__ w,
                                                          float eps, T *y, int vec) {
    const int64_t row = (int64_t)blockIdx.x * kNormRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;                      // the whole wavefront leaves
    const int lane = threadIdx.x & 63;
    const T *xr = x + row * ldx;
    T *yr = y + row * (int64_t)H;
    constexpr int G = NPack<T>::n;
    double ss = 0.0;
    if (vec) {
        for (int c = lane * G; c < H; c += kWave * G) {
            float v[G];
            NPack<T>::load(xr + c, v);
#pragma unroll
            for (int e = 0; e < G; ++e) ss = fma((double)v[e], (double)v[e], ss);
        }
    } else {
        for (int c = lane; c < H; c += kWave) {
            const double v = (double)ld1(xr + c);
            ss = fma(v, v, ss);
        }
    }
    ss = wave_sum_f64(ss);
    const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
    if (vec) {
        for (int c = lane * G; c < H; c += kWave * G) {
            float v[G], wv[G];
            NPack<T>::load(xr + c, v);
            if (w) NPack<T>::load(w + c, wv);
#pragma unroll
            for (int e = 0; e < G; ++e) v[e] = w ? (v[e] * inv) * wv[e] : v[e] * inv;
            NPack<T>::store(yr + c, v);
        }
    } else {
        for (int c = lane; c < H; c += kWave) {
            const float v = ld1(xr + c) * inv;
            st1(yr + c, w ? v * ld1(w + c) : v);
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void *x, int64_t rows, int H, int64_t ldx, const void *w, float eps,
                          jf_dtype dtype, void *y, hipStream_t s) {
    const int G = dtype == JF_BF16 ? 8 : 4;
    const int vec = H % G == 0 && ldx % G == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0 &&
                    (!w || (uintptr_t)w % 16 == 0);
    const dim3 grid((unsigned)((rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock));
    if (dtype == JF_BF16)
        hipLaunchKernelGGL(k_rmsnorm<uint16_t>, grid, dim3(kNormThreads), 0, s, (const uint16_t *)x,
                           rows, H, ldx, (const uint16_t *)w, eps, (uint16_t *)y, vec);
    else
        hipLaunchKernelGGL(k_rmsnorm<float>, grid, dim3(kNormThreads), 0, s, (const float *)x, rows,
                           H, ldx, (const float *)w, eps, (float *)y, vec);
    return hipGetLastError();
}

}  // namespace jf
