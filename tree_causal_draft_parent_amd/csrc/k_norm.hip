// k_norm.hip -- root-mean-square normalisation of rows.
//
// The Qwen3 models the pages draft for (abstract) normalise the hidden state
// of a layer, and per head its queries and keys, by the root mean square:
//     y[r][c] = x[r][c] / sqrt(mean_c(x[r][c]^2) + eps) * w[c].
// The sum of squares is accumulated in fp64 (so the result does not depend on
// the row length's rounding), the inverse root is rounded once to fp32, and
// x * inv * w is formed in fp32, rounded to the storage type.  Rows of whole
// 16-byte vectors (stride and pointers aligned) are held in registers by a
// group of lanes (several short rows a wavefront); other rows take one
// wavefront and two passes.
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

// Vector path: lanes work in groups of LPR (a power of two, <= 64); a group
// owns one row and holds it in registers (NV 16-byte vectors a lane, at most
// kNormMaxV), so the row is read once.  Scalar path: one row a wavefront, two
// passes over the row.
constexpr int kNormMaxV = 16;

template <typename T>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm_vec(const T *__restrict__ x, int64_t rows,
                                                              int H, int64_t ldx,
                                                              const T *__restrict__ w, float eps,
                                                              T *y, int lpr_log2) {
    constexpr int G = NPack<T>::n;
    const int lpr = 1 << lpr_log2;
    const int lane = threadIdx.x & 63;
    const int grp = lane >> lpr_log2, gl = lane & (lpr - 1);
    const int64_t row = ((int64_t)blockIdx.x * kNormRowsPerBlock + (threadIdx.x >> 6)) * (kWave / lpr) + grp;
    const bool live = row < rows;
    const T *xr = x + (live ? row : 0) * ldx;
    float v[kNormMaxV][G];
#pragma unroll
    for (int i = 0; i < kNormMaxV; ++i) {
        const int c = (i * lpr + gl) * G;
        if (c < H) NPack<T>::load(xr + c, v[i]);
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kNormMaxV; ++i) {
        const int c = (i * lpr + gl) * G;
        if (c < H) {
#pragma unroll
            for (int e = 0; e < G; ++e) ss = fma((double)v[i][e], (double)v[i][e], ss);
        }
    }
    for (int m = lpr >> 1; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, kWave);   // within the group
    const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
    if (!live) return;
    T *yr = y + row * (int64_t)H;
#pragma unroll
    for (int i = 0; i < kNormMaxV; ++i) {
        const int c = (i * lpr + gl) * G;
        if (c < H) {
            float wv[G];
            if (w) NPack<T>::load(w + c, wv);
#pragma unroll
            for (int e = 0; e < G; ++e) v[i][e] = w ? (v[i][e] * inv) * wv[e] : v[i][e] * inv;
            NPack<T>::store(yr + c, v[i]);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const T *__restrict__ x, int64_t rows,
                                                          int H, int64_t ldx, const T *__restrict__ w,
                                                          float eps, T *y) {
    const int64_t row = (int64_t)blockIdx.x * kNormRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;                      // the whole wavefront leaves
    const int lane = threadIdx.x & 63;
    const T *xr = x + row * ldx;
    T *yr = y + row * (int64_t)H;
    double ss = 0.0;
    for (int c = lane; c < H; c += kWave) {
        const double v = (double)ld1(xr + c);
        ss = fma(v, v, ss);
    }
    ss = wave_sum_f64(ss);
    const float inv = (float)(1.0 / sqrt(ss / (double)H + (double)eps));
    for (int c = lane; c < H; c += kWave) {
        const float v = ld1(xr + c) * inv;
        st1(yr + c, w ? v * ld1(w + c) : v);
    }
}

}  // namespace

hipError_t launch_rmsnorm(const void *x, int64_t rows, int H, int64_t ldx, const void *w, float eps,
                          jf_dtype dtype, void *y, hipStream_t s) {
    const int G = dtype == JF_BF16 ? 8 : 4;
    const bool aligned16 = (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0 &&
                           (!w || (uintptr_t)w % 16 == 0);
    const int nvec = H / G;                       // 16-byte vectors a row
    // lanes a row: the largest power of two <= min(64, nvec); the row must then
    // fit in kNormMaxV vectors a lane
    int lg = 0;
    while (lg < 6 && (2 << lg) <= nvec) ++lg;
    const bool vec = H % G == 0 && ldx % G == 0 && aligned16 && nvec >= 1 &&
                     (nvec + (1 << lg) - 1) / (1 << lg) <= kNormMaxV;
    if (vec) {
        const int64_t per_block = (int64_t)kNormRowsPerBlock * (kWave >> lg);
        const dim3 grid((unsigned)((rows + per_block - 1) / per_block));
        if (dtype == JF_BF16)
            hipLaunchKernelGGL(k_rmsnorm_vec<uint16_t>, grid, dim3(kNormThreads), 0, s,
                               (const uint16_t *)x, rows, H, ldx, (const uint16_t *)w, eps,
                               (uint16_t *)y, lg);
        else
            hipLaunchKernelGGL(k_rmsnorm_vec<float>, grid, dim3(kNormThreads), 0, s, (const float *)x,
                               rows, H, ldx, (const float *)w, eps, (float *)y, lg);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock));
    if (dtype == JF_BF16)
        hipLaunchKernelGGL(k_rmsnorm<uint16_t>, grid, dim3(kNormThreads), 0, s, (const uint16_t *)x,
                           rows, H, ldx, (const uint16_t *)w, eps, (uint16_t *)y);
    else
        hipLaunchKernelGGL(k_rmsnorm<float>, grid, dim3(kNormThreads), 0, s, (const float *)x, rows,
                           H, ldx, (const float *)w, eps, (float *)y);
    return hipGetLastError();
}

}  // namespace jf
