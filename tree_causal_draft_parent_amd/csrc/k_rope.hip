// k_rope.hip -- rotary position embedding of the draft-tree nodes' queries
// and keys at their tree positions.
//
// The pages draft for Qwen3 target models (abstract), whose attention rotates
// queries and keys by position (rotary embedding, RoFormer).  A node's
// position is the prefix length plus its depth minus one: the positions of
// ordinary decoding along its branch.  Pairs are (j, j + D/2), as in the
// Qwen3 models, turned by pos * theta^(-2j/D).
//
// One workgroup per node: the D/2 angles are formed in fp64 from inverse
// frequencies computed on the host (positions reach tens of thousands of
// radians, where fp32 angles would be ~1e-3 rad off) and reduced modulo 2 pi
// in fp64; their fp32 cosines and sines go to LDS, and every query and key
// head of the node is rotated in place in fp32, 16 bytes per load.
#include <math.h>

#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeMaxHalf = 128;

struct RopeArgs {
    double inv_freq[kRopeMaxHalf];   // theta^(-2j/D), formed on the host in fp64
};

__device__ __forceinline__ float ld_elem(const float *p) { return *p; }
__device__ __forceinline__ float ld_elem(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void st_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ void st_elem(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }

// 16 bytes of a row: 8 bf16 or 4 fp32 values, widened to fp32
template <typename T> struct Pack;
template <> struct Pack<uint16_t> {
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
template <> struct Pack<float> {
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

// One workgroup per node.  Angle a = pos * inv_freq[j] in fp64, reduced to
// [-pi, pi] with a two-term 2*pi (Cody-Waite), then fp32 sine and cosine of
// the reduced angle (its fp32 rounding moves it by at most pi * 2^-24).
template <typename T>
__global__ __launch_bounds__(kRopeThreads) void k_tree_rope(T *__restrict__ q, T *__restrict__ k,
                                                            const int32_t *__restrict__ depth,
                                                            const int32_t *__restrict__ prefix_len,
                                                            int N, int Hq, int Hkv, int D,
                                                            int vec, RopeArgs ra) {
    __shared__ float cs[kRopeMaxHalf], sn[kRopeMaxHalf];
    const int64_t node = blockIdx.x;
    const int b = (int)(node / N);
    const int d = depth[node];
    if (d < 1) return;                         // bad row of the mask builder: unchanged
    const double pos = (double)prefix_len[b] + (double)d - 1.0;
    const int half = D / 2;
    for (int j = threadIdx.x; j < half; j += kRopeThreads) {
        const double a = pos * ra.inv_freq[j];
        const double kq = rint(a * 0.15915494309189535);          // a / (2 pi)
        double r = fma(-kq, 6.283185307179586, a);                 // 2 pi, high part
        r = fma(-kq, 2.4492935982947064e-16, r);                   // 2 pi, low part
        float sr, cr;
        sincosf((float)r, &sr, &cr);
        cs[j] = cr;
        sn[j] = sr;
    }
    __syncthreads();
    const int H = Hq + (k ? Hkv : 0);
    constexpr int G = Pack<T>::n;
    if (vec) {
        // 16-byte groups (whole groups per half row, rows 16-byte aligned):
        // task = (head, group of G pairs); a thread's loads are issued before
        // its rotations
        const int gph = half / G, tasks = H * gph;
        for (int t0 = threadIdx.x; t0 < tasks; t0 += 2 * kRopeThreads) {
            float x0[2][G], x1[2][G];
            T *row[2];
            int j0[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = min(t0 + u * kRopeThreads, tasks - 1);
                const int h = t / gph;
                j0[u] = (t % gph) * G;
                row[u] = h < Hq ? q + (node * Hq + h) * D : k + (node * Hkv + (h - Hq)) * D;
                Pack<T>::load(row[u] + j0[u], x0[u]);
                Pack<T>::load(row[u] + j0[u] + half, x1[u]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (t0 + u * kRopeThreads >= tasks) continue;
                float y0[G], y1[G];
#pragma unroll
                for (int e = 0; e < G; ++e) {
                    const float c = cs[j0[u] + e], s = sn[j0[u] + e];
                    y0[e] = x0[u][e] * c - x1[u][e] * s;
                    y1[e] = x1[u][e] * c + x0[u][e] * s;
                }
                Pack<T>::store(row[u] + j0[u], y0);
                Pack<T>::store(row[u] + j0[u] + half, y1);
            }
        }
        return;
    }
    // other head dims: one pair a thread
    const int pq = Hq * half, pall = H * half;
    for (int p = threadIdx.x; p < pall; p += kRopeThreads) {
        T *row;
        int j;
        if (p < pq) {
            row = q + (node * Hq + p / half) * D;
            j = p % half;
        } else {
            const int pp = p - pq;
            row = k + (node * Hkv + pp / half) * D;
            j = pp % half;
        }
        const float x0 = ld_elem(row + j), x1 = ld_elem(row + j + half);
        const float c = cs[j], s = sn[j];
        st_elem(row + j, x0 * c - x1 * s);
        st_elem(row + j + half, x1 * c + x0 * s);
    }
}

}  // namespace

hipError_t launch_tree_rope(void *q, void *k, const int32_t *depth, const int32_t *prefix_len,
                            int B, int N, int Hq, int Hkv, int D, double theta, jf_dtype dtype,
                            hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)B * N));
    // 16-byte groups need whole groups per half row and 16-byte aligned rows
    const int G = dtype == JF_BF16 ? 8 : 4;
    const int vec = (D / 2) % G == 0 && (uintptr_t)q % 16 == 0 && (!k || (uintptr_t)k % 16 == 0);
    RopeArgs ra;
    for (int j = 0; j < kRopeMaxHalf; ++j)
        ra.inv_freq[j] = j < D / 2 ? pow(theta, -2.0 * (double)j / (double)D) : 0.0;
    if (dtype == JF_BF16)
        hipLaunchKernelGGL(k_tree_rope<uint16_t>, grid, dim3(kRopeThreads), 0, s, (uint16_t *)q,
                           (uint16_t *)k, depth, prefix_len, N, Hq, Hkv, D, vec, ra);
    else
        hipLaunchKernelGGL(k_tree_rope<float>, grid, dim3(kRopeThreads), 0, s, (float *)q,
                           (float *)k, depth, prefix_len, N, Hq, Hkv, D, vec, ra);
    return hipGetLastError();
}

}  // namespace jf
