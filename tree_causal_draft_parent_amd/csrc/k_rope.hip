// k_rope.hip -- rotary position embedding of the draft-tree nodes' queries
// and keys at their tree positions.
//
// The pages draft for Qwen3 target models (abstract), whose attention rotates
// queries and keys by position (rotary embedding, RoFormer).  A node's
// position is the prefix length plus its depth minus one: the positions of
// ordinary decoding along its branch.  Pairs are (j, j + D/2), as in the
// Qwen3 models, turned by pos * theta^(-2j/D).
//
// One workgroup per node: the D/2 angles are formed in fp64 (positions reach
// tens of thousands of radians, where fp32 would lose ~1e-3 rad), their
// cosines and sines rounded to fp32 into LDS, and every query and key head of
// the node is rotated in place in fp32.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeMaxHalf = 128;

__device__ __forceinline__ float ld_elem(const float *p) { return *p; }
__device__ __forceinline__ float ld_elem(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void st_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ void st_elem(uint16_t *p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void k_tree_rope(T *__restrict__ q, T *__restrict__ k,
                                                            const int32_t *__restrict__ depth,
                                                            const int32_t *__restrict__ prefix_len,
                                                            int N, int Hq, int Hkv, int D,
                                                            double theta) {
    __shared__ float cs[kRopeMaxHalf], sn[kRopeMaxHalf];
    const int64_t node = blockIdx.x;
    const int b = (int)(node / N);
    const int d = depth[node];
    if (d < 1) return;                         // bad row of the mask builder: unchanged
    const double pos = (double)prefix_len[b] + (double)d - 1.0;
    const int half = D / 2;
    for (int j = threadIdx.x; j < half; j += kRopeThreads) {
        const double a = pos * pow(theta, -2.0 * (double)j / (double)D);
        cs[j] = (float)cos(a);
        sn[j] = (float)sin(a);
    }
    __syncthreads();
    const int pq = Hq * half, pall = (Hq + (k ? Hkv : 0)) * half;
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
    if (dtype == JF_BF16)
        hipLaunchKernelGGL(k_tree_rope<uint16_t>, grid, dim3(kRopeThreads), 0, s, (uint16_t *)q,
                           (uint16_t *)k, depth, prefix_len, N, Hq, Hkv, D, theta);
    else
        hipLaunchKernelGGL(k_tree_rope<float>, grid, dim3(kRopeThreads), 0, s, (float *)q,
                           (float *)k, depth, prefix_len, N, Hq, Hkv, D, theta);
    return hipGetLastError();
}

}  // namespace jf
