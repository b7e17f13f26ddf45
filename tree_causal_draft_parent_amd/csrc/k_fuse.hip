// k_fuse.hip -- projection of hidden states fused from several target layers.
//
// The draft head runs over hidden states "fused" from the frozen target model
// (abstract on every page; JetFlow blog page, "What JetFlow Does
// Differently"); the pages do not name the fusion operator.  Taken here:
// concatenate the k layers and apply one bias-free linear map,
//     y[m, o] = sum_l sum_c x_l[m, c] * w[o, l*H_in + c],
// i.e. an NT GEMM with K = k*H_in in which the A operand's K axis hops from one
// layer's tensor to the next every H_in columns (no concatenated copy).
//
// bf16 path: 128x128 output tiles, 64-deep K steps, four waves each owning a
// 64x64 quarter as 2x2 blocks of v_mfma_f32_32x32x16_bf16.  Both operands are
// K-contiguous in memory and in LDS (rows padded to avoid bank conflicts), so
// the MFMA operands are plain 16-byte LDS reads.  Tiles are prefetched into
// registers one K step ahead and double-buffered in LDS.  When the output has
// too few tiles to fill the GPU, K is split and the slices' fp32 partials are
// summed by a second kernel.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRowB = kBK * 2 + 16;      // bytes per LDS row (padded)
constexpr int kTileA = kBM * kRowB;
constexpr int kTileB = kBN * kRowB;
constexpr int kStageB = kTileA + kTileB;
constexpr int kMaxLayers = 8;

struct FuseArgs {
    const uint16_t *x[kMaxLayers];
    const uint16_t *w;
    void *y;
    float *part;
    int64_t M, N, H_in, ldx, K;
    int64_t k_per_split;
    int out_bf16;
    int split_k;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct GemmRegs {
    u32x4 a[4];
    u32x4 b[4];
};

__device__ __forceinline__ void gemm_load(const FuseArgs &f, int64_t m0, int64_t n0, int64_t kk0,
                                          int tid, GemmRegs &g) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int ch = tid & 7, rr = tid >> 3;
    const int layer = (int)(kk0 / f.H_in);
    const int64_t col = kk0 - (int64_t)layer * f.H_in + ch * 8;
    const uint16_t *xa = f.x[layer];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + rr + 32 * r;
        g.a[r] = m < f.M ? *(const u32x4 *)(xa + m * f.ldx + col) : zero;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + rr + 32 * r;
        g.b[r] = n < f.N ? *(const u32x4 *)(f.w + n * f.K + kk0 + ch * 8) : zero;
    }
}

__device__ __forceinline__ void gemm_store(char *stage, int tid, const GemmRegs &g) {
    const int ch = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *(u32x4 *)(stage + (rr + 32 * r) * kRowB + ch * 16) = g.a[r];
        *(u32x4 *)(stage + kTileA + (rr + 32 * r) * kRowB + ch * 16) = g.b[r];
    }
}

__global__ __launch_bounds__(256) void k_fuse_gemm_bf16(FuseArgs f) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kStageB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;

    const int total = f.tiles_m * f.tiles_n * f.split_k;
    const int item = xcd_remap(blockIdx.x, total);
    // tiles sharing a weight slab (same n tile) are adjacent
    const int tm = item % f.tiles_m;
    const int rest = item / f.tiles_m;
    const int tn = rest % f.tiles_n;
    const int sk = rest / f.tiles_n;
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    const int64_t kb = (int64_t)sk * f.k_per_split;
    const int64_t ke = min(f.K, kb + f.k_per_split);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    GemmRegs g;
    int buf = 0;
    if (kb < ke) {
        gemm_load(f, m0, n0, kb, tid, g);
        gemm_store(smem, tid, g);
    }
    __syncthreads();
    for (int64_t kk = kb; kk < ke; kk += kBK) {
        const bool more = kk + kBK < ke;
        if (more) gemm_load(f, m0, n0, kk + kBK, tid, g);
        const char *sa = smem + buf * kStageB;
        const char *sb = sa + kTileA;
#pragma unroll
        for (int t = 0; t < kBK / 16; ++t) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = *(const bf16x8 *)(sa + (wm * 64 + i * 32 + l32) * kRowB + t * 32 + half * 16);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *(const bf16x8 *)(sb + (wn * 64 + j * 32 + l32) * kRowB + t * 32 + half * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (more) gemm_store(smem + (buf ^ 1) * kStageB, tid, g);
        __syncthreads();
        buf ^= 1;
    }

    // lane holds rows (r/4)*8 + half*4 + r%4 of each 32x32 block, column l32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + j * 32 + l32;
            if (n >= f.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (m >= f.M) continue;
                const float v = acc[i][j][r];
                if (f.split_k > 1) {
                    f.part[((int64_t)sk * f.M + m) * f.N + n] = v;
                } else if (f.out_bf16) {
                    ((uint16_t *)f.y)[m * f.N + n] = (uint16_t)f32_to_bf16_rne(v);
                } else {
                    ((float *)f.y)[m * f.N + n] = v;
                }
            }
        }
}

// y = sum over K slices of the fp32 partials, converted to the output type.
__global__ __launch_bounds__(256) void k_fuse_reduce(const float *__restrict__ part, int split_k,
                                                     int64_t MN, void *y, int out_bf16) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    if (i + 4 <= MN) {
        f32x4 s = *(const f32x4 *)(part + i);
        for (int k = 1; k < split_k; ++k) {
            f32x4 v = *(const f32x4 *)(part + (int64_t)k * MN + i);
            s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
        }
        if (out_bf16) {
            u32x2 w;
            w[0] = pack_bf16x2(s[0], s[1]);
            w[1] = pack_bf16x2(s[2], s[3]);
            *(u32x2 *)((uint16_t *)y + i) = w;
        } else {
            *(f32x4 *)((float *)y + i) = s;
        }
    } else {
        for (int64_t e = i; e < MN; ++e) {
            float s = 0.f;
            for (int k = 0; k < split_k; ++k) s += part[(int64_t)k * MN + e];
            if (out_bf16) ((uint16_t *)y)[e] = (uint16_t)f32_to_bf16_rne(s);
            else ((float *)y)[e] = s;
        }
    }
}

// fp32 inputs: classic 16x16 LDS-tiled FMA GEMM (small problems).
struct FuseArgsF32 {
    const float *x[kMaxLayers];
    const float *w;
    float *y;
    int64_t M, N, H_in, ldx, K;
};

__global__ __launch_bounds__(256) void k_fuse_gemm_f32(FuseArgsF32 f) {
    __shared__ float As[16][17];
    __shared__ float Bs[16][17];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int64_t m = (int64_t)blockIdx.y * 16 + ty;
    const int64_t n = (int64_t)blockIdx.x * 16 + tx;
    const int64_t nb = (int64_t)blockIdx.x * 16 + ty;  // row of w this thread stages
    float acc = 0.f;
    for (int64_t k0 = 0; k0 < f.K; k0 += 16) {
        const int64_t ka = k0 + tx;
        float av = 0.f, bv = 0.f;
        if (m < f.M && ka < f.K) {
            const int layer = (int)(ka / f.H_in);
            av = f.x[layer][m * f.ldx + (ka - (int64_t)layer * f.H_in)];
        }
        if (nb < f.N && ka < f.K) bv = f.w[nb * f.K + ka];
        As[ty][tx] = av;
        Bs[ty][tx] = bv;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 16; ++c) acc = fmaf(As[ty][c], Bs[tx][c], acc);
        __syncthreads();
    }
    if (m < f.M && n < f.N) f.y[m * f.N + n] = acc;
}

}  // namespace

void plan_fuse(FusePlan &p, int64_t M, int64_t H_in, int k, int64_t H_out, jf_dtype in_dtype) {
    p.M = M;
    p.H_in = H_in;
    p.H_out = H_out;
    p.k = k;
    p.bm = kBM;
    p.bn = kBN;
    const int64_t K = (int64_t)k * H_in;
    if (in_dtype != JF_BF16) {
        p.split_k = 1;
        p.k_per_split = K;
        return;
    }
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((H_out + kBN - 1) / kBN);
    const int64_t target = 2 * (int64_t)num_cus();
    int64_t s = (target + tiles - 1) / tiles;
    const int64_t ksteps = K / kBK;
    int64_t max_s = ksteps / 8;  // at least eight K steps per slice
    if (max_s < 1) max_s = 1;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    int64_t per = (ksteps + s - 1) / s;
    p.k_per_split = per * kBK;
    p.split_k = (int)((ksteps + per - 1) / per);
}

size_t fuse_workspace_bytes(const FusePlan &p) {
    if (p.split_k <= 1) return 0;
    return (size_t)p.split_k * p.M * p.H_out * sizeof(float);
}

hipError_t launch_fuse_bf16(const FusePlan &p, const void *const *x, int64_t ldx, const void *w,
                            void *y, jf_dtype out_dtype, void *workspace, hipStream_t s) {
    FuseArgs f;
    for (int l = 0; l < kMaxLayers; ++l) f.x[l] = l < p.k ? (const uint16_t *)x[l] : nullptr;
    f.w = (const uint16_t *)w;
    f.y = y;
    f.part = (float *)workspace;
    f.M = p.M;
    f.N = p.H_out;
    f.H_in = p.H_in;
    f.ldx = ldx;
    f.K = (int64_t)p.k * p.H_in;
    f.k_per_split = p.k_per_split;
    f.out_bf16 = out_dtype == JF_BF16;
    f.split_k = p.split_k;
    f.tiles_m = (int)((p.M + kBM - 1) / kBM);
    f.tiles_n = (int)((p.H_out + kBN - 1) / kBN);
    const unsigned grid = (unsigned)(f.tiles_m * f.tiles_n * f.split_k);
    hipLaunchKernelGGL(k_fuse_gemm_bf16, dim3(grid), dim3(256), 0, s, f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split_k <= 1) return e;
    const int64_t MN = p.M * p.H_out;
    const unsigned g2 = (unsigned)(((MN + 3) / 4 + 255) / 256);
    hipLaunchKernelGGL(k_fuse_reduce, dim3(g2), dim3(256), 0, s, (const float *)workspace, p.split_k,
                       MN, y, (int)f.out_bf16);
    return hipGetLastError();
}

hipError_t launch_fuse_f32(const FusePlan &p, const void *const *x, int64_t ldx, const void *w,
                           float *y, hipStream_t s) {
    FuseArgsF32 f;
    for (int l = 0; l < kMaxLayers; ++l) f.x[l] = l < p.k ? (const float *)x[l] : nullptr;
    f.w = (const float *)w;
    f.y = y;
    f.M = p.M;
    f.N = p.H_out;
    f.H_in = p.H_in;
    f.ldx = ldx;
    f.K = (int64_t)p.k * p.H_in;
    dim3 grid((unsigned)((p.H_out + 15) / 16), (unsigned)((p.M + 15) / 16));
    hipLaunchKernelGGL(k_fuse_gemm_f32, grid, dim3(256), 0, s, f);
    return hipGetLastError();
}

}  // namespace jf
