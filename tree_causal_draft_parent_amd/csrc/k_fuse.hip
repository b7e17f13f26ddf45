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
// bf16 path: output tiles of 256x128 (M >= 192: every weight is read once;
// eight waves, two per SIMD so that one covers the other's LDS and barrier
// stalls), 128x128 (four waves) or, for at most 32 rows, 32x128 (four waves
// side by side along N, a weight stream with a 6-deep ring), 64-deep K steps,
// each wave owning 64x64 (32x32 for 32-row tiles) of the tile as 32x32
// blocks of v_mfma_f32_32x32x16_bf16.  A and B tiles go from
// HBM straight into a 3-stage (256-row tiles) or 4-stage LDS ring with
// buffer_load ... lds (no registers); one copy fills 1 KiB = 8 K-contiguous rows
// (rows n, n+T/8, ... of a T-row tile) and 16-byte block padding keeps the
// 16-byte operand reads conflict-free.  Per-lane row offsets are computed once;
// the K position rides in the scalar offset.  When the output has fewer tiles
// than half the GPU's compute units, K is split; the slices write fp32
// partials in the accumulators' own layout (16 bytes a lane) and a second
// kernel sums them in slice order.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kBN = 128, kBK = 64;
constexpr int kRowG = kBK * 2;           // bytes per tile row (64 bf16)
constexpr int kBlkG = 8 * kRowG + 16;    // LDS block: 8 rows + pad
constexpr int kMaxLayers = 8;
constexpr int kGroupM = 4;              // m tiles per group of the item order
constexpr uint32_t kOobRow = 0xf0000000u; // past every buffer even after adding the K offset

struct FuseArgs {
    const uint16_t *x[kMaxLayers];
    const uint16_t *w;
    void *y;
    float *part;
    int64_t M, N, H_in, ldx, K;
    int64_t k_per_split;
    uint32_t x_bytes, w_bytes;
    int out_bf16;
    int split_k;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ void copy16s(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff,
                                        uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}

template <int BM>
struct Cfg {
    static constexpr int kStages = BM == 256 ? 3 : (BM == 128 ? 4 : 6);   // copy ring depth (LDS <= 150 KiB)
    static constexpr int kWaves = BM == 256 ? 8 : 4;    // 256-row tiles: two waves per SIMD
    static constexpr int kANb = BM / 8;             // LDS blocks of the A tile
    static constexpr int kBNb = kBN / 8;            // 16
    static constexpr int kATile = kANb * kBlkG;
    static constexpr int kBTile = kBNb * kBlkG;
    static constexpr int kStage = kATile + kBTile;
    static constexpr int WM = BM == 256 ? 4 : (BM == 128 ? 2 : 1);   // waves along M
    static constexpr int WN = kWaves / WM;          // waves along N
    static constexpr int TM = BM / WM / 32;         // 32x32 blocks per wave along M
    static constexpr int TN = kBN / WN / 32;        // ... along N
    static constexpr int kACopies = kANb / kWaves;  // copies per wave per K step
    static constexpr int kBCopies = kBNb / kWaves;
};

// LDS byte offset of row r of a tile with nb blocks
__device__ __forceinline__ int g_lds(int r, int nb) { return (r % nb) * kBlkG + (r / nb) * kRowG; }

template <int BM>
__global__ __launch_bounds__(Cfg<BM>::kWaves * kWave) void k_fuse_gemm_bf16(FuseArgs f) {
    typedef Cfg<BM> C;
    __shared__ __attribute__((aligned(1024))) char ring[C::kStages][C::kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int wm = wave / C::WN, wn = wave % C::WN;

    const int total = f.tiles_m * f.tiles_n * f.split_k;
    const int item = xcd_remap(blockIdx.x, total);
    // Grouped order inside a K slice: groups of up to four m tiles, the n tiles
    // of a group in turn, the m tiles of a group fastest.  An XCD's contiguous
    // range of items is then a block of m x n tiles that share A rows and
    // weight rows in its L2 (with one m tile this is plain n-tile order).
    const int per_slice = f.tiles_m * f.tiles_n;
    const int sk = item / per_slice;
    const int t = item % per_slice;
    const int group = t / (kGroupM * f.tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(f.tiles_m - first_m, kGroupM);
    const int tin = t % (kGroupM * f.tiles_n);
    const int tm = first_m + tin % gm;
    const int tn = tin / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * kBN;
    const int64_t kb = (int64_t)sk * f.k_per_split;
    const int64_t ke = min(f.K, kb + f.k_per_split);
    const int nk = (int)((ke - kb) / kBK);

    // per-lane row offsets of this wave's copies (K-step independent)
    const int sub = lane >> 3, ch = lane & 7;
    uint32_t aoff[C::kACopies], boff[C::kBCopies];
#pragma unroll
    for (int i = 0; i < C::kACopies; ++i) {
        const int n = wave * C::kACopies + i;          // block
        const int64_t m = m0 + n + C::kANb * sub;       // row
        aoff[i] = m < f.M ? (uint32_t)((m * f.ldx + ch * 8) * 2) : kOobRow;
    }
#pragma unroll
    for (int i = 0; i < C::kBCopies; ++i) {
        const int n = wave * C::kBCopies + i;
        const int64_t nn = n0 + n + C::kBNb * sub;
        boff[i] = nn < f.N ? (uint32_t)((nn * f.K + ch * 8) * 2) : kOobRow;
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.w, f.w_bytes);

    // Copies are issued in K order, so the layer of the next step and the
    // offset inside it advance by one K step at a time (H_in is a multiple
    // of the K step); no division per step.
    int ilayer = (int)(kb / f.H_in);
    uint32_t ioff = (uint32_t)((kb - (int64_t)ilayer * f.H_in) * 2);   // bytes into the layer's rows
    uint32_t ikk = (uint32_t)(kb * 2);                                  // bytes into the weight rows
    const uint32_t layer_bytes = (uint32_t)(f.H_in * 2);
    __amdgpu_buffer_rsrc_t rx = make_rsrc(f.x[ilayer], f.x_bytes);
    auto issue = [&](uint32_t dst) {
        const uint32_t da = __builtin_amdgcn_readfirstlane(dst + wave * C::kACopies * kBlkG);
        const uint32_t db = __builtin_amdgcn_readfirstlane(dst + C::kATile + wave * C::kBCopies * kBlkG);
#pragma unroll
        for (int i = 0; i < C::kACopies; ++i) copy16s(rx, da + i * kBlkG, aoff[i], ioff);
#pragma unroll
        for (int i = 0; i < C::kBCopies; ++i) copy16s(rw, db + i * kBlkG, boff[i], ikk);
        ikk += kBK * 2;
        ioff += kBK * 2;
        if (ioff == layer_bytes && ilayer + 1 < kMaxLayers) {
            ioff = 0;
            ++ilayer;
            rx = make_rsrc(f.x[ilayer], f.x_bytes);
        }
    };

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // operand bases: A rows wm*(BM/WM) + i*32 + l32, B rows wn*(128/WN) + j*32 + l32
    const int a_lane = g_lds(wm * (BM / C::WM) + l32, C::kANb) + half * 16;
    const int b_lane = C::kATile + g_lds(wn * (kBN / C::WN) + l32, C::kBNb) + half * 16;
    auto rd = [&](const lds_t *st, int t, bf16x8 *av, bf16x8 *bv) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            av[i] = *(const __attribute__((address_space(3))) bf16x8 *)(st + a_lane + (i * 32 / C::kANb) * kRowG + t * 32);
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            bv[j] = *(const __attribute__((address_space(3))) bf16x8 *)(st + b_lane + (j * 32 / C::kBNb) * kRowG + t * 32);
    };
    auto mma = [&](const bf16x8 *av, const bf16x8 *bv) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Copy ring: step i lives in stage i % NS; steps i+1 .. i+NS-1 are in
    // flight while step i is multiplied.  Each wave issues kCopies copies a
    // step, so "step i has landed" is "at most kCopies * (steps issued after
    // i) copies outstanding".  The wait and barrier for step i+1 sit before
    // the last MFMA group of step i, and the first operands of step i+1 are
    // read while that group runs; a wave issues the copies of step i+NS-1
    // (into the stage of step i-1, which every wave finished reading before
    // that barrier) after the first MFMA group of step i.
    constexpr int NS = C::kStages;
    static_assert(NS >= 3, "the ring needs three stages or more");
    static_assert(kBK / 16 == 4, "four 16-deep MFMA groups per K step");
    constexpr int kCopies = C::kACopies + C::kBCopies;
    const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_t *)&ring[0][0];
    auto wait_step = [&](int i) {
        const int ahead = min(NS - 2, nk - 1 - i);   // steps issued after i and still in flight
        if (ahead >= 4) ring_barrier<(NS >= 6 ? 4 : 0) * kCopies>();
        else if (ahead == 3) ring_barrier<(NS >= 5 ? 3 : 0) * kCopies>();
        else if (ahead == 2) ring_barrier<2 * kCopies>();
        else if (ahead == 1) ring_barrier<kCopies>();
        else ring_barrier<0>();
    };
    auto stage = [&](int i) { return (const lds_t *)&ring[i % NS][0]; };
    bf16x8 a0[C::TM], b0[C::TN], a1[C::TM], b1[C::TN];
    for (int i = 0; i < NS - 1 && i < nk; ++i) issue(ring0 + i * C::kStage);
    if (nk > 0) {
        wait_step(0);
        rd(stage(0), 0, a0, b0);
    }
    for (int i = 0; i < nk; ++i) {
        const lds_t *st = stage(i);
        rd(st, 1, a1, b1);
        mma(a0, b0);
        if (i + NS - 1 < nk) issue(ring0 + ((i + NS - 1) % NS) * C::kStage);
        rd(st, 2, a0, b0);
        mma(a1, b1);
        rd(st, 3, a1, b1);
        mma(a0, b0);
        if (i + 1 < nk) {
            wait_step(i + 1);
            rd(stage(i + 1), 0, a0, b0);
        }
        mma(a1, b1);
    }

    // lane holds rows (r/4)*8 + half*4 + r%4 of each 32x32 block, column l32
    if (f.split_k > 1) {
        // Split-K partials keep the accumulators' own layout: tile by tile,
        // wave by wave, each 32x32 block as 1024 floats ordered [r/4][lane][r%4].
        // Every store is then 16 bytes a lane and 1 KiB contiguous a wave
        // (k_fuse_reduce undoes the layout).
        float *blk = f.part + ((int64_t)sk * f.tiles_m * f.tiles_n + (int64_t)tm * f.tiles_n + tn) * (BM * kBN)
                     + (int64_t)wave * (C::TM * C::TN * 1024) + lane * 4;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                    *(f32x4 *)(blk + (i * C::TN + j) * 1024 + q * 256) = v;
                }
        return;
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int64_t n = n0 + wn * (kBN / C::WN) + j * 32 + l32;
            if (n >= f.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * (BM / C::WM) + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (m >= f.M) continue;
                const float v = acc[i][j][r];
                if (f.out_bf16) {
                    ((uint16_t *)f.y)[m * f.N + n] = (uint16_t)f32_to_bf16_rne(v);
                } else {
                    ((float *)f.y)[m * f.N + n] = v;
                }
            }
        }
}

// y = sum over K slices of the fp32 partials (in slice order), converted to
// the output type.  A thread takes one 16-byte chunk of the partial layout
// (four rows of one column of a 32x32 block: chunk c of a BM x 128 tile is
// block c / 256, row group (c / 64) % 4, lane c % 64), so every load is 1 KiB
// contiguous a wave; four slices are loaded per round so that a thread's
// loads overlap.  Rows past M and columns past N are computed and dropped.
template <int BM>
__global__ __launch_bounds__(256) void k_fuse_reduce(const float *__restrict__ part, int split_k,
                                                     int64_t M, int64_t N, int tiles_n, int64_t chunks,
                                                     void *y, int out_bf16) {
    typedef Cfg<BM> C;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t slice = chunks * 4;   // floats a slice
    const float *p = part + c * 4;
    f32x4 s = *(const f32x4 *)p;
    int k = 1;
    for (; k + 4 <= split_k; k += 4) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const f32x4 *)(p + (int64_t)(k + u) * slice);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s[0] += v[u][0]; s[1] += v[u][1]; s[2] += v[u][2]; s[3] += v[u][3];
        }
    }
    for (; k < split_k; ++k) {
        const f32x4 v = *(const f32x4 *)(p + (int64_t)k * slice);
        s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    constexpr int kTileChunks = BM * kBN / 4;
    const int64_t tile = c / kTileChunks;
    const int rem = (int)(c % kTileChunks);
    const int blk = rem >> 8, q = (rem >> 6) & 3, lane = rem & 63;
    const int wave = blk / (C::TM * C::TN), i = (blk / C::TN) % C::TM, j = blk % C::TN;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
    const int64_t m0 = tm * BM + wm * (BM / C::WM) + i * 32 + q * 8 + (lane >> 5) * 4;
    const int64_t n = tn * kBN + wn * (kBN / C::WN) + j * 32 + (lane & 31);
    if (n >= N) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + r;
        if (m >= M) break;
        if (out_bf16) ((uint16_t *)y)[m * N + n] = (uint16_t)f32_to_bf16_rne(s[r]);
        else ((float *)y)[m * N + n] = s[r];
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

void plan_fuse(FusePlan &p, int64_t M, int64_t H_in, int k, int64_t H_out, jf_dtype in_dtype,
               int cus) {
    p.M = M;
    p.H_in = H_in;
    p.H_out = H_out;
    p.k = k;
    p.bm = M >= 192 ? 256 : (M > 32 ? 128 : 32);      // 32-row tiles: a weight stream for few rows
    p.bn = kBN;
    const int64_t K = (int64_t)k * H_in;
    if (in_dtype != JF_BF16) {
        p.split_k = 1;
        p.k_per_split = K;
        return;
    }
    const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((H_out + kBN - 1) / kBN);
    // one workgroup per compute unit of the budget (all units unless a caller
    // leaves some to work on another stream)
    const int64_t target = cus > 0 && cus < num_cus() ? (int64_t)cus : (int64_t)num_cus();
    int64_t s = (target + tiles - 1) / tiles;
    // With more than half a wave of tiles a split cannot shorten the call: two
    // slices give two waves of half-length workgroups (the same total) plus
    // the partials' write and read back.
    if (2 * tiles > target) s = 1;
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
    // whole tiles: the partials keep the GEMM tiles' layout
    const size_t tiles = (size_t)((p.M + p.bm - 1) / p.bm) * (size_t)((p.H_out + kBN - 1) / kBN);
    return (size_t)p.split_k * tiles * p.bm * kBN * sizeof(float);
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
    f.x_bytes = (uint32_t)(((p.M - 1) * ldx + p.H_in) * 2);
    f.w_bytes = (uint32_t)(p.H_out * f.K * 2);
    f.out_bf16 = out_dtype == JF_BF16;
    f.split_k = p.split_k;
    f.tiles_m = (int)((p.M + p.bm - 1) / p.bm);
    f.tiles_n = (int)((p.H_out + kBN - 1) / kBN);
    const unsigned grid = (unsigned)(f.tiles_m * f.tiles_n * f.split_k);
    if (p.bm == 256)
        hipLaunchKernelGGL(k_fuse_gemm_bf16<256>, dim3(grid), dim3(Cfg<256>::kWaves * kWave), 0, s, f);
    else if (p.bm == 128)
        hipLaunchKernelGGL(k_fuse_gemm_bf16<128>, dim3(grid), dim3(Cfg<128>::kWaves * kWave), 0, s, f);
    else
        hipLaunchKernelGGL(k_fuse_gemm_bf16<32>, dim3(grid), dim3(Cfg<32>::kWaves * kWave), 0, s, f);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split_k <= 1) return e;
    const int64_t chunks = (int64_t)f.tiles_m * f.tiles_n * p.bm * kBN / 4;
    const unsigned g2 = (unsigned)((chunks + 255) / 256);
#define JF_REDUCE(BMV)                                                                              \
    hipLaunchKernelGGL(k_fuse_reduce<BMV>, dim3(g2), dim3(256), 0, s, (const float *)workspace,      \
                       p.split_k, p.M, p.H_out, f.tiles_n, chunks, y, (int)f.out_bf16)
    if (p.bm == 256) JF_REDUCE(256);
    else if (p.bm == 128) JF_REDUCE(128);
    else JF_REDUCE(32);
#undef JF_REDUCE
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
