// k_topk.hip -- per-node top-k of the draft logits and the row log-sum-exp.
//
// The draft tree is grown from each node's most likely next tokens, and a
// branch's probability is the product of per-node conditionals (JetFlow blog
// page, "What JetFlow Does Differently"): every node row needs its k best
// logits (value descending, ties by lower index) and its normaliser.
//
// The scan is HBM-bound (one pass over R x V logits).  Stage 1: one wavefront
// per (row, slice of the vocabulary).  Each lane streams 16-byte vectors; an
// element can only enter the top-k if it beats the wave's current k-th best
// (value, index) pair, so almost every element costs one compare.  Passing
// elements are compacted into a per-wave LDS buffer with ballot + mbcnt; when
// the buffer fills, the wave selects its k best keys (k rounds of a wave-wide
// max), raising the threshold.  The online (max, sum-exp) of the slice rides
// along.  Stage 2: one wavefront per row merges the slices' k-best lists and
// (max, sum-exp) pairs.
//
// Candidates are 64-bit keys: high word = order-preserving image of the fp32
// value (-0 folded onto +0), low word = ~index, so that a larger key is a
// better candidate and keys are unique within a row.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kT1Waves = 4;
constexpr int kCap = 512;     // candidate buffer entries per wave
constexpr int kUnroll = 4;    // 16-byte vectors in flight per lane
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t ordered_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ordered_to_float(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t make_key(float x, uint32_t idx) {
    return ((uint64_t)ordered_bits(x) << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, off);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Select the k best keys among buf[0..n); lanes 0..k-1 receive them in order.
// Returns the key held by this lane (0 for lanes >= min(k, n)).
__device__ uint64_t wave_select(const uint64_t *buf, int n, int k, int lane) {
    uint64_t mine = 0, prev = ~0ull;
    const int rounds = n < k ? n : k;
    for (int t = 0; t < rounds; ++t) {
        uint64_t best = 0;
        for (int e = lane; e < n; e += kWave) {
            uint64_t x = buf[e];
            best = (x < prev && x > best) ? x : best;
        }
        best = wave_max_u64(best);
        if (lane == t) mine = best;
        prev = best;
    }
    return mine;
}

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {  // bf16 bits
    static constexpr int n = 8;
    typedef u32x4 raw;
    __device__ static void unpack(const raw &r, float *x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[2 * j] = bf16_lo(r[j]); x[2 * j + 1] = bf16_hi(r[j]); }
    }
    __device__ static float scalar(const uint16_t *p) { return __uint_as_float((uint32_t)(*p) << 16); }
};
template <> struct Vec<float> {
    static constexpr int n = 4;
    typedef f32x4 raw;
    __device__ static void unpack(const raw &r, float *x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = r[j];
    }
    __device__ static float scalar(const float *p) { return *p; }
};

template <typename T, bool kLse>
__global__ __launch_bounds__(kT1Waves * kWave) void k_topk_stage1(
    const T *__restrict__ logits, int64_t ld, int64_t V, int64_t chunk_len, int chunks, int64_t R,
    int k, uint64_t *__restrict__ cand, float2 *__restrict__ stats) {
    __shared__ uint64_t sbuf[kT1Waves][kCap];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * kT1Waves + wv;
    if (gw >= R * chunks) return;  // whole wave leaves; no block barriers below
    const int64_t r = gw / chunks;
    const int c = (int)(gw % chunks);
    const int64_t start = (int64_t)c * chunk_len;
    const int64_t end = min(V, start + chunk_len);
    const T *row = logits + r * ld;
    uint64_t *buf = sbuf[wv];

    constexpr int VEC = Vec<T>::n;
    constexpr int PER_ITER = kWave * VEC * kUnroll;
    float tv = -INFINITY;       // threshold value (k-th best so far)
    uint32_t ti = 0xffffffffu;  // and its index
    int n = 0;                  // buffered candidates
    float m = -INFINITY, s = 0.f;

    auto flush = [&]() {
        uint64_t mine = wave_select(buf, n, k, lane);
        const int kept = n < k ? n : k;
        if (lane < kept) buf[lane] = mine;
        if (n >= k) {
            uint64_t kth = __shfl(mine, k - 1);
            tv = ordered_to_float((uint32_t)(kth >> 32));
            ti = ~(uint32_t)kth;
        }
        n = kept;
    };

    auto consider = [&](float x, uint32_t idx, bool valid) {
        bool pass = valid && ((x > tv) || (x == tv && idx < ti));
        uint64_t bal = __ballot(pass);
        if (bal) {
            if (n + kWave > kCap) flush();
            // re-test against a possibly raised threshold
            pass = valid && ((x > tv) || (x == tv && idx < ti));
            bal = __ballot(pass);
            if (pass) {
                int pos = n + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
                buf[pos] = make_key(x, idx);
            }
            n += __popcll(bal);
        }
    };

    auto lse_update = [&](const float *x, int cnt) {
        float mx = m;
#pragma unroll
        for (int j = 0; j < VEC; ++j) if (j < cnt) mx = fmaxf(mx, x[j]);
        const float base = mx == -INFINITY ? 0.f : mx * kLog2e;
        float acc = s * __builtin_amdgcn_exp2f(m * kLog2e - base);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            if (j < cnt) acc += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -base));
        s = acc;
        m = mx;
    };

    int64_t base = start;
    // full iterations: every lane has kUnroll whole vectors
    for (; base + PER_ITER <= end; base += PER_ITER) {
        typename Vec<T>::raw raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            raw[u] = *(const typename Vec<T>::raw *)(row + base + (int64_t)(u * kWave + lane) * VEC);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[VEC];
            Vec<T>::unpack(raw[u], x);
            const uint32_t i0 = (uint32_t)(base + (int64_t)(u * kWave + lane) * VEC);
            if (kLse) lse_update(x, VEC);
            // fast reject of the whole vector
            float vmax = x[0];
#pragma unroll
            for (int j = 1; j < VEC; ++j) vmax = fmaxf(vmax, x[j]);
            bool any = vmax > tv || vmax == tv;
            if (__ballot(any)) {
#pragma unroll
                for (int j = 0; j < VEC; ++j) consider(x[j], i0 + j, true);
            }
        }
    }
    // one whole vector per lane
    for (; base + kWave * VEC <= end; base += kWave * VEC) {
        typename Vec<T>::raw raw = *(const typename Vec<T>::raw *)(row + base + (int64_t)lane * VEC);
        float x[VEC];
        Vec<T>::unpack(raw, x);
        const uint32_t i0 = (uint32_t)(base + (int64_t)lane * VEC);
        if (kLse) lse_update(x, VEC);
#pragma unroll
        for (int j = 0; j < VEC; ++j) consider(x[j], i0 + j, true);
    }
    // tail: element-wise, bounds-checked
    for (; base < end; base += kWave) {
        const int64_t e = base + lane;
        const bool valid = e < end;
        float x = valid ? Vec<T>::scalar(row + e) : -INFINITY;
        if (kLse && valid) lse_update(&x, 1);
        consider(x, (uint32_t)e, valid);
    }
    flush();
    // write this slice's k best (padding with key 0 when the slice is short)
    uint64_t *out = cand + ((int64_t)r * chunks + c) * k;
    for (int t = lane; t < k; t += kWave) out[t] = t < n ? buf[t] : 0ull;
    if (kLse) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float mo = __shfl_xor(m, off), so = __shfl_xor(s, off);
            float mn = fmaxf(m, mo);
            float bn = mn == -INFINITY ? 0.f : mn * kLog2e;
            s = s * __builtin_amdgcn_exp2f(m * kLog2e - bn) + so * __builtin_amdgcn_exp2f(mo * kLog2e - bn);
            m = mn;
        }
        if (lane == 0) stats[(int64_t)r * chunks + c] = make_float2(m, s);
    }
}

constexpr int kMaxCand = 4096;

template <bool kLse>
__global__ __launch_bounds__(kWave) void k_topk_stage2(const uint64_t *__restrict__ cand,
                                                      const float2 *__restrict__ stats, int chunks,
                                                      int k, int32_t *__restrict__ idx,
                                                      float *__restrict__ val,
                                                      float *__restrict__ lse) {
    __shared__ uint64_t buf[kMaxCand];
    const int lane = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int n = chunks * k;
    const uint64_t *src = cand + r * (int64_t)n;
    for (int e = lane; e < n; e += kWave) buf[e] = src[e];
    __syncthreads();
    uint64_t mine = wave_select(buf, n, k, lane);
    if (lane < k) {
        idx[r * k + lane] = (int32_t)(~(uint32_t)mine);
        val[r * k + lane] = ordered_to_float((uint32_t)(mine >> 32));
    }
    if (kLse) {
        float m = -INFINITY, s = 0.f;
        for (int c = lane; c < chunks; c += kWave) {
            float2 st = stats[r * chunks + c];
            float mn = fmaxf(m, st.x);
            float bn = mn == -INFINITY ? 0.f : mn * kLog2e;
            s = s * __builtin_amdgcn_exp2f(m * kLog2e - bn) + st.y * __builtin_amdgcn_exp2f(st.x * kLog2e - bn);
            m = mn;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float mo = __shfl_xor(m, off), so = __shfl_xor(s, off);
            float mn = fmaxf(m, mo);
            float bn = mn == -INFINITY ? 0.f : mn * kLog2e;
            s = s * __builtin_amdgcn_exp2f(m * kLog2e - bn) + so * __builtin_amdgcn_exp2f(mo * kLog2e - bn);
            m = mn;
        }
        if (lane == 0) lse[r] = m == -INFINITY ? -INFINITY : m + logf(s);
    }
}

}  // namespace

void plan_topk(TopkPlan &p, int64_t R, int64_t V, int k) {
    p.R = R;
    p.V = V;
    p.k = k;
    int64_t chunks = (4096 + R - 1) / R;  // aim for >= 4096 wavefronts
    if (chunks < 1) chunks = 1;
    if (chunks > 64) chunks = 64;
    if (chunks * k > kMaxCand) chunks = kMaxCand / k;
    int64_t len = (V + chunks - 1) / chunks;
    len = (len + 511) / 512 * 512;
    p.chunk_len = len;
    p.chunks = (int)((V + len - 1) / len);
}

size_t topk_workspace_bytes(const TopkPlan &p) {
    const size_t rows = (size_t)p.R * p.chunks;
    size_t cand = rows * p.k * sizeof(uint64_t);
    size_t st = rows * sizeof(float2);
    return ((cand + 255) / 256) * 256 + st;
}

hipError_t launch_topk(const TopkPlan &p, const void *logits, int64_t ld, jf_dtype dtype,
                       int32_t *idx, float *val, float *lse, void *workspace, hipStream_t s) {
    const size_t rows = (size_t)p.R * p.chunks;
    uint64_t *cand = (uint64_t *)workspace;
    size_t cand_bytes = ((rows * p.k * sizeof(uint64_t) + 255) / 256) * 256;
    float2 *stats = (float2 *)((char *)workspace + cand_bytes);
    const unsigned g1 = (unsigned)((rows + kT1Waves - 1) / kT1Waves);
    const bool with_lse = lse != nullptr;
    if (dtype == JF_BF16) {
        if (with_lse)
            hipLaunchKernelGGL((k_topk_stage1<uint16_t, true>), dim3(g1), dim3(kT1Waves * kWave), 0, s,
                               (const uint16_t *)logits, ld, p.V, p.chunk_len, p.chunks, p.R, p.k, cand, stats);
        else
            hipLaunchKernelGGL((k_topk_stage1<uint16_t, false>), dim3(g1), dim3(kT1Waves * kWave), 0, s,
                               (const uint16_t *)logits, ld, p.V, p.chunk_len, p.chunks, p.R, p.k, cand, stats);
    } else {
        if (with_lse)
            hipLaunchKernelGGL((k_topk_stage1<float, true>), dim3(g1), dim3(kT1Waves * kWave), 0, s,
                               (const float *)logits, ld, p.V, p.chunk_len, p.chunks, p.R, p.k, cand, stats);
        else
            hipLaunchKernelGGL((k_topk_stage1<float, false>), dim3(g1), dim3(kT1Waves * kWave), 0, s,
                               (const float *)logits, ld, p.V, p.chunk_len, p.chunks, p.R, p.k, cand, stats);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (with_lse)
        hipLaunchKernelGGL((k_topk_stage2<true>), dim3((unsigned)p.R), dim3(kWave), 0, s, cand, stats,
                           p.chunks, p.k, idx, val, lse);
    else
        hipLaunchKernelGGL((k_topk_stage2<false>), dim3((unsigned)p.R), dim3(kWave), 0, s, cand, stats,
                           p.chunks, p.k, idx, val, lse);
    return hipGetLastError();
}

}  // namespace jf
