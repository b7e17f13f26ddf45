// k_topk.hip -- per-node top-k of the draft logits and the row log-sum-exp.
//
// The draft tree is grown from each node's most likely next tokens, and a
// branch's probability is the product of per-node conditionals (JetFlow blog
// page, "What JetFlow Does Differently"): every node row needs its k best
// logits (value descending, ties by lower index) and its normaliser.
//
// The scan is HBM-bound (one pass over R x V logits).  Stage 1: one wavefront
// per (row, slice of the vocabulary).  Every lane issues all of its 16-byte
// loads at once and keeps the slice in registers.  Pass 1 folds each vector
// into the lane maximum and the running (max, sum-exp) as it arrives.  The
// k-th largest of the 64 lane maxima bounds the slice's k-th best from below,
// so only elements at or above it can survive, and they sit in the few lanes
// whose maximum reaches it: those lanes copy their vectors to LDS, the whole
// wave scans them, and the survivors are compacted (ballot prefix sums) and
// ranked against each other.  Stage 2: one block per row merges the slices'
// k-best lists and (max, sum-exp) pairs.
//
// Candidates are 64-bit keys: high word = order-preserving image of the fp32
// value (-0 folded onto +0), low word = ~index, so that a larger key is a
// better candidate and keys are unique within a row.
#include <mutex>
#include <type_traits>

#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kT1Waves = 4;
constexpr int kFuseWaves = 16;    // one block a row: up to 16 slices
constexpr int kFuseMinRows = 128; // rows that fill the chip with one block a row
constexpr int kCap = 512;     // survivors a wave can buffer before the selection from memory
constexpr int kMaxVec = 19;   // 16-byte vectors per lane a wave holds in registers
constexpr int kHot = 16;      // hot lanes whose vectors go through LDS
constexpr int kScan = (kHot * kMaxVec + 63) / 64;   // scan rounds over the hot vectors
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 5.545177444479562f;   // 8 * ln 2: rescale the running sum past 2^8

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

// DPP lane moves within 16-lane rows (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror): after the four steps every lane holds the
// maximum of its row.
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, kCtrl, 0xf, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), kCtrl, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wavefront, returned to every lane (wave-uniform).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = umax64(v, dpp_u64<0xb1>(v));
    v = umax64(v, dpp_u64<0x4e>(v));
    v = umax64(v, dpp_u64<0x141>(v));
    v = umax64(v, dpp_u64<0x140>(v));
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, row * 16);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), row * 16);
        r = umax64(r, ((uint64_t)hi << 32) | lo);
    }
    return r;
}

// Rank of `key` among the n keys in LDS (the number of larger ones; keys are
// unique).  Every lane reads the same entries, so each read is a broadcast.
__device__ __forceinline__ int rank_in(const uint64_t *keys, int n, uint64_t key) {
    int rank = 0;
    int j = 0;
#pragma unroll 4
    for (; j + 2 <= n; j += 2) {
        const u32x4 q = *(const u32x4 *)(keys + j);       // keys j, j+1 (16-byte aligned)
        rank += (((uint64_t)q[1] << 32) | q[0]) > key;
        rank += (((uint64_t)q[3] << 32) | q[2]) > key;
    }
    if (j < n) rank += keys[j] > key;
    return rank;
}

// Rank of a key among `runs` runs of k keys, each in decreasing order (a
// slice's candidates in rank order, zero padded): the keys above it, counted
// in each run by a binary search (k <= 64).
// Four runs are searched side by side so that their LDS reads overlap.
__device__ __forceinline__ int rank_in_runs(const uint64_t *keys, int runs, int k, uint64_t key) {
    int rank = 0;
    int c = 0;
    for (; c + 4 <= runs; c += 4) {
        const uint64_t *run = keys + c * k;
        int p0 = 0, p1 = 0, p2 = 0, p3 = 0;          // keys of each run above `key`
#pragma unroll
        for (int step = 64; step >= 1; step >>= 1) {
            const bool in = (step <= k);              // p + step <= k needs step <= k
            if (in && p0 + step <= k && run[p0 + step - 1] > key) p0 += step;
            if (in && p1 + step <= k && run[k + p1 + step - 1] > key) p1 += step;
            if (in && p2 + step <= k && run[2 * k + p2 + step - 1] > key) p2 += step;
            if (in && p3 + step <= k && run[3 * k + p3 + step - 1] > key) p3 += step;
        }
        rank += p0 + p1 + p2 + p3;
    }
    for (; c < runs; ++c) {
        const uint64_t *run = keys + c * k;
        int pos = 0;
#pragma unroll
        for (int step = 64; step >= 1; step >>= 1)
            if (pos + step <= k && run[pos + step - 1] > key) pos += step;
        rank += pos;
    }
    return rank;
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
    __device__ static uint32_t load1(__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
    __device__ static float widen(uint32_t b) { return __uint_as_float(b << 16); }
};
template <> struct Vec<float> {
    static constexpr int n = 4;
    typedef f32x4 raw;
    __device__ static void unpack(const raw &r, float *x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = r[j];
    }
    __device__ static float scalar(const float *p) { return *p; }
    __device__ static uint32_t load1(__amdgpu_buffer_rsrc_t r, int off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    __device__ static float widen(uint32_t b) { return __uint_as_float(b); }
};

// kFused = false: kWB waves a block, one (row, slice) a wave; the k best keys
// and (max, sum-exp) of every slice go to the workspace for the merge kernel.
// kFused = true: one block a row, wave c taking slice c (chunks <= kWB); the
// slices' results stay in LDS and wave 0 merges them.
template <typename T, bool kLse, int kWB, bool kFused>
__global__ __launch_bounds__(kWB * kWave) void k_topk_stage1(
    const T *__restrict__ logits, int64_t ld, int64_t V, int64_t chunk_len, int chunks, int64_t R,
    int k, uint64_t *__restrict__ cand, float2 *__restrict__ stats, int32_t *__restrict__ idx,
    float *__restrict__ val, float *__restrict__ lse) {
    __shared__ __attribute__((aligned(16))) uint64_t sbuf[kWB][kCap];
    __shared__ __attribute__((aligned(16))) u32x4 hbuf[kWB][kHot * kMaxVec];
    __shared__ int hlane[kWB][kHot];
    __shared__ __attribute__((aligned(16))) uint64_t mkeys[kFused ? kWB * 64 : 2];   // slices' k best
    __shared__ float2 mstats[kFused ? kWB : 1];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const int64_t gw = kFused ? (int64_t)blockIdx.x * chunks + wv : (int64_t)blockIdx.x * kWB + wv;
    if (!kFused && gw >= R * chunks) return;  // whole wave leaves; no block barriers below
    const int64_t r = gw / chunks;
    const int c = (int)(gw % chunks);
    const int64_t start = (int64_t)c * chunk_len;
    const int64_t end = min(V, start + chunk_len);
    const T *row = logits + r * ld;
    uint64_t *buf = sbuf[wv];

    constexpr int VEC = Vec<T>::n;
    constexpr int STEP = kWave * VEC;          // elements per wave-wide vector
    constexpr int MAXV = kMaxVec;              // vectors per lane held in registers
    typedef typename Vec<T>::raw Raw;
    // whole vectors of the slice (<= MAXV by the plan); every slice but a
    // row's last is full, and a full slice runs with nv a compile-time constant
    const int nv_rt = (int)((end - start) / STEP);
    auto slice = [&](auto NV) {
        const int nv = NV;
        const int64_t tail0 = start + (int64_t)nv * STEP;

        // ---- all loads in flight at once ----
        // Range-checked buffer loads: a read past the slice returns zeros instead
        // of faulting, so every load is issued unconditionally and the compiler
        // can wait for each vector on its own (vmcnt counts) as pass 1 reaches it.
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(row + start, (uint32_t)((end - start) * (int64_t)sizeof(T)));
        Raw d[MAXV];
#pragma unroll
        for (int v = 0; v < MAXV; ++v)
            d[v] = __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(
                       rs, (v * STEP + lane * VEC) * (int)sizeof(T), 0, 0));
        uint32_t traw[VEC];                        // tail: element tail0 + lane + 64 t (raw bits)
#pragma unroll
        for (int t = 0; t < VEC; ++t)
            traw[t] = Vec<T>::load1(rs, (nv * STEP + lane + t * kWave) * (int)sizeof(T));
        const int ntail = (int)(end - tail0);      // 0 .. STEP-1, wave-uniform
        float tx[VEC];
        auto tail_values = [&]() {
#pragma unroll
            for (int t = 0; t < VEC; ++t)
                tx[t] = lane + t * kWave < ntail ? Vec<T>::widen(traw[t]) : -INFINITY;
        };

        // ---- pass 1: lane maximum and the running log-sum-exp ----
        float lmax = -INFINITY;
        float m = -INFINITY, s = 0.f;
        float base = 0.f;                          // m * log2(e), 0 while m = -inf
        auto lse_add = [&](const float *x, float vmax, int cnt) {
            // the running maximum moves rarely once the first vectors are in,
            // so the rescale sits behind a wave-uniform branch
            if (__ballot(vmax > m + kLazy)) {
                asm volatile("");                  // a real branch: not computed speculatively
                if (vmax > m + kLazy) {
                    s *= __builtin_amdgcn_exp2f((m - vmax) * kLog2e);
                    m = vmax;
                    base = m * kLog2e;
                }
            }
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                if (j < cnt) s += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -base));
        };
#pragma unroll
        for (int v = 0; v < MAXV; ++v) {
            if (v < nv) {
                float x[VEC];
                Vec<T>::unpack(d[v], x);
                float vmax = x[0];
#pragma unroll
                for (int j = 1; j < VEC; ++j) vmax = fmaxf(vmax, x[j]);
                lmax = fmaxf(lmax, vmax);
                if (kLse) lse_add(x, vmax, VEC);
            }
        }
        tail_values();
        if (kLse && ntail > 0) {
#pragma unroll
            for (int t = 0; t < VEC; ++t) {
                const bool ok = lane + t * kWave < ntail;
                float x1 = ok ? tx[t] : -INFINITY;
                if (ok) lse_add(&x1, x1, 1);
            }
        }

        // Make the raw vectors look modified so that the compiler recomputes the
        // unpacked values in pass 2 instead of keeping them all live from pass 1.
        auto touch = [&]() {
#pragma unroll
            for (int v = 0; v < MAXV; ++v) asm volatile("" : "+v"(d[v]));
        };
        touch();

        // ---- threshold ----
        // tv = the k-th largest lane maximum.  k lanes hold an element >= tv, so
        // the slice's k-th largest element is >= tv and everything below tv is
        // out: survivors sit only in the "hot" lanes (lane maximum >= tv) and in
        // the tail.  tv is found by bisection on the order-preserving bits: the
        // largest key that at least k lane maxima reach (k <= 64).
        float tv = -INFINITY;
        uint64_t hot = 0;
        if (nv > 0) {
            const uint32_t key = ordered_bits(lmax);
            constexpr int kLow = VEC == 8 ? 16 : 0;   // widened bf16: the low half follows the sign
            uint32_t p = 0;
#pragma unroll
            for (int b = 31; b >= kLow; --b) {
                const uint32_t cb = p | (1u << b);
                p = __popcll(__ballot(key >= cb)) >= (uint32_t)k ? cb : p;
            }
            if (kLow) p |= (p & 0x80000000u) ? 0u : 0xffffu;
            tv = ordered_to_float(p);
            hot = __ballot(lmax >= tv);
        }
        const int nhot = __popcll(hot);

        // survivor bits (x >= tv) of one 16-byte vector
        auto survivors = [&](const Raw &rv) -> uint32_t {
            uint32_t pm = 0;
            if (VEC == 8 && tv > 0.f) {
                // bf16 with a positive threshold: x >= tv exactly when x's bit
                // pattern, read as a signed integer, is >= tv's (negative values
                // and -0 read as negative integers), and tv's low 16 bits are
                // zero, so each packed word is tested without unpacking.
                const int32_t tb = __float_as_int(tv);
                const u32x4 raw = __builtin_bit_cast(u32x4, rv);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    pm |= (uint32_t)((int32_t)(raw[w] << 16) >= tb) << (2 * w);
                    pm |= (uint32_t)((int32_t)raw[w] >= tb) << (2 * w + 1);
                }
            } else {
                float x[VEC];
                Vec<T>::unpack(rv, x);
#pragma unroll
                for (int j = 0; j < VEC; ++j) pm |= (uint32_t)(x[j] >= tv) << j;
            }
            return pm;
        };
        // element j of a raw vector as fp32
        auto element = [&](const Raw &rv, int j) -> float {
            const u32x4 raw = __builtin_bit_cast(u32x4, rv);
            if (VEC == 8) {
                const uint32_t word = raw[j >> 1];
                return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
            }
            return __uint_as_float(raw[j & 3]);
        };
        uint32_t tmark = 0;
#pragma unroll
        for (int t = 0; t < VEC; ++t)
            tmark |= (uint32_t)(lane + t * kWave < ntail && tx[t] >= tv) << t;

        // one wave prefix sum over the per-lane survivor counts (each < 256)
        int pre = 0, tot = 0;
        auto place = [&](int cnt) {
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) {
                const uint64_t b = __ballot((cnt >> bit) & 1);
                pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0)) << bit;
                tot += __popcll(b) << bit;
            }
        };
        auto put_tail = [&](int &pos) {
#pragma unroll
            for (int t = 0; t < VEC; ++t)
                if ((tmark >> t) & 1u) buf[pos++] = make_key(tx[t], (uint32_t)(tail0 + lane + t * kWave));
        };

        if (nhot <= kHot) {
            // ---- few hot lanes: they copy their vectors to LDS and the whole
            // wave scans them, one vector a lane per round ----
            u32x4 *hv = hbuf[wv];                    // [nhot][nv] vectors, slot-major
            int *hl = hlane[wv];                     // slot -> lane
            if ((hot >> lane) & 1ull) {
                const int slot = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hot >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)hot, 0));
                hl[slot] = lane;
#pragma unroll
                for (int v = 0; v < MAXV; ++v)
                    if (v < nv) hv[slot * nv + v] = __builtin_bit_cast(u32x4, d[v]);
            }
            __builtin_amdgcn_wave_barrier();
            const int nvec = nhot * nv;
            Raw sv[kScan];
            uint32_t spm[kScan];
            int cnt = __popc(tmark);
#pragma unroll
            for (int i = 0; i < kScan; ++i) {
                const int q = lane + i * kWave;
                spm[i] = 0;
                if (q < nvec) {
                    sv[i] = __builtin_bit_cast(Raw, hv[q]);
                    spm[i] = survivors(sv[i]);
                    cnt += __popc(spm[i]);
                }
            }
            place(cnt);
            if (tot <= kCap) {
                int pos = pre;
#pragma unroll
                for (int i = 0; i < kScan; ++i) {
                    uint32_t pm = spm[i];
                    if (pm) {
                        const int q = lane + i * kWave;
                        const int sl = q / nv, v = q - sl * nv;
                        const uint32_t i0 = (uint32_t)(start + (int64_t)v * STEP + (int64_t)hl[sl] * VEC);
                        while (pm) {
                            const int j = __builtin_ctz(pm);
                            pm &= pm - 1u;
                            buf[pos++] = make_key(element(sv[i], j), i0 + j);
                        }
                    }
                }
                put_tail(pos);
            }
        } else {
            // ---- many hot lanes (k above kHot, or ties at the threshold):
            // every lane marks its own vectors, then writes its survivors ----
            uint32_t marks[(MAXV * VEC + 31) / 32];
#pragma unroll
            for (int w = 0; w < (MAXV * VEC + 31) / 32; ++w) marks[w] = 0u;
            int cnt = __popc(tmark);
#pragma unroll
            for (int v = 0; v < MAXV; ++v) {
                if (v < nv) {
                    const uint32_t pm = survivors(d[v]);
                    marks[(v * VEC) / 32] |= pm << ((v * VEC) % 32);
                    cnt += __popc(pm);
                }
            }
            place(cnt);
            if (tot > 2 * k) {
                // With k above kHot the k-th largest lane maximum leaves several
                // survivors a lane (hundreds a wave, at times more than the
                // buffer).  Any threshold that keeps at least k elements keeps
                // the k best, so raise it: a 256-bin histogram of the
                // survivors' order-preserving keys above tv's (the top 16 bits
                // for bf16, so every bin edge is a bf16 value; bins 2^sh keys
                // wide, sh the least that spans the wave's largest key), then
                // the highest bin edge that still keeps k.  The histogram sits
                // in this wave's hot-vector area, unused on this path.
                constexpr int kLow = VEC == 8 ? 16 : 0;
                float wmax = lmax;
#pragma unroll
                for (int q = 0; q < VEC; ++q) wmax = fmaxf(wmax, tx[q]);   // -inf past the tail
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) wmax = fmaxf(wmax, __shfl_xor(wmax, off));
                const uint32_t base = ordered_bits(tv) >> kLow;
                const uint32_t span = (ordered_bits(wmax) >> kLow) - base;   // wmax >= tv
                const int sh = span < 256u ? 0 : 24 - __builtin_clz(span);  // span >> sh < 256
                uint32_t *hist = (uint32_t *)hbuf[wv];
                hbuf[wv][lane] = u32x4{0u, 0u, 0u, 0u};
                __builtin_amdgcn_wave_barrier();
                auto bin_of = [&](float x) -> uint32_t {
                    return ((ordered_bits(x) >> kLow) - base) >> sh;
                };
#pragma unroll
                for (int v = 0; v < MAXV; ++v) {
                    uint32_t pm = (marks[(v * VEC) / 32] >> ((v * VEC) % 32)) & ((1u << VEC) - 1u);
                    if (v < nv && __ballot(pm != 0)) {
                        while (pm) {
                            const int j = __builtin_ctz(pm);
                            pm &= pm - 1u;
                            atomicAdd(&hist[bin_of(element(d[v], j))], 1u);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    if ((tmark >> q) & 1u) atomicAdd(&hist[bin_of(tx[q])], 1u);
                __builtin_amdgcn_wave_barrier();
                const u32x4 h = hbuf[wv][lane];              // bins 4 lane .. 4 lane + 3
                int above = (int)(h[0] + h[1] + h[2] + h[3]);  // then: bins >= 4 lane
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const int o = __shfl_down(above, off);
                    above += lane + off < kWave ? o : 0;
                }
                const int s3 = above - (int)(h[0] + h[1] + h[2]);   // bins >= 4 lane + 3
                const int s2 = s3 + (int)h[2], s1 = s2 + (int)h[1];
                const int j = s3 >= k ? 3 : s2 >= k ? 2 : s1 >= k ? 1 : 0;
                const uint64_t ok = __ballot(above >= k);     // lane 0 always: all survivors
                const int L = 63 - __builtin_clzll(ok);
                const int b = 4 * L + __shfl(j, L);
                const uint32_t key = base + ((uint32_t)b << sh);
                uint32_t pk = key << kLow;
                if (kLow) pk |= (pk & 0x80000000u) ? 0u : 0xffffu;
                tv = ordered_to_float(pk);
                tmark = 0;
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    tmark |= (uint32_t)(lane + q * kWave < ntail && tx[q] >= tv) << q;
#pragma unroll
                for (int w = 0; w < (MAXV * VEC + 31) / 32; ++w) marks[w] = 0u;
                cnt = __popc(tmark);
#pragma unroll
                for (int v = 0; v < MAXV; ++v) {
                    if (v < nv) {
                        const uint32_t pm = survivors(d[v]);
                        marks[(v * VEC) / 32] |= pm << ((v * VEC) % 32);
                        cnt += __popc(pm);
                    }
                }
                pre = 0;
                tot = 0;
                place(cnt);
            }
            if (tot <= kCap) {
                int pos = pre;
#pragma unroll
                for (int v = 0; v < MAXV; ++v) {
                    uint32_t pm = (marks[(v * VEC) / 32] >> ((v * VEC) % 32)) & ((1u << VEC) - 1u);
                    if (v < nv && __ballot(pm != 0)) {
                        const uint32_t i0 = (uint32_t)(start + (int64_t)v * STEP + (int64_t)lane * VEC);
                        while (pm) {
                            const int j = __builtin_ctz(pm);
                            pm &= pm - 1u;
                            buf[pos++] = make_key(element(d[v], j), i0 + j);
                        }
                    }
                }
                put_tail(pos);
            }
        }

        uint64_t *out = kFused ? mkeys + c * k : cand + ((int64_t)r * chunks + c) * k;
        if (tot <= kCap) {
            __builtin_amdgcn_wave_barrier();
            // every buffered survivor learns its rank; the k best write themselves
            for (int e = lane; e < tot; e += kWave) {
                const uint64_t key = buf[e];
                const int rk = rank_in(buf, tot, key);
                if (rk < k) out[rk] = key;
            }
            for (int e = tot + lane; e < k; e += kWave) out[e] = 0ull;   // short slice
        } else {
            // Too many ties at the threshold for the buffer (rare): select straight
            // from memory, k rounds of "best key below the previous pick".  Kept
            // out of registers on purpose so that it costs the common path nothing.
            uint64_t prev = ~0ull, mine = 0;
            for (int t = 0; t < k; ++t) {
                uint64_t best = 0;
                for (int64_t e = start + lane; e < end; e += kWave) {
                    const uint64_t kk = make_key(Vec<T>::scalar(row + e), (uint32_t)e);
                    best = (kk < prev && kk > best) ? kk : best;
                }
                best = wave_max_u64(best);
                if (lane == t) mine = best;
                prev = best;
            }
            if (lane < k) out[lane] = mine;
        }
        if (kLse) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                float mo = __shfl_xor(m, off), so = __shfl_xor(s, off);
                float mn = fmaxf(m, mo);
                float bn = mn == -INFINITY ? 0.f : mn * kLog2e;
                s = s * __builtin_amdgcn_exp2f(m * kLog2e - bn) + so * __builtin_amdgcn_exp2f(mo * kLog2e - bn);
                m = mn;
            }
            if (lane == 0) {
                if (kFused) mstats[c] = make_float2(m, s);
                else stats[(int64_t)r * chunks + c] = make_float2(m, s);
            }
        }
    };
    if (nv_rt == MAXV) slice(std::integral_constant<int, MAXV>());
    else slice(nv_rt);

    if constexpr (kFused) {
        // ---- merge the row's slices: rank every candidate among the
        // chunks * k keys with all of the block's waves (a group of G lanes a
        // candidate, G the largest power of two with G * k <= 64, each lane
        // counting the larger keys in its 1/G share); then wave 0 combines
        // the (max, sum-exp) pairs ----
        __syncthreads();
        const int n = chunks * k;
        if (k > kHot) {
            // large k: a thread a candidate (n <= chunks * 64 threads), ranked
            // by binary searches in the slices' sorted runs
            const int e = (int)threadIdx.x;
            const uint64_t key = e < n ? mkeys[e] : 0ull;
            if (key != 0ull) {
                const int cnt = rank_in_runs(mkeys, chunks, k, key);
                if (cnt < k) {
                    idx[r * k + cnt] = (int32_t)(~(uint32_t)key);
                    val[r * k + cnt] = ordered_to_float((uint32_t)(key >> 32));
                }
            }
        } else {
            int lg = 0;
            while (lg < 6 && (2 << lg) * k <= kWave) ++lg;
            const int G = 1 << lg;
            const int e = (int)threadIdx.x >> lg;           // candidate; < chunks * 64 / G, >= n only as spare
            const int part = (int)threadIdx.x & (G - 1);
            const uint64_t key = e < n ? mkeys[e] : 0ull;
            // eight keys a round in flight (the reads are LDS broadcasts)
            int cnt = 0;
            int j = part;
            for (; j + 7 * G < n; j += 8 * G) {
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = mkeys[j + u * G];
#pragma unroll
                for (int u = 0; u < 8; ++u) cnt += v[u] > key;
            }
            for (; j < n; j += G) cnt += mkeys[j] > key;
            for (int m = G >> 1; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m);
            // key 0: padding of a short slice, or a spare lane
            if (part == 0 && key != 0ull && cnt < k) {
                idx[r * k + cnt] = (int32_t)(~(uint32_t)key);
                val[r * k + cnt] = ordered_to_float((uint32_t)(key >> 32));
            }
        }
        if (wv != 0) return;
        if (kLse) {
            float m = lane < chunks ? mstats[lane].x : -INFINITY;
            float s = lane < chunks ? mstats[lane].y : 0.f;
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
}

constexpr int kMaxCand = 4096;   // chunks * k candidates merged per row
constexpr int kMergeTarget = 256;  // preferred bound on chunks * k

template <bool kLse, int kThreads>
__global__ __launch_bounds__(kThreads) void k_topk_stage2(const uint64_t *__restrict__ cand,
                                                    const float2 *__restrict__ stats, int chunks,
                                                    int k, int32_t *__restrict__ idx,
                                                    float *__restrict__ val,
                                                    float *__restrict__ lse) {
    __shared__ __attribute__((aligned(16))) uint64_t keys[kMaxCand];
    __shared__ float2 part[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t r = blockIdx.x;
    const int n = chunks * k;                    // <= kMaxCand
    const uint64_t *src = cand + r * (int64_t)n;
    for (int e = tid; e < n; e += kThreads) keys[e] = src[e];
    __syncthreads();
    for (int e = tid; e < n; e += kThreads) {
        const uint64_t key = keys[e];
        if (key == 0ull) continue;               // padding of a short slice
        const int rk = k > kHot ? rank_in_runs(keys, chunks, k, key) : rank_in(keys, n, key);
        if (rk < k) {
            idx[r * k + rk] = (int32_t)(~(uint32_t)key);
            val[r * k + rk] = ordered_to_float((uint32_t)(key >> 32));
        }
    }
    if (kLse) {
        float m = -INFINITY, s = 0.f;
        // the slices' (max, sum-exp) pairs are combined by the first 256
        // threads in the same order at every block size
        constexpr int kLseThreads = 256;
        for (int c = tid; tid < kLseThreads && c < chunks; c += kLseThreads) {
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
        if (lane == 0 && wv < kLseThreads / kWave) part[wv] = make_float2(m, s);
        __syncthreads();
        if (tid == 0) {
            m = -INFINITY;
            s = 0.f;
            for (int w = 0; w < kLseThreads / kWave; ++w) {
                float mn = fmaxf(m, part[w].x);
                float bn = mn == -INFINITY ? 0.f : mn * kLog2e;
                s = s * __builtin_amdgcn_exp2f(m * kLog2e - bn) +
                    part[w].y * __builtin_amdgcn_exp2f(part[w].x * kLog2e - bn);
                m = mn;
            }
            lse[r] = m == -INFINITY ? -INFINITY : m + logf(s);
        }
    }
}

}  // namespace

void plan_topk(TopkPlan &p, int64_t R, int64_t V, int k, jf_dtype dtype) {
    p.R = R;
    p.V = V;
    p.k = k;
    // a slice must fit one wave's registers: kMaxVec 16-byte vectors a lane
    const int64_t max_len = (int64_t)kMaxVec * kWave * (dtype == JF_BF16 ? 8 : 4);
    int64_t chunks = (2048 + R - 1) / R;  // aim for >= 2048 wavefronts
    // ... but the merge ranks every candidate against all chunks * k of them,
    // so keep that list short (256) unless the slice size forces more slices
    int64_t cap = kMergeTarget / k;
    const int64_t min_chunks = (V + max_len - 1) / max_len;
    if (cap < min_chunks) cap = min_chunks;
    if (chunks > cap) chunks = cap;
    if (chunks > kMaxCand / k) chunks = kMaxCand / k;
    if (chunks < 1) chunks = 1;
    int64_t len = (V + chunks - 1) / chunks;
    len = (len + 511) / 512 * 512;
    if (len > max_len) len = max_len;
    chunks = (V + len - 1) / len;
    if (chunks * k > kMaxCand) {          // too many slices to merge: the plan is refused
        p.chunks = 0;
        p.chunk_len = 0;
        return;
    }
    p.chunk_len = len;
    p.chunks = (int)chunks;
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
    // One block a row when the row's slices fit one block and the rows alone
    // fill the chip; else slices as independent waves and a merge kernel.
    const bool fused = p.chunks <= kFuseWaves && p.R >= kFuseMinRows;
#define JF_TOPK1(T, L, WB, F, grid, block)                                                           \
    hipLaunchKernelGGL((k_topk_stage1<T, L, WB, F>), dim3(grid), dim3(block), 0, s, (const T *)logits, \
                       ld, p.V, p.chunk_len, p.chunks, p.R, p.k, cand, stats, idx, val, lse)
    if (fused) {
        const unsigned gr = (unsigned)p.R, bl = (unsigned)(p.chunks * kWave);
        if (dtype == JF_BF16) {
            if (with_lse) JF_TOPK1(uint16_t, true, kFuseWaves, true, gr, bl);
            else JF_TOPK1(uint16_t, false, kFuseWaves, true, gr, bl);
        } else {
            if (with_lse) JF_TOPK1(float, true, kFuseWaves, true, gr, bl);
            else JF_TOPK1(float, false, kFuseWaves, true, gr, bl);
        }
        return hipGetLastError();
    }
    if (dtype == JF_BF16) {
        if (with_lse) JF_TOPK1(uint16_t, true, kT1Waves, false, g1, kT1Waves * kWave);
        else JF_TOPK1(uint16_t, false, kT1Waves, false, g1, kT1Waves * kWave);
    } else {
        if (with_lse) JF_TOPK1(float, true, kT1Waves, false, g1, kT1Waves * kWave);
        else JF_TOPK1(float, false, kT1Waves, false, g1, kT1Waves * kWave);
    }
#undef JF_TOPK1
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // k above kHot: ranks by binary searches, latency-bound chains, so four
    // times the threads a row
#define JF_TOPK2(L, TH)                                                                             \
    hipLaunchKernelGGL((k_topk_stage2<L, TH>), dim3((unsigned)p.R), dim3(TH), 0, s, cand, stats,     \
                       p.chunks, p.k, idx, val, lse)
    if (p.k > kHot) {
        if (with_lse) JF_TOPK2(true, 1024);
        else JF_TOPK2(false, 1024);
    } else {
        if (with_lse) JF_TOPK2(true, 256);
        else JF_TOPK2(false, 256);
    }
#undef JF_TOPK2
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (jf_node_topk_noalloc): the
// stage-1 candidates and (max, sum-exp) pairs live in this file-scope device
// array instead of a caller's workspace.  Each device holds its own copy for
// the life of the process.  Its address is taken once per device with
// hipGetSymbolAddress, with that device current; host code passes only that
// address to kernels (the array's name is a host-side stand-in).  Nothing in
// it needs to start at zero: stage 1 writes every slot that stage 2 reads.
static __device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

hipError_t topk_scratch(void **ptr) {
    static std::mutex mu;
    static void *per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

}  // namespace jf
