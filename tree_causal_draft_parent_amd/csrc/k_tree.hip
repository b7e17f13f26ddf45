// k_tree.hip -- path scores of draft-tree nodes and one budgeted best-first
// expansion of the tree.
//
// A branch's draft probability is the product of the per-node conditionals
// along it (JetFlow blog page, "What JetFlow Does Differently"), so a node's
// path score is the sum of the conditional log-probabilities over its
// ancestors (itself included).  Growing the tree best-first under a node
// budget (the pages' 16- and 256-token draft budgets) takes, among every
// node's top candidates, those whose extended path scores are highest.
//
//   k_path_scores : one workgroup per sequence; parents and log-probabilities
//                   staged in LDS; each lane walks its nodes' chains and sums
//                   in fp64 from the node up to the prefix, then rounds once.
//   k_tree_expand : one workgroup per sequence; every (node, rank) candidate
//                   becomes one 64-bit key that orders (score desc, node asc,
//                   rank asc); a bitonic sort of the keys in LDS (stages of
//                   stride < 64 in registers with cross-lane moves), and the
//                   first M keys decode into the new nodes.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kPathThreads = 256;
constexpr int kPathMaxN = 4096;

__global__ __launch_bounds__(kPathThreads) void k_path_scores(const int32_t *__restrict__ parent,
                                                              const float *__restrict__ logp,
                                                              int N, float *__restrict__ score,
                                                              int32_t *__restrict__ seq_status) {
    __shared__ int32_t par[kPathMaxN];
    __shared__ float lp[kPathMaxN];
    __shared__ int32_t first_bad;
    const int b = blockIdx.x;
    const int64_t base = (int64_t)b * N;
    for (int i = threadIdx.x; i < N; i += kPathThreads) {
        par[i] = parent[base + i];
        lp[i] = logp[base + i];
    }
    if (threadIdx.x == 0) first_bad = INT32_MAX;
    __syncthreads();

    for (int i = threadIdx.x; i < N; i += kPathThreads) {
        // Node first, then each parent in turn: the same order of additions
        // on every run, in fp64, so the one rounding to fp32 is the only one.
        double sum = 0.0;
        int j = i, steps = 0;
        bool ok = true;
        while (j != -1) {
            if (j < -1 || j >= N || steps >= N) { ok = false; break; }
            sum += (double)lp[j];
            j = par[j];
            ++steps;
        }
        if (!ok) atomicMin(&first_bad, i);
        score[base + i] = ok ? (float)sum : 0.0f;
    }
    __syncthreads();
    if (threadIdx.x == 0 && seq_status) seq_status[b] = first_bad == INT32_MAX ? -1 : first_bad;
}

// ---------------------------------------------------------------------------
constexpr int kExpThreads = 1024;
constexpr uint64_t kNoCand = ~0ull;

// Order-preserving image of a float: a < b  <=>  ord(a) < ord(b) (NaN aside);
// -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t ord_f32(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u << 1) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

// Compare-exchange of a lane's key with the key of lane (lane ^ j), j < 64,
// toward ascending order inside runs of length kk (descending in odd runs).
__device__ __forceinline__ uint64_t xchg_lanes(uint64_t key, int e, int j, int kk) {
    const int lane = threadIdx.x & 63;
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const int src = (lane ^ j) << 2;
    const uint32_t olo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)lo);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)hi);
    const uint64_t other = ((uint64_t)ohi << 32) | olo;
    const bool up = (e & kk) == 0;          // this run sorts ascending
    const bool lower = (e & j) == 0;        // this lane holds the lower slot of the pair
    const bool take_min = up == lower;
    const uint64_t mn = key < other ? key : other;
    const uint64_t mx = key < other ? other : key;
    return take_min ? mn : mx;
}

template <int LMAX>
__global__ __launch_bounds__(kExpThreads) void k_tree_expand(
    const float *__restrict__ score, const int32_t *__restrict__ depth,
    const int32_t *__restrict__ idx, const float *__restrict__ val, const float *__restrict__ lse,
    int N, int k, int M, int max_depth, int L, int32_t *__restrict__ new_parent,
    int32_t *__restrict__ new_token, float *__restrict__ new_score,
    int32_t *__restrict__ new_depth) {
    __shared__ uint64_t keys[LMAX];           // L = 2^n, 64 <= L <= LMAX, L >= N*k
    const int b = blockIdx.x;
    const int nc = N * k;
    const int64_t nbase = (int64_t)b * N;
    const int64_t cbase = nbase * k;

    // Keys: high word ~ord(score) (descending score first), low word the flat
    // candidate index p*k + r (node ascending, then rank ascending).
    for (int e = threadIdx.x; e < L; e += kExpThreads) {
        uint64_t key = kNoCand;
        if (e < nc) {
            const int p = e / k;
            const int d = depth[nbase + p];
            if (d >= 1 && d < max_depth) {            // child depth d + 1 <= max_depth
                const float t = val[cbase + e] - lse[nbase + p];   // rounded to fp32
                const float s = score[nbase + p] + t;              // rounded to fp32
                key = ((uint64_t)(~ord_f32(s)) << 32) | (uint32_t)e;
            }
        }
        keys[e] = key;
    }
    __syncthreads();

    // Bitonic sort, ascending.  Runs of length kk are merged with strides
    // j = kk/2 .. 1.  Strides >= 64 pair slots in different wavefronts and go
    // through LDS; the strides below 64 of one run are done in registers
    // between a load and a store of the lane's slots.
    for (int kk = 2; kk <= L; kk <<= 1) {
        int j = kk >> 1;
        for (; j >= 64; j >>= 1) {
            for (int t = threadIdx.x; t < (L >> 1); t += kExpThreads) {
                const int lo = ((t & ~(j - 1)) << 1) | (t & (j - 1));
                const int hi = lo | j;
                const uint64_t a = keys[lo], c = keys[hi];
                const bool up = (lo & kk) == 0;
                if ((a > c) == up) {
                    keys[lo] = c;
                    keys[hi] = a;
                }
            }
            __syncthreads();
        }
        // j < 64: each lane owns slot e; pairs (e, e ^ j) sit in one wavefront.
        for (int e = threadIdx.x; e < L; e += kExpThreads) {
            uint64_t key = keys[e];
            for (int jj = j; jj >= 1; jj >>= 1) key = xchg_lanes(key, e, jj, kk);
            keys[e] = key;
        }
        __syncthreads();
    }

    // The first M keys, in order, are the new nodes.
    const int64_t obase = (int64_t)b * M;
    for (int m = threadIdx.x; m < M; m += kExpThreads) {
        const uint64_t key = m < L ? keys[m] : kNoCand;
        if (key != kNoCand) {
            const int e = (int)(uint32_t)key;
            const int p = e / k;
            new_parent[obase + m] = p;
            new_token[obase + m] = idx[cbase + e];
            new_score[obase + m] = unord_f32(~(uint32_t)(key >> 32));
            new_depth[obase + m] = depth[nbase + p] + 1;
        } else {
            new_parent[obase + m] = -2;
            new_token[obase + m] = -1;
            new_score[obase + m] = -__builtin_inff();
            new_depth[obase + m] = 0;
        }
    }
}

}  // namespace

hipError_t launch_path_scores(const int32_t *parent, const float *logp, int B, int N, float *score,
                              int32_t *seq_status, hipStream_t s) {
    hipLaunchKernelGGL(k_path_scores, dim3(B), dim3(kPathThreads), 0, s, parent, logp, N, score,
                       seq_status);
    return hipGetLastError();
}

int tree_expand_slots(int N, int k) {
    int L = 64;
    while (L < N * k) L <<= 1;
    return L;
}

hipError_t launch_tree_expand(const float *score, const int32_t *depth, const int32_t *idx,
                              const float *val, const float *lse, int B, int N, int k, int M,
                              int max_depth, int32_t *new_parent, int32_t *new_token,
                              float *new_score, int32_t *new_depth, hipStream_t s) {
    const int L = tree_expand_slots(N, k);
    if (L <= 2048)
        hipLaunchKernelGGL(k_tree_expand<2048>, dim3(B), dim3(kExpThreads), 0, s, score, depth, idx,
                           val, lse, N, k, M, max_depth, L, new_parent, new_token, new_score,
                           new_depth);
    else
        hipLaunchKernelGGL(k_tree_expand<kExpandMaxCands>, dim3(B), dim3(kExpThreads), 0, s, score,
                           depth, idx, val, lse, N, k, M, max_depth, L, new_parent, new_token,
                           new_score, new_depth);
    return hipGetLastError();
}

}  // namespace jf
