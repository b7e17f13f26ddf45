// k_tree.hip -- path scores of draft-tree nodes, one budgeted best-first
// expansion of the tree, and greedy verification of a drafted tree.
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
//   k_tree_expand : one workgroup per sequence; the candidates that are
//                   already children in the tree are marked in an LDS bitmap;
//                   every other (node, rank) candidate
//                   becomes one 64-bit key that orders (score desc, node asc,
//                   rank asc); the M smallest keys are found with a score-bin
//                   histogram and ranks counted inside a bin (a full bitonic
//                   sort when a bin near the cut is crowded), and decode into
//                   the new nodes.
//   k_tree_accept : one workgroup per sequence; each lane walks its nodes'
//                   chains checking the target's tokens; the deepest fully
//                   accepted node and its path are written.
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
constexpr int kExpThreads = 256;           // four wavefronts
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

__device__ __forceinline__ uint64_t lane_xor(uint64_t v, int m) {
    const int src = (((int)threadIdx.x & 63) ^ m) << 2;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Compare-exchange of the slot pairs (r, r ^ J) inside one lane's registers,
// toward ascending order in runs of length kk (descending in odd runs).
template <int R, int J>
__device__ __forceinline__ void local_step(uint64_t (&key)[R], int e0, int kk) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r & J) continue;
        const bool up = ((e0 + r) & kk) == 0;
        const uint64_t a = key[r], c = key[r | J];
        const bool swap = (a > c) == up;
        key[r] = swap ? c : a;
        key[r | J] = swap ? a : c;
    }
}

template <int R>
__device__ __forceinline__ void local_steps(uint64_t (&key)[R], int e0, int kk, int j) {
    // strides below R, largest first
    if constexpr (R > 32) if (j >= 32) local_step<R, 32>(key, e0, kk);
    if constexpr (R > 16) if (j >= 16) local_step<R, 16>(key, e0, kk);
    if constexpr (R > 8) if (j >= 8) local_step<R, 8>(key, e0, kk);
    if constexpr (R > 4) if (j >= 4) local_step<R, 4>(key, e0, kk);
    if constexpr (R > 2) if (j >= 2) local_step<R, 2>(key, e0, kk);
    if constexpr (R > 1) local_step<R, 1>(key, e0, kk);
}

// Bitonic sort of the L = 256*R keys held R per lane (slot e = thread*R + r),
// ascending.  Strides j < R stay in a lane's registers, R <= j < 64R pair
// lanes of one wavefront (cross-lane moves), j >= 64R pair wavefronts through
// LDS.  Used when a selection bin near the top is crowded (mass ties).
template <int R>
__device__ __forceinline__ void bitonic_sort(uint64_t (&key)[R], uint64_t *lds, int e0) {
    constexpr int L = kExpThreads * R;
    const int lane = threadIdx.x & 63;
    for (int kk = 2; kk <= L; kk <<= 1) {
        int j = kk >> 1;
        for (; j >= 64 * R; j >>= 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) lds[e0 + r] = key[r];
            __syncthreads();
            const bool lower = (e0 & j) == 0, up = (e0 & kk) == 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t o = lds[(e0 + r) ^ j];
                const uint64_t mn = key[r] < o ? key[r] : o, mx = key[r] < o ? o : key[r];
                key[r] = (up == lower) ? mn : mx;
            }
            __syncthreads();
        }
        for (; j >= R; j >>= 1) {
            const int m = j / R;
            const bool lower = (lane & m) == 0, up = (e0 & kk) == 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t o = lane_xor(key[r], m);
                const uint64_t mn = key[r] < o ? key[r] : o, mx = key[r] < o ? o : key[r];
                key[r] = (up == lower) ? mn : mx;
            }
        }
        if (j >= 1) local_steps<R>(key, e0, kk, j);
    }
}

constexpr int kSelBins = 1024;          // selection histogram bins
constexpr int kSelMaxBin = 96;          // larger bin at or above the cut: sort instead

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ m) << 2,
                                                                  __float_as_int(v))));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fminf(v, __int_as_float(__builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ m) << 2,
                                                                  __float_as_int(v))));
    return v;
}

// Inclusive prefix sum across a wavefront: shifts of 1, 2, 4 and 8 lanes
// inside each row of 16 (DPP row_shr, zero from outside the row), then the
// last lane of row 0 into rows 1 and 3 and of row 1 into rows 2 and 3
// (row_bcast:15 / row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return (uint32_t)x;
}

// One workgroup per sequence, R candidate slots per lane (slot e =
// thread*R + r).  Selection of the M best keys:
//   1. bins: bin(s) = floor((s_max - s) * kSelBins / (s_max - s_min)), clamped
//      to [0, kSelBins); non-increasing in s, so a lower bin holds only
//      strictly better scores and equal scores share a bin;
//   2. an LDS histogram whose atomic return value is each key's place in its
//      bin; one scan gives each bin's offset and the cut bin c, the first bin
//      whose inclusive count reaches M;
//   3. the keys of bins <= c go to their bin's segment of an LDS array, and
//      each one's rank is its bin offset plus the number of smaller keys in
//      its segment; ranks below M are output slots.
// A bin of more than kSelMaxBin keys at or below the cut (mass ties) switches
// the workgroup to the full bitonic sort.
// A candidate (p, r) whose token idx[p][r] some node j of the tree already
// carries as a child of p (parent[j] == p, token[j] == idx[p][r]) is not
// eligible: the step grows the tree as it stands, and a second child with
// the same token would be the same branch twice.
template <int R>
__global__ __launch_bounds__(kExpThreads) void k_tree_expand(
    const float *__restrict__ score, const int32_t *__restrict__ depth,
    const int32_t *__restrict__ idx, const float *__restrict__ val, const float *__restrict__ lse,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ token,
    int N, int k, int M, int max_depth, int32_t *__restrict__ new_parent,
    int32_t *__restrict__ new_token, float *__restrict__ new_score,
    int32_t *__restrict__ new_depth) {
    constexpr int L = kExpThreads * R;
    __shared__ uint64_t lds[L];
    __shared__ uint32_t hist[kSelBins];
    __shared__ uint32_t boff[kSelBins];
    __shared__ float red[2][kExpThreads / 64];
    __shared__ int sel[3];                  // cut bin, eligible count, use the sort
    __shared__ uint32_t taken[kExpandMaxCands / 32];   // bit p*k + r: already a child
    const int b = blockIdx.x;
    const int nc = N * k;
    const int64_t nbase = (int64_t)b * N;
    const int64_t cbase = nbase * k;
    const int e0 = threadIdx.x * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    for (int i = threadIdx.x; i < kSelBins; i += kExpThreads) hist[i] = 0;
    for (int i = threadIdx.x; i < (nc + 31) / 32; i += kExpThreads) taken[i] = 0u;

    // Keys: high word ~ord(score) (descending score first), low word the flat
    // candidate index p*k + r (node ascending, then rank ascending).  Every
    // slot issues its loads unconditionally (indices clamped into range), so a
    // lane's loads are in flight together instead of one slot after another.
    int pr[R];
    int32_t dr[R], tk[R];
    float vr[R], lr[R], sr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = min(e0 + r, nc - 1);
        pr[r] = e / k;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = min(e0 + r, nc - 1);
        dr[r] = depth[nbase + pr[r]];
        vr[r] = val[cbase + e];
        lr[r] = lse[nbase + pr[r]];
        sr[r] = score[nbase + pr[r]];
        tk[r] = idx[cbase + e];
    }
    // Pin the loaded values here so no pass sinks a load back into the
    // eligibility branch below (that would serialise the round trips again).
#pragma unroll
    for (int r = 0; r < R; ++r)
        asm volatile("" : "+v"(dr[r]), "+v"(vr[r]), "+v"(lr[r]), "+v"(sr[r]), "+v"(tk[r]));
    __syncthreads();                          // taken[] cleared
    // Mark the candidates that are already children: node j is the child of
    // parent[j] carrying token[j], so the rank of that token in the parent's
    // list (if it is listed) is taken.
#pragma unroll 4
    for (int j = threadIdx.x; j < N; j += kExpThreads) {
        const int p = parent[nbase + j];
        const int32_t t = token[nbase + j];
        if (p < 0 || p >= N) continue;        // a root, or a parent that names no node
        const int32_t *row = idx + cbase + (int64_t)p * k;
        for (int r = 0; r < k; ++r)
            if (row[r] == t) atomicOr(&taken[(p * k + r) >> 5], 1u << ((p * k + r) & 31));
    }
    __syncthreads();
    uint64_t key[R];
    float sc[R];
    float smax = -__builtin_inff(), smin = __builtin_inff();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = e0 + r;
        const float t = vr[r] - lr[r];            // rounded to fp32
        sc[r] = sr[r] + t;                        // rounded to fp32
        // eligible: child depth d + 1 <= max_depth, not already a child
        const bool ok = e < nc && dr[r] >= 1 && dr[r] < max_depth &&
                        !((taken[min(e, nc - 1) >> 5] >> (e & 31)) & 1u);
        key[r] = ok ? (((uint64_t)(~ord_f32(sc[r])) << 32) | (uint32_t)e) : kNoCand;
        if (ok && __builtin_isfinite(sc[r])) {
            smax = fmaxf(smax, sc[r]);
            smin = fminf(smin, sc[r]);
        }
    }
    smax = wave_max(smax);
    smin = wave_min(smin);
    if (lane == 0) {
        red[0][wave] = smax;
        red[1][wave] = smin;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kExpThreads / 64; ++w) {
        smax = fmaxf(smax, red[0][w]);
        smin = fminf(smin, red[1][w]);
    }
    // Bin width from the finite range (0 when there is no range: one bin).
    const float inv_w = smax > smin ? (float)kSelBins / (smax - smin) : 0.f;

    int bin[R];
    uint32_t pos[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float x = (smax - sc[r]) * inv_w;         // NaN only for s = +inf with no range
        x = x >= 0.f ? x : 0.f;                   // s above the finite maximum (+inf)
        bin[r] = (int)fminf(x, (float)(kSelBins - 1));
        pos[r] = key[r] != kNoCand ? atomicAdd(&hist[bin[r]], 1u) : 0u;
    }
    __syncthreads();

    // Wave 0: exclusive bin offsets, the cut bin and the crowding test.
    if (wave == 0) {
        constexpr int PER = kSelBins / 64;
        uint32_t c[PER];
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            c[i] = hist[lane * PER + i];
            sum += c[i];
        }
        const uint32_t incl = wave_incl_scan(sum);   // inclusive scan of lane sums
        const uint32_t total = (uint32_t)__builtin_amdgcn_ds_bpermute(63 << 2, (int)incl);
        const uint32_t need = min((uint32_t)M, total);
        uint32_t run = incl - sum;
        int cut = kSelBins;                       // first bin whose inclusive count reaches need
        uint32_t crowd = 0;                       // largest bin at or below the cut
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            boff[lane * PER + i] = run;
            const uint32_t before = run;
            run += c[i];
            if (before < need) crowd = max(crowd, c[i]);
            if (cut == kSelBins && run >= need && need > 0) cut = lane * PER + i;
        }
        // smallest cut over lanes, largest crowding over lanes
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            cut = min(cut, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, cut));
            crowd = max(crowd, (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)crowd));
        }
        if (lane == 0) {
            sel[0] = cut;
            sel[1] = (int)total;
            sel[2] = crowd > (uint32_t)kSelMaxBin;
        }
    }
    __syncthreads();
    const int cut = sel[0], n_elig = sel[1];

    int rank[R];
    if (!sel[2]) {
        // scatter the keys at or below the cut into their bins' segments
        // (indices are in range by construction; the clamps keep every LDS
        // access inside the array whatever the offsets hold)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (key[r] != kNoCand && bin[r] <= cut) lds[min((int)(boff[bin[r]] + pos[r]), L - 1)] = key[r];
        __syncthreads();
        // rank = bin offset + smaller keys in the bin; the R keys' segment
        // scans run side by side (a key outside the cut scans nothing)
        int o[R], n[R], less[R];
        int nmax = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool in = key[r] != kNoCand && bin[r] <= cut;
            o[r] = in ? (int)boff[bin[r]] : 0;
            n[r] = in ? (int)hist[bin[r]] : 0;
            less[r] = 0;
            nmax = max(nmax, n[r]);
        }
        for (int i = 0; i < nmax; ++i) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint64_t v = lds[min(o[r] + min(i, max(n[r] - 1, 0)), L - 1)];
                less[r] += (i < n[r]) & (v < key[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) rank[r] = n[r] > 0 ? o[r] + less[r] : -1;
    } else {
        bitonic_sort<R>(key, lds, e0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            rank[r] = key[r] != kNoCand ? e0 + r : -1;
            // the sort moved the keys: gather their tokens and depths
            const int e = rank[r] >= 0 ? (int)(uint32_t)key[r] : 0;
            tk[r] = idx[cbase + e];
            dr[r] = depth[nbase + e / k];
        }
    }

    // Keys with rank < M are the new nodes.
    const int64_t obase = (int64_t)b * M;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int m = rank[r];
        if (m < 0 || m >= M) continue;
        const int e = (int)(uint32_t)key[r];
        new_parent[obase + m] = e / k;
        new_token[obase + m] = tk[r];
        new_score[obase + m] = unord_f32(~(uint32_t)(key[r] >> 32));
        new_depth[obase + m] = dr[r] + 1;
    }
    // Budget slots beyond the eligible candidates are empty.
    for (int m = n_elig + threadIdx.x; m < M; m += kExpThreads) {
        new_parent[obase + m] = -2;
        new_token[obase + m] = -1;
        new_score[obase + m] = -__builtin_inff();
        new_depth[obase + m] = 0;
    }
}


// ---------------------------------------------------------------------------
// Greedy verification: node i is accepted when its token is the target's next
// token after its parent (after the prefix for a root) and every ancestor is
// accepted; the deepest accepted node wins, ties to the lower index.  One
// workgroup per sequence with parents, tokens and the target's tokens in LDS.
constexpr int kAccThreads = 256;

__global__ __launch_bounds__(kAccThreads) void k_tree_accept(
    const int32_t *__restrict__ parent, const int32_t *__restrict__ token,
    const int32_t *__restrict__ target_next, const int32_t *__restrict__ root_next, int N,
    int32_t *__restrict__ accept_len, int32_t *__restrict__ accept_node,
    int32_t *__restrict__ next_token, int32_t *__restrict__ path,
    int32_t *__restrict__ seq_status) {
    __shared__ int32_t par[kPathMaxN];
    __shared__ int32_t tok[kPathMaxN];
    __shared__ int32_t nxt[kPathMaxN];
    __shared__ int32_t first_bad;
    __shared__ int32_t best;                  // depth * 8192 + (8191 - node), 0: none
    const int b = blockIdx.x;
    const int64_t base = (int64_t)b * N;
    for (int i = threadIdx.x; i < N; i += kAccThreads) {
        par[i] = parent[base + i];
        tok[i] = token[base + i];
        nxt[i] = target_next[base + i];
    }
    if (threadIdx.x == 0) {
        first_bad = INT32_MAX;
        best = 0;
    }
    const int32_t root = root_next[b];
    __syncthreads();

    for (int i = threadIdx.x; i < N; i += kAccThreads) {
        int j = i, steps = 0;
        bool ok = true, acc = true;
        while (j != -1) {
            if (j < -1 || j >= N || steps >= N) { ok = false; break; }
            const int pj = par[j];
            const int32_t pred = pj == -1 ? root : (pj >= 0 && pj < N ? nxt[pj] : -1);
            acc = acc && tok[j] == pred;
            j = pj;
            ++steps;
        }
        if (!ok) atomicMin(&first_bad, i);
        else if (acc) atomicMax(&best, steps * 8192 + (8191 - i));
    }
    __syncthreads();

    const bool bad = first_bad != INT32_MAX;
    const int key = bad ? 0 : best;
    const int len = key >> 13;
    const int node = key ? 8191 - (key & 8191) : -1;
    // Path slot d holds the ancestor of `node` at depth d + 1: lane 0 walks
    // up once and writes slots len-1 .. 0; the other slots read -1.
    if (path) {
        for (int d = len + threadIdx.x; d < N; d += kAccThreads) path[base + d] = -1;
        if (threadIdx.x == 0)
            for (int a = node, d = len - 1; d >= 0; a = par[a], --d) path[base + d] = a;
    }
    if (threadIdx.x == 0) {
        accept_len[b] = len;
        accept_node[b] = node;
        next_token[b] = node >= 0 ? nxt[node] : root;
        if (seq_status) seq_status[b] = bad ? first_bad : -1;
    }
}

}  // namespace

hipError_t launch_path_scores(const int32_t *parent, const float *logp, int B, int N, float *score,
                              int32_t *seq_status, hipStream_t s) {
    hipLaunchKernelGGL(k_path_scores, dim3(B), dim3(kPathThreads), 0, s, parent, logp, N, score,
                       seq_status);
    return hipGetLastError();
}

hipError_t launch_tree_accept(const int32_t *parent, const int32_t *token,
                              const int32_t *target_next, const int32_t *root_next, int B, int N,
                              int32_t *accept_len, int32_t *accept_node, int32_t *next_token,
                              int32_t *path, int32_t *seq_status, hipStream_t s) {
    hipLaunchKernelGGL(k_tree_accept, dim3(B), dim3(kAccThreads), 0, s, parent, token, target_next,
                       root_next, N, accept_len, accept_node, next_token, path, seq_status);
    return hipGetLastError();
}

hipError_t launch_tree_expand(const float *score, const int32_t *depth, const int32_t *idx,
                              const float *val, const float *lse, const int32_t *parent,
                              const int32_t *token, int B, int N, int k, int M,
                              int max_depth, int32_t *new_parent, int32_t *new_token,
                              float *new_score, int32_t *new_depth, hipStream_t s) {
    int R = 1;                                    // slots per lane: 256*R >= N*k
    while (kExpThreads * R < N * k) R <<= 1;
#define JF_EXPAND(RR)                                                                            \
    hipLaunchKernelGGL(k_tree_expand<RR>, dim3(B), dim3(kExpThreads), 0, s, score, depth, idx,   \
                       val, lse, parent, token, N, k, M, max_depth, new_parent, new_token,         \
                       new_score, new_depth)
    switch (R) {
        case 1: JF_EXPAND(1); break;
        case 2: JF_EXPAND(2); break;
        case 4: JF_EXPAND(4); break;
        case 8: JF_EXPAND(8); break;
        case 16: JF_EXPAND(16); break;
        case 32: JF_EXPAND(32); break;
        case 64: JF_EXPAND(64); break;
        default: return hipErrorInvalidValue;
    }
#undef JF_EXPAND
    return hipGetLastError();
}

}  // namespace jf
