// k_attn.hip -- tree-causal attention of all draft nodes in one pass.
//
// For tree node i and query head h (KV head g = h / G): softmax attention over
// the sequence's prefix keys followed by the keys of i's ancestors (i included)
// -- the visibility rule of the JetFlow blog page, "What JetFlow Does
// Differently", realised as one masked attention over a block appended to the
// prefix ("block-level causal attention", arxivlens methodology / arXiv page
// section 1).
//
// bf16 path (gfx950 MFMA), split over keys:
//   * A sequence's keys are cut into 64-key blocks: ceil(P/64) prefix blocks
//     (read through the page table), then ceil(N/64) tree blocks (the nodes'
//     own K/V).  Consecutive blocks form a split ("chunk"); one workgroup
//     handles one (chunk, KV head, tile of 128 query rows).  Query row
//     r = node * G + (h % G), so the G heads of a node share a mask row.
//   * Per block, each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in
//     registers as B), so each lane ends up owning one query row's scores.
//     The softmax statistics of that row then live in the lane (and its
//     partner lane+32), and O^T = V^T P^T (V^T from LDS as A, P^T straight
//     from the score registers as B) leaves the output row in the same lane:
//     no shuffles besides one max exchange between the two half-waves.
//   * Tree blocks apply the ancestor bitmask: the lane's row reads one 64-bit
//     word per block; a tree block no row of the workgroup can see is skipped.
//   * Online softmax in base 2 with a lazy rescale: the running maximum is
//     only moved when a block's maximum exceeds it by more than 2^8, which
//     keeps every exponent bounded while leaving the arithmetic exact.
//   * K/V tiles are prefetched into registers one block ahead and written to
//     a double-buffered LDS stage (K row-major, V transposed in registers so
//     that the PV operand reads are contiguous in keys); one barrier a block.
//   * Each split writes (O / l, log-sum-exp) partials; a merge kernel combines
//     the splits of a row with LSE weights.  A sequence with one split writes
//     the final output directly.
#include "jf_internal.h"

namespace jf {
namespace {

constexpr int kKB = 64;                  // keys per block
constexpr int kNW = 4;                   // waves per workgroup
constexpr int kTQ = 32 * kNW;            // query rows per workgroup
constexpr int kD = 128;                  // head dim of the bf16 path
constexpr int kKRow = kD * 2 + 16;       // bytes per K row in LDS (padded)
constexpr int kVRow = kKB * 2 + 8;       // bytes per V^T row in LDS (padded)
constexpr int kKTile = kKB * kKRow;
constexpr int kVTile = kD * kVRow;
constexpr int kStage = kKTile + kVTile;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;

struct AttnArgs {
    const uint16_t *q, *k_tree, *v_tree;
    const uint64_t *mask;
    const uint16_t *k_cache, *v_cache;
    const int32_t *block_table;
    void *out;
    float *lse, *part_o, *part_lse;
    int32_t *page_status;
    int64_t num_pages;
    int page_size, max_pages, B, N, Hq, Hkv, G, R, W, n_qt, chunk_blocks, n_tree_blocks,
        total_items;
    float scale, c2, lazy_raw;
    int prefix_len[kMaxBatch];
    int chunk_start[kMaxBatch + 1];
};

__device__ __forceinline__ int find_seq(const AttnArgs &a, int cg) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a.chunk_start[mid] <= cg) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct TileRegs {
    u32x4 k[4];
    u32x4 v[4];
};

// Row offset (in elements) of prefix position pos of sequence b, KV head g, or
// -1 when the page id is out of range.
__device__ __forceinline__ int64_t prefix_row(const AttnArgs &a, int b, int g, int pos) {
    int64_t page;
    int slot;
    if (a.max_pages == 1) {
        page = a.block_table[b * a.max_pages];
        slot = pos;
    } else {
        page = a.block_table[(int64_t)b * a.max_pages + pos / a.page_size];
        slot = pos % a.page_size;
    }
    if (page < 0 || page >= a.num_pages) return -1;
    return ((page * a.page_size + slot) * a.Hkv + g) * (int64_t)kD;
}

__device__ __forceinline__ void load_tile(const AttnArgs &a, int b, int g, int P, int nPB, int kb,
                                          int tid, TileRegs &t, bool &bad_page) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int kc = tid & 15;   // K: 16-byte chunk of a key row
    const int kr = tid >> 4;   // K: key kr + 16 r
    const int vq = tid & 15;   // V: key quad (keys 4 vq .. 4 vq + 3)
    const int vd = tid >> 4;   // V: 8-wide d chunk
    if (kb < nPB) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = kb * kKB + kr + 16 * r;
            t.k[r] = zero;
            if (pos < P) {
                int64_t off = prefix_row(a, b, g, pos);
                if (off >= 0) t.k[r] = *(const u32x4 *)(a.k_cache + off + kc * 8);
                else bad_page = true;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = kb * kKB + 4 * vq + r;
            t.v[r] = zero;
            if (pos < P) {
                int64_t off = prefix_row(a, b, g, pos);
                if (off >= 0) t.v[r] = *(const u32x4 *)(a.v_cache + off + vd * 8);
                else bad_page = true;
            }
        }
    } else {
        const int j0 = (kb - nPB) * kKB;
        const int64_t base = ((int64_t)b * a.N) * a.Hkv + g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + kr + 16 * r;
            t.k[r] = j < a.N ? *(const u32x4 *)(a.k_tree + (base + (int64_t)j * a.Hkv) * kD + kc * 8) : zero;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + 4 * vq + r;
            t.v[r] = j < a.N ? *(const u32x4 *)(a.v_tree + (base + (int64_t)j * a.Hkv) * kD + vd * 8) : zero;
        }
    }
}

__device__ __forceinline__ void store_tile(char *stage, int tid, const TileRegs &t) {
    const int kc = tid & 15, kr = tid >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4 *)(stage + (kr + 16 * r) * kKRow + kc * 16) = t.k[r];
    // V^T: this thread holds V[4vq + r][8vd .. 8vd + 7] for r = 0..3; word w of
    // each row packs d = 8vd + 2w (low half) and 8vd + 2w + 1 (high half).
    char *vt = stage + kKTile;
    const int vq = tid & 15, vd = tid >> 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = t.v[0][w], a1 = t.v[1][w], a2 = t.v[2][w], a3 = t.v[3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        *(u32x2 *)(vt + (8 * vd + 2 * w) * kVRow + vq * 8) = lo;
        *(u32x2 *)(vt + (8 * vd + 2 * w + 1) * kVRow + vq * 8) = hi;
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 cvt8(const f32x16 &s, int base) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(s[base + 2 * j], s[base + 2 * j + 1]);
    return as_bf16x8(w);
}

__global__ __launch_bounds__(kNW * kWave) void k_tree_attn_split(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
    __shared__ uint32_t s_used;
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    // ---- work item ----
    const int item = xcd_remap(blockIdx.x, a.total_items);
    const int qt = item % a.n_qt;
    const int tmp = item / a.n_qt;
    const int g = tmp % a.Hkv;
    const int cg = tmp / a.Hkv;
    const int b = find_seq(a, cg);
    const int c = cg - a.chunk_start[b];
    const int nchunks = a.chunk_start[b + 1] - a.chunk_start[b];
    const int P = a.prefix_len[b];
    const int nPB = (P + kKB - 1) / kKB;
    const int nB = nPB + a.n_tree_blocks;
    const int kb0 = c * a.chunk_blocks;
    const int kb1 = min(kb0 + a.chunk_blocks, nB);

    // ---- this lane's query row ----
    const int r = qt * kTQ + wave * 32 + l32;
    const bool row_ok = r < a.R;
    const int node = row_ok ? r / a.G : 0;
    const int hq = g * a.G + (row_ok ? r % a.G : 0);
    bf16x8 qf[kD / 16];
    {
        const uint16_t *qrow = a.q + (((int64_t)b * a.N + node) * a.Hq + hq) * kD + half * 8;
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *(const u32x4 *)(qrow + t * 16);
            qf[t] = as_bf16x8(v);
        }
    }
    const uint64_t *mrow = a.mask + ((int64_t)b * a.N + node) * a.W;

    // ---- which tree blocks of this chunk does any row of the tile see? ----
    if (tid == 0) { s_used = 0u; s_bad = 0; }
    __syncthreads();
    if (kb1 > nPB && tid < kTQ) {
        const int rr = qt * kTQ + tid;
        if (rr < a.R) {
            const uint64_t *mr = a.mask + ((int64_t)b * a.N + rr / a.G) * a.W;
            uint32_t bits = 0;
            for (int kb = max(kb0, nPB); kb < kb1; ++kb)
                if (mr[kb - nPB] != 0ull) bits |= 1u << (kb - nPB);
            if (bits) atomicOr(&s_used, bits);
        }
    }
    __syncthreads();
    const uint32_t used = s_used;
    auto usable = [&](int kb) { return kb < nPB || ((used >> (kb - nPB)) & 1u); };
    auto next_block = [&](int kb) {
        ++kb;
        while (kb < kb1 && !usable(kb)) ++kb;
        return kb;
    };

    f32x16 o[kD / 32];
#pragma unroll
    for (int d = 0; d < kD / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    bool bad_page = false;

    int kb = kb0;
    while (kb < kb1 && !usable(kb)) ++kb;
    TileRegs tr;
    uint64_t word = 0ull;
    if (kb < kb1) {
        load_tile(a, b, g, P, nPB, kb, tid, tr, bad_page);
        store_tile(smem, tid, tr);
        if (kb >= nPB && row_ok) word = mrow[kb - nPB];
    }
    __syncthreads();
    int buf = 0;
    while (kb < kb1) {
        const int kbn = next_block(kb);
        uint64_t word_n = 0ull;
        if (kbn < kb1) {
            load_tile(a, b, g, P, nPB, kbn, tid, tr, bad_page);
            if (kbn >= nPB && row_ok) word_n = mrow[kbn - nPB];
        }
        const char *stage = smem + buf * kStage;

        // S^T (keys x rows) for the two 32-key halves of the block
        f32x16 s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
        {
            const char *k0p = stage + l32 * kKRow + half * 16;
            const char *k1p = k0p + 32 * kKRow;
#pragma unroll
            for (int t = 0; t < kD / 16; ++t) {
                bf16x8 ka = *(const bf16x8 *)(k0p + t * 32);
                bf16x8 kbv = *(const bf16x8 *)(k1p + t * 32);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[t], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbv, qf[t], s1, 0, 0, 0);
            }
        }
        // register i of a half holds key (i/4)*8 + half*4 + i%4 (+32 for s1)
        const bool is_tree = kb >= nPB;
        const bool tail = !is_tree && (kb + 1) * kKB > P;
        if (is_tree) {
            const int jbase = (kb - nPB) * kKB;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = (i >> 2) * 8 + half * 4 + (i & 3);
                const bool v0 = ((word >> key) & 1ull) && (jbase + key < a.N);
                const bool v1 = ((word >> (key + 32)) & 1ull) && (jbase + key + 32 < a.N);
                s0[i] = v0 ? s0[i] : -INFINITY;
                s1[i] = v1 ? s1[i] : -INFINITY;
            }
        } else if (tail) {
            const int lim = P - kb * kKB;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = (i >> 2) * 8 + half * 4 + (i & 3);
                s0[i] = key < lim ? s0[i] : -INFINITY;
                s1[i] = key + 32 < lim ? s1[i] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx > m_run + a.lazy_raw;
        if (__ballot(need)) {
            const float m_new = need ? mx : m_run;
            const float alpha = need ? __builtin_amdgcn_exp2f((m_run - m_new) * a.c2) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
            m_run = m_new;
        }
        const float base = m_run == -INFINITY ? 0.f : m_run * a.c2;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], a.c2, -base));
            s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], a.c2, -base));
            l_run += s0[i] + s1[i];
        }
        bf16x8 p[4];
        p[0] = cvt8(s0, 0);
        p[1] = cvt8(s0, 8);
        p[2] = cvt8(s1, 0);
        p[3] = cvt8(s1, 8);

        // O^T (d x rows) += V^T P^T
        {
            const char *vt = stage + kKTile + l32 * kVRow + half * 8;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d) {
                const char *vrow = vt + d * 32 * kVRow;
#pragma unroll
                for (int st = 0; st < 4; ++st) {  // k-step: keys (st/2)*32 + (st%2)*16 ...
                    const int key0 = (st >> 1) * 32 + (st & 1) * 16;
                    u32x2 lo = *(const u32x2 *)(vrow + key0 * 2);
                    u32x2 hi = *(const u32x2 *)(vrow + (key0 + 8) * 2);
                    u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), p[st], o[d], 0, 0, 0);
                }
            }
        }

        if (kbn < kb1) store_tile(smem + (buf ^ 1) * kStage, tid, tr);
        __syncthreads();
        buf ^= 1;
        kb = kbn;
        word = word_n;
    }

    if (bad_page) s_bad = 1;  // benign race: every writer stores 1
    l_run += __shfl_xor(l_run, 32);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse_v = l_run > 0.f ? m_run * a.scale + logf(l_run) : -INFINITY;
    if (row_ok) {
        if (nchunks == 1) {
            const int64_t orow = ((int64_t)b * a.N + node) * a.Hq + hq;
            uint16_t *op = (uint16_t *)a.out + orow * kD + half * 4;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    u32x2 w;
                    w[0] = pack_bf16x2(o[d][gi * 4 + 0] * inv, o[d][gi * 4 + 1] * inv);
                    w[1] = pack_bf16x2(o[d][gi * 4 + 2] * inv, o[d][gi * 4 + 3] * inv);
                    *(u32x2 *)(op + d * 32 + gi * 8) = w;
                }
            if (a.lse && half == 0) a.lse[orow] = lse_v;
        } else {
            const int64_t prow = ((int64_t)cg * a.Hkv + g) * a.R + r;
            float *op = a.part_o + prow * kD + half * 4;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    f32x4 w = {o[d][gi * 4 + 0] * inv, o[d][gi * 4 + 1] * inv,
                               o[d][gi * 4 + 2] * inv, o[d][gi * 4 + 3] * inv};
                    *(f32x4 *)(op + d * 32 + gi * 8) = w;
                }
            if (half == 0) a.part_lse[prow] = lse_v;
        }
    }
    __syncthreads();
    if (tid == 0 && s_bad && a.page_status) *a.page_status = JF_ERR_BAD_PAGE;
}

// Combine the splits of one row: O = sum_s w_s O_s / sum_s w_s with
// w_s = exp(lse_s - max lse); lse = max + log sum w_s.  One wave per row.
__global__ __launch_bounds__(256) void k_tree_attn_merge(AttnArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t flat = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t total = (int64_t)a.B * a.N * a.Hq;
    if (flat >= total) return;
    const int hq = (int)(flat % a.Hq);
    const int node = (int)((flat / a.Hq) % a.N);
    const int b = (int)(flat / ((int64_t)a.Hq * a.N));
    const int c0 = a.chunk_start[b];
    const int nc = a.chunk_start[b + 1] - c0;
    if (nc == 1) return;
    const int g = hq / a.G;
    const int r = node * a.G + hq % a.G;
    float M = -INFINITY;
    for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_lse[((int64_t)(c0 + c) * a.Hkv + g) * a.R + r]);
    float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
    for (int c = 0; c < nc; ++c) {
        const int64_t prow = ((int64_t)(c0 + c) * a.Hkv + g) * a.R + r;
        const float l = a.part_lse[prow];
        const float w = l == -INFINITY ? 0.f : expf(l - M);
        const float2 v = *(const float2 *)(a.part_o + prow * kD + 2 * lane);
        acc0 += w * v.x;
        acc1 += w * v.y;
        wsum += w;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t *op = (uint16_t *)a.out + flat * kD + 2 * lane;
    *(uint32_t *)op = pack_bf16x2(acc0 * inv, acc1 * inv);
    if (a.lse && lane == 0) a.lse[flat] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 path: one wavefront per (sequence, node, query head); keys are taken 64
// at a time (one per lane), scores in fp32, online softmax with expf, each lane
// accumulating D/64 output columns.  Meant for small problems.
struct AttnArgsF32 {
    const float *q, *k_tree, *v_tree;
    const uint64_t *mask;
    const float *k_cache, *v_cache;
    const int32_t *block_table;
    float *out, *lse;
    int32_t *page_status;
    int64_t num_pages;
    int page_size, max_pages, B, N, Hq, Hkv, G, W, D;
    float scale;
    int prefix_len[kMaxBatch];
};

constexpr int kF32MaxD = 128;

__global__ __launch_bounds__(256) void k_tree_attn_f32(AttnArgsF32 a) {
    __shared__ float sq[4][kF32MaxD];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t flat = (int64_t)blockIdx.x * 4 + wv;
    const int64_t total = (int64_t)a.B * a.N * a.Hq;
    if (flat >= total) return;
    const int hq = (int)(flat % a.Hq);
    const int node = (int)((flat / a.Hq) % a.N);
    const int b = (int)(flat / ((int64_t)a.Hq * a.N));
    const int g = hq / a.G;
    const int D = a.D;
    const int P = a.prefix_len[b];
    for (int d = lane; d < D; d += 64) sq[wv][d] = a.q[flat * D + d];
    __builtin_amdgcn_wave_barrier();
    const uint64_t *mrow = a.mask + ((int64_t)b * a.N + node) * a.W;
    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    bool bad = false;
    const int nkeys = P + a.N;
    for (int kc = 0; kc < nkeys; kc += 64) {
        const int key = kc + lane;
        bool valid = false;
        int64_t off = 0;
        const float *kbase = a.k_cache, *vbase = a.v_cache;
        if (key < P) {
            int64_t page = a.block_table[(int64_t)b * a.max_pages + key / a.page_size];
            if (page >= 0 && page < a.num_pages) {
                off = ((page * a.page_size + key % a.page_size) * a.Hkv + g) * (int64_t)D;
                valid = true;
            } else {
                bad = true;
            }
        } else if (key < nkeys) {
            const int j = key - P;
            valid = (mrow[j >> 6] >> (j & 63)) & 1ull;
            off = (((int64_t)b * a.N + j) * a.Hkv + g) * (int64_t)D;
            kbase = a.k_tree;
            vbase = a.v_tree;
        }
        float s = -INFINITY;
        if (valid) {
            const float *kr = kbase + off;
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(sq[wv][d], kr[d], dot);
            s = dot * a.scale;
        }
        float cm = s;
        for (int o = 32; o >= 1; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
        const float mn = fmaxf(m, cm);
        const float base = mn == -INFINITY ? 0.f : mn;
        const float p = valid ? expf(s - base) : 0.f;
        const float alpha = expf(m - base);
        float ps = p;
        for (int o = 32; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
        l = l * alpha + ps;
        acc0 *= alpha;
        acc1 *= alpha;
        const float *vrow_base = vbase;
        for (int jj = 0; jj < 64; ++jj) {
            const float pj = __shfl(p, jj);
            if (pj == 0.f) continue;  // uniform across the wave
            const int64_t oj = __shfl(off, jj);
            const bool tree_j = (kc + jj) >= P;
            const float *vr = (tree_j ? a.v_tree : a.v_cache) + oj;
            if (lane < D) acc0 = fmaf(pj, vr[lane], acc0);
            if (lane + 64 < D) acc1 = fmaf(pj, vr[lane + 64], acc1);
        }
        (void)vrow_base;
        m = mn;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (lane < D) a.out[flat * D + lane] = acc0 * inv;
    if (lane + 64 < D) a.out[flat * D + lane + 64] = acc1 * inv;
    if (a.lse && lane == 0) a.lse[flat] = l > 0.f ? m + logf(l) : -INFINITY;
    if (bad && a.page_status) *a.page_status = JF_ERR_BAD_PAGE;
}

}  // namespace

// ---------------------------------------------------------------------------
// Split planning.  Every (sequence, KV head, query tile) is a row of blocks;
// cut all rows into splits of the same block count so that about two
// workgroups per compute unit come out, never less than two blocks a split.
void plan_tree_attn(AttnPlan &p, int B, int N, int Hq, int Hkv, int D,
                    const int32_t *prefix_len, jf_dtype dtype) {
    p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.D = D;
    p.G = Hq / Hkv;
    p.R = N * p.G;
    p.W = (N + 63) / 64;
    p.tq = kTQ;
    p.n_qt = (p.R + kTQ - 1) / kTQ;
    p.n_tree_blocks = (N + kKB - 1) / kKB;
    int64_t units = 0;
    int max_blocks = 1;
    for (int b = 0; b < B; ++b) {
        p.prefix_len[b] = prefix_len[b];
        int nb = (prefix_len[b] + kKB - 1) / kKB + p.n_tree_blocks;
        units += (int64_t)nb;
        if (nb > max_blocks) max_blocks = nb;
    }
    units *= (int64_t)Hkv * p.n_qt;
    const int64_t target = 2 * (int64_t)num_cus();
    int64_t cb = (units + target - 1) / target;
    if (cb < 2) cb = 2;
    if (cb > max_blocks) cb = max_blocks;
    if (dtype == JF_F32) cb = max_blocks;  // the fp32 path does not split
    p.chunk_blocks = (int)cb;
    int cs = 0;
    p.any_split = false;
    for (int b = 0; b < B; ++b) {
        p.chunk_start[b] = cs;
        int nb = (prefix_len[b] + kKB - 1) / kKB + p.n_tree_blocks;
        int nc = (nb + p.chunk_blocks - 1) / p.chunk_blocks;
        if (nc > 1) p.any_split = true;
        cs += nc;
    }
    p.chunk_start[B] = cs;
    p.total_chunks = cs;
    p.total_items = cs * Hkv * p.n_qt;
}

size_t tree_attn_workspace_bytes(const AttnPlan &p) {
    if (!p.any_split) return 0;
    const size_t rows = (size_t)p.total_chunks * p.Hkv * p.R;
    size_t o = rows * kD * sizeof(float);
    o = (o + 255) / 256 * 256;
    return o + rows * sizeof(float);
}

hipError_t launch_tree_attn_bf16(const AttnPlan &p, const void *q, const void *k_tree,
                                 const void *v_tree, const uint64_t *mask, const void *k_cache,
                                 const void *v_cache, int64_t num_pages, int page_size,
                                 const int32_t *block_table, int max_pages, float scale, void *out,
                                 float *lse, void *workspace, int32_t *page_status, hipStream_t s) {
    AttnArgs a;
    a.q = (const uint16_t *)q;
    a.k_tree = (const uint16_t *)k_tree;
    a.v_tree = (const uint16_t *)v_tree;
    a.mask = mask;
    a.k_cache = (const uint16_t *)k_cache;
    a.v_cache = (const uint16_t *)v_cache;
    a.block_table = block_table;
    a.out = out;
    a.lse = lse;
    const size_t rows = (size_t)p.total_chunks * p.Hkv * p.R;
    size_t obytes = (rows * kD * sizeof(float) + 255) / 256 * 256;
    a.part_o = p.any_split ? (float *)workspace : nullptr;
    a.part_lse = p.any_split ? (float *)((char *)workspace + obytes) : nullptr;
    a.page_status = page_status;
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.max_pages = max_pages;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.R = p.R; a.W = p.W;
    a.n_qt = p.n_qt;
    a.chunk_blocks = p.chunk_blocks;
    a.n_tree_blocks = p.n_tree_blocks;
    a.total_items = p.total_items;
    a.scale = scale;
    a.c2 = scale * kLog2e;
    a.lazy_raw = kLazyLog2 / a.c2;
    for (int b = 0; b < p.B; ++b) a.prefix_len[b] = p.prefix_len[b];
    for (int b = 0; b <= p.B; ++b) a.chunk_start[b] = p.chunk_start[b];
    hipLaunchKernelGGL(k_tree_attn_split, dim3(p.total_items), dim3(kNW * kWave), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.any_split) return e;
    const int64_t total = (int64_t)p.B * p.N * p.Hq;
    hipLaunchKernelGGL(k_tree_attn_merge, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tree_attn_f32(const AttnPlan &p, const float *q, const float *k_tree,
                                const float *v_tree, const uint64_t *mask, const float *k_cache,
                                const float *v_cache, int64_t num_pages, int page_size,
                                const int32_t *block_table, int max_pages, float scale,
                                float *out, float *lse, int32_t *page_status, hipStream_t s) {
    AttnArgsF32 a;
    a.q = q; a.k_tree = k_tree; a.v_tree = v_tree; a.mask = mask;
    a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.out = out; a.lse = lse; a.page_status = page_status;
    a.num_pages = num_pages; a.page_size = page_size; a.max_pages = max_pages;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.W = p.W; a.D = p.D;
    a.scale = scale;
    for (int b = 0; b < p.B; ++b) a.prefix_len[b] = p.prefix_len[b];
    const int64_t total = (int64_t)p.B * p.N * p.Hq;
    hipLaunchKernelGGL(k_tree_attn_f32, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace jf
