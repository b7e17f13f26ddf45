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
//   * K and V tiles go straight from HBM into LDS (buffer_load ... lds, 16
//     bytes a lane) one block ahead, into a double-buffered stage; no
//     registers are spent on the prefetch.  One copy instruction fills 1 KiB
//     of LDS; block n of a tile holds rows n, n+16, n+32, n+48, and the
//     blocks are padded (16 bytes for K, 64 for V) so that both the K operand
//     reads (ds_read_b128) and the V operand reads hit distinct banks, while
//     every operand address is one base register plus an immediate.  V stays
//     row-major:
//     ds_read_b64_tr_b16 hands each lane four consecutive keys of one head-dim
//     column, which is exactly the V^T operand layout.  One wait + barrier a
//     block.
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
constexpr int kRow = kD * 2;             // bytes per K or V row
constexpr int kKBlk = 4 * kRow + 16;     // LDS block of 4 K rows (n, n+16, n+32, n+48)
constexpr int kVBlk = 4 * kRow + 64;     // LDS block of 4 V rows
constexpr int kKTile = 16 * kKBlk;
constexpr int kVTile = 16 * kVBlk;
constexpr int kStage = kKTile + kVTile;  // K tile then V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;

struct AttnArgs {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const uint64_t *mask;
    const int32_t *block_table;
    void *out;
    float *lse, *part_o, *part_lse;
    int32_t *page_status;
    uint32_t q_bytes, tree_bytes, cache_bytes, mask_bytes;
    int64_t num_pages;
    int page_mode;  // 1: one page per sequence; 2: power-of-two pages >= 16; 0: other
    int page_size, page_shift, max_pages, B, N, Hq, Hkv, G, R, W, n_qt, chunk_blocks,
        n_tree_blocks, total_items;
    float scale, c2, lazy_raw;
    int prefix_len[kMaxBatch];
    int chunk_start[kMaxBatch + 1];
};

constexpr int kPageLds = 1024;     // page ids of one split staged in LDS

__device__ __forceinline__ int find_seq(const AttnArgs &a, int cg) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a.chunk_start[mid] <= cg) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) { return make_rsrc(p, bytes); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte offset of (key row, 16-byte chunk) of block kb in its buffer, or kOob.
// Prefix rows go through the split's page ids in LDS; tree rows index the
// nodes' own K/V.  An out-of-range page id reads as zeros and is flagged.
__device__ __forceinline__ uint32_t row_offset(const AttnArgs &a, const int *pages, int page0, int b,
                                               int g, int P, int nPB, int kb, int row, int chunk,
                                               bool &bad) {
    if (kb < nPB) {
        const int pos = kb * kKB + row;
        if (pos >= P) return kOob;
        int pg, slot;
        if (a.page_shift >= 0) {
            pg = pos >> a.page_shift;
            slot = pos & (a.page_size - 1);
        } else {
            pg = pos / a.page_size;
            slot = pos - pg * a.page_size;
        }
        const int page = pages[pg - page0];
        if (page < 0 || page >= a.num_pages) {
            bad = true;
            return kOob;
        }
        return ((((uint32_t)page * a.page_size + slot) * a.Hkv + g) * kD + chunk * 8) * 2u;
    }
    const int j = (kb - nPB) * kKB + row;
    if (j >= a.N) return kOob;
    return ((((uint32_t)b * a.N + j) * a.Hkv + g) * kD + chunk * 8) * 2u;
}

// LDS byte offset of key row r of a tile: block r % 16, slot r / 16
__device__ __forceinline__ int k_lds(int r) { return (r & 15) * kKBlk + (r >> 4) * kRow; }
__device__ __forceinline__ int v_lds(int r) { return (r & 15) * kVBlk + (r >> 4) * kRow; }

__device__ __forceinline__ bf16x8 cvt8(const f32x16 &s, int base) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(s[base + 2 * j], s[base + 2 * j + 1]);
    return as_bf16x8(w);
}

struct SplitCtx {
    __amdgpu_buffer_rsrc_t r_kt, r_vt, r_kc, r_vc, r_m;
    int b, g, P, nPB, kb1, page0, lane, wave;
    uint32_t moff;
};

// Start the copy of block kb's K and V tiles into stage `dst` (asynchronous;
// each wave fills 4 of the 16 LDS blocks of each tile, one copy each: LDS
// block n holds rows n + 16*slot, lane L copying row n + 16*(L/16), 16-byte
// chunk L%16).  K and V rows share their byte offsets.  Also loads this lane's
// 64-bit mask word of the block (zero for prefix blocks).
__device__ __forceinline__ uint64_t issue_block(const AttnArgs &a, const SplitCtx &c, const int *pages,
                                                uint32_t dst, int kb, bool &bad) {
    const bool tree = kb >= c.nPB;
    const __amdgpu_buffer_rsrc_t rk = tree ? c.r_kt : c.r_kc;
    const __amdgpu_buffer_rsrc_t rv = tree ? c.r_vt : c.r_vc;
    const int sub = c.lane >> 4, ch = c.lane & 15;
    const uint32_t rowb = (uint32_t)a.Hkv * kD * 2;       // bytes between consecutive keys
    const uint32_t dstk = __builtin_amdgcn_readfirstlane(dst + 4 * c.wave * kKBlk);
    const uint32_t dstv = __builtin_amdgcn_readfirstlane(dst + kKTile + 4 * c.wave * kVBlk);
    uint32_t off[4];
    if (tree || a.page_mode != 0) {
        // rows 16*sub + n (n < 16) are contiguous keys of one page (or of the tree)
        uint32_t vbase = kOob;
        int lim;
        if (tree) {
            const int j0 = (kb - c.nPB) * kKB;
            lim = a.N - j0;
            vbase = ((((uint32_t)c.b * a.N + j0 + 16 * sub) * a.Hkv + c.g) * kD + ch * 8) * 2u;
        } else {
            const int pos = kb * kKB + 16 * sub;
            lim = c.P - kb * kKB;
            if (16 * sub < lim) {
                int pg, slot;
                if (a.page_mode == 1) {                    // one page per sequence
                    pg = c.page0;
                    slot = pos;
                } else {                                   // power-of-two pages of >= 16
                    pg = pos >> a.page_shift;
                    slot = pos & (a.page_size - 1);
                }
                const int page = pages[pg - c.page0];
                if (page >= 0 && page < a.num_pages)
                    vbase = ((((uint32_t)page * a.page_size + slot) * a.Hkv + c.g) * kD + ch * 8) * 2u;
                else
                    bad = true;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * c.wave + i;
            off[i] = (16 * sub + n < lim && vbase != kOob) ? vbase + n * rowb : kOob;
        }
    } else {
        // small or irregular pages: look every row up
#pragma unroll
        for (int i = 0; i < 4; ++i)
            off[i] = row_offset(a, pages, c.page0, c.b, c.g, c.P, c.nPB, kb, 4 * c.wave + i + 16 * sub,
                                ch, bad);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16(rk, dstk + i * kKBlk, off[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16(rv, dstv + i * kVBlk, off[i]);
    const uint32_t moff = (tree && c.moff != kOob) ? c.moff + (kb - c.nPB) * 8 : kOob;
    u32x2 mw = __builtin_amdgcn_raw_buffer_load_b64(c.r_m, moff, 0, 0);
    return ((uint64_t)mw[1] << 32) | mw[0];
}

struct SoftmaxState {
    f32x16 o[kD / 32];
    float m, l;
};

// One 64-key block: S^T = K Q^T, masking, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void compute_block(const AttnArgs &a, const lds_t *__restrict__ st,
                                              const bf16x8 *qf, int kb, int nPB, int P,
                                              uint64_t word, int lane, SoftmaxState &S) {
    const int half = lane >> 5, l32 = lane & 31;
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
    // K operand reads run one k-step ahead of the MFMAs; the scheduling
    // fences keep the compiler from hoisting every read of the block (which
    // would cost ~130 registers and halve occupancy).
    const lds_t *kbase = st + k_lds(l32) + half * 16;   // row l32, chunk half; + 32 rows = 2 slots
    auto kread = [&](int t, bf16x8 &k0, bf16x8 &k1) {
        k0 = *(const __attribute__((address_space(3))) bf16x8 *)(kbase + t * 32);
        k1 = *(const __attribute__((address_space(3))) bf16x8 *)(kbase + 2 * kRow + t * 32);
    };
    bf16x8 ka0, ka1, kb0v, kb1v;
    kread(0, ka0, ka1);
#pragma unroll
    for (int t = 0; t < kD / 16; t += 2) {
        kread(t + 1, kb0v, kb1v);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qf[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qf[t], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (t + 2 < kD / 16) kread(t + 2, ka0, ka1);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb0v, qf[t + 1], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb1v, qf[t + 1], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Register i of a half-wave holds key 4*(2*(i/4) + half) + i%4 (+32 for
    // s1): the half-wave's keys are the nibbles half, half+2, ... of the
    // block's 64-bit visibility word.  Gather them into bits 0-15 (s0) and
    // 16-31 (s1) of one 32-bit word and test bit i.
    const bool is_tree = kb >= nPB;
    const bool tail = !is_tree && (kb + 1) * kKB > P;
    if (is_tree || tail) {
        uint64_t vis;
        if (is_tree) {
            const int left = a.N - (kb - nPB) * kKB;     // tree keys that exist in this block
            vis = word & (left >= 64 ? ~0ull : ((1ull << left) - 1ull));
        } else {
            const int left = P - kb * kKB;
            vis = (1ull << left) - 1ull;                 // 0 < left < 64
        }
        uint64_t x = (vis >> (4 * half)) & 0x0F0F0F0F0F0F0F0Full;
        x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
        x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
        const uint32_t m = (uint32_t)(x | (x >> 16));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = ((m >> i) & 1u) ? s0[i] : -INFINITY;
            s1[i] = ((m >> (16 + i)) & 1u) ? s1[i] : -INFINITY;
        }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(fmaxf(mx, s0[i]), s1[i]);   // v_max3_f32
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > S.m + a.lazy_raw;
    if (__ballot(need)) {
        const float m_new = need ? mx : S.m;
        const float alpha = need ? __builtin_amdgcn_exp2f((S.m - m_new) * a.c2) : 1.f;
        S.l *= alpha;
#pragma unroll
        for (int d = 0; d < kD / 32; ++d)
#pragma unroll
            for (int i = 0; i < 16; ++i) S.o[d][i] *= alpha;
        S.m = m_new;
    }
    const float base = S.m == -INFINITY ? 0.f : S.m * a.c2;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], a.c2, -base));
        s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], a.c2, -base));
        ls += s0[i] + s1[i];
    }
    S.l += ls;
    bf16x8 p[4];
    p[0] = cvt8(s0, 0);
    p[1] = cvt8(s0, 8);
    p[2] = cvt8(s1, 0);
    p[3] = cvt8(s1, 8);

    // O^T (d x rows) += V^T P^T.  Within each 16-lane group, ds_read_b64_tr_b16
    // gives lane i element (i%4) of the 8-byte rows supplied by lanes i/4 + 4e
    // (e = 0..3): if lane q + 4e points at V[key0 + e][d0 + 4q], lane i receives
    // V[key0 .. key0+3][d0 + i].  Two such reads (keys key0 and key0 + 8) form
    // the operand slots 0-3 and 4-7 that match the score registers in p[].
    const int grp = l32 >> 4, gi = lane & 15, q4 = gi & 3, e4 = gi >> 2;
    // lane (group grp, q4, e4) points at row key0 + e4, columns grp*16 + 4*q4 ...;
    // key0 = sb*32 + 16*t + 4*half (+8 for the second read): row % 16 =
    // 4*half + e4 (+8), row / 16 = 2*sb + t.
    const lds_t *vbase = st + kKTile + (4 * half + e4) * kVBlk + (grp * 16 + 4 * q4) * 2;
    auto vread = [&](int idx) -> bf16x8 {
        const int d = idx >> 2, stp = idx & 3;           // stp = 2*sb + t
        const lds_t *pa = vbase + stp * kRow + d * 64;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pa);
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(pa + 8 * kVBlk));
        u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
        u32x4 w = {lw[0], lw[1], hw[0], hw[1]};
        return as_bf16x8(w);
    };
    bf16x8 va = vread(0), vb;
#pragma unroll
    for (int idx = 0; idx < (kD / 32) * 4; idx += 2) {
        vb = vread(idx + 1);
        S.o[idx >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[idx & 3], S.o[idx >> 2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (idx + 2 < (kD / 32) * 4) va = vread(idx + 2);
        S.o[(idx + 1) >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, p[(idx + 1) & 3], S.o[(idx + 1) >> 2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ void run_block(const AttnArgs &a, const SplitCtx &c, const int *pages,
                                          const lds_t *cur, uint32_t nxt, const bf16x8 *qf,
                                          uint32_t used, int &kb, uint64_t &word, SoftmaxState &S,
                                          bool &bad) {
    stage_barrier();
    int kbn = kb + 1;
    while (kbn < c.kb1 && kbn >= c.nPB && !((used >> (kbn - c.nPB)) & 1u)) ++kbn;
    uint64_t word_n = 0ull;
    if (kbn < c.kb1) word_n = issue_block(a, c, pages, nxt, kbn, bad);
    compute_block(a, cur, qf, kb, c.nPB, c.P, word, c.lane, S);
    kb = kbn;
    word = word_n;
}

__global__ __launch_bounds__(kNW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_tree_attn_split(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char stage0[kStage];
    __shared__ __attribute__((aligned(1024))) char stage1[kStage];
    __shared__ int s_pages[kPageLds];
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
    const int cidx = cg - a.chunk_start[b];
    const int nchunks = a.chunk_start[b + 1] - a.chunk_start[b];
    const int P = a.prefix_len[b];
    const int nPB = (P + kKB - 1) / kKB;
    const int nB = nPB + a.n_tree_blocks;
    const int kb0 = cidx * a.chunk_blocks;
    const int kb1 = min(kb0 + a.chunk_blocks, nB);

    SplitCtx c;
    c.r_kt = rsrc(a.k_tree, a.tree_bytes);
    c.r_vt = rsrc(a.v_tree, a.tree_bytes);
    c.r_kc = rsrc(a.k_cache, a.cache_bytes);
    c.r_vc = rsrc(a.v_cache, a.cache_bytes);
    c.r_m = rsrc(a.mask, a.mask_bytes);
    c.b = b; c.g = g; c.P = P; c.nPB = nPB; c.kb1 = kb1; c.lane = lane; c.wave = wave;

    // ---- page ids of this split's prefix range ----
    c.page0 = 0;
    {
        const int pos0 = kb0 * kKB;
        const int pos1 = min(kb1 * kKB, P);
        if (pos1 > pos0) {
            int pend;
            if (a.page_shift >= 0) {
                c.page0 = pos0 >> a.page_shift;
                pend = ((pos1 - 1) >> a.page_shift) + 1;
            } else {
                c.page0 = pos0 / a.page_size;
                pend = (pos1 - 1) / a.page_size + 1;
            }
            const int32_t *bt = a.block_table + (int64_t)b * a.max_pages;
            for (int i = tid; i < pend - c.page0; i += kNW * kWave) s_pages[i] = bt[c.page0 + i];
        }
    }

    // ---- this lane's query row ----
    const int r = qt * kTQ + wave * 32 + l32;
    const bool row_ok = r < a.R;
    const int node = row_ok ? r / a.G : 0;
    const int hq = g * a.G + (row_ok ? r % a.G : 0);
    bf16x8 qf[kD / 16];
    {
        const __amdgpu_buffer_rsrc_t r_q = rsrc(a.q, a.q_bytes);
        const uint32_t qoff = row_ok ? (uint32_t)(((((int64_t)b * a.N + node) * a.Hq + hq) * kD + half * 8) * 2) : kOob;
#pragma unroll
        for (int t = 0; t < kD / 16; ++t)
            qf[t] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(r_q, row_ok ? qoff + t * 32 : kOob, 0, 0));
    }
    c.moff = row_ok ? (uint32_t)(((int64_t)b * a.N + node) * a.W * 8) : kOob;

    // ---- which tree blocks of this split does any row of the tile see? ----
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

    SoftmaxState S;
#pragma unroll
    for (int d = 0; d < kD / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) S.o[d][i] = 0.f;
    S.m = -INFINITY;
    S.l = 0.f;
    bool bad = false;

    lds_t *st0 = (lds_t *)stage0;
    lds_t *st1 = (lds_t *)stage1;
    uint32_t a0 = (uint32_t)(uintptr_t)st0, a1 = (uint32_t)(uintptr_t)st1;
    int kb = kb0;
    while (kb < kb1 && kb >= nPB && !((used >> (kb - nPB)) & 1u)) ++kb;
    uint64_t word = 0ull;
    if (kb < kb1) word = issue_block(a, c, s_pages, a0, kb, bad);
    while (kb < kb1) {
        run_block(a, c, s_pages, st0, a1, qf, used, kb, word, S, bad);
        lds_t *t = st0;
        st0 = st1;
        st1 = t;
        const uint32_t ta = a0;
        a0 = a1;
        a1 = ta;
    }

    if (bad) s_bad = 1;  // benign race: every writer stores 1
    float l_run = S.l + __shfl_xor(S.l, 32);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse_v = l_run > 0.f ? S.m * a.scale + logf(l_run) : -INFINITY;
    if (row_ok) {
        if (nchunks == 1) {
            const int64_t orow = ((int64_t)b * a.N + node) * a.Hq + hq;
            uint16_t *op = (uint16_t *)a.out + orow * kD + half * 4;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2 w;
                    w[0] = pack_bf16x2(S.o[d][gq * 4 + 0] * inv, S.o[d][gq * 4 + 1] * inv);
                    w[1] = pack_bf16x2(S.o[d][gq * 4 + 2] * inv, S.o[d][gq * 4 + 3] * inv);
                    *(u32x2 *)(op + d * 32 + gq * 8) = w;
                }
            if (a.lse && half == 0) a.lse[orow] = lse_v;
        } else {
            const int64_t prow = ((int64_t)cg * a.Hkv + g) * a.R + r;
            float *op = a.part_o + prow * kD + half * 4;
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    f32x4 w = {S.o[d][gq * 4 + 0] * inv, S.o[d][gq * 4 + 1] * inv,
                               S.o[d][gq * 4 + 2] * inv, S.o[d][gq * 4 + 3] * inv};
                    *(f32x4 *)(op + d * 32 + gq * 8) = w;
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
void plan_tree_attn(AttnPlan &p, int B, int N, int Hq, int Hkv, int D, int page_size,
                    const int32_t *prefix_len, jf_dtype dtype) {
    p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.D = D;
    p.page_size = page_size;
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
    // a split's page ids must fit the LDS staging array
    int64_t Pmax = 0;
    for (int b = 0; b < B; ++b) Pmax = prefix_len[b] > Pmax ? prefix_len[b] : Pmax;
    if (page_size < Pmax) {
        int64_t cap = ((int64_t)(kPageLds - 2) * page_size) / kKB;
        if (cap < 1) cap = 1;
        if (cb > cap) cb = cap;
    }
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
    a.q_bytes = (uint32_t)((int64_t)p.B * p.N * p.Hq * kD * 2);
    a.tree_bytes = (uint32_t)((int64_t)p.B * p.N * p.Hkv * kD * 2);
    a.cache_bytes = (uint32_t)(num_pages * page_size * (int64_t)p.Hkv * kD * 2);
    a.mask_bytes = (uint32_t)((int64_t)p.B * p.N * p.W * 8);
    a.num_pages = num_pages;
    a.page_size = page_size;
    a.page_shift = -1;
    if ((page_size & (page_size - 1)) == 0) {
        int sh = 0;
        while ((1 << sh) < page_size) ++sh;
        a.page_shift = sh;
    }
    a.max_pages = max_pages;
    {
        int Pmax = 0;
        for (int b = 0; b < p.B; ++b) Pmax = p.prefix_len[b] > Pmax ? p.prefix_len[b] : Pmax;
        a.page_mode = (max_pages == 1 && page_size >= Pmax) ? 1
                      : (a.page_shift >= 4 ? 2 : 0);
    }
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
