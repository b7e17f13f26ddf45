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
//     own K/V).  A row (sequence, KV head, tile of 256 query rows) with all
//     of its blocks is cut into pieces of nearly equal size; one workgroup of
//     eight waves (two per SIMD) handles one piece.  Query row
//     r = node * G + (h % G), so the G heads of a node share a mask row.
//   * Per block, each wave computes S^T = K Q^T for its 32 rows with
//     v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand, Q^T held in
//     registers as B), so each lane ends up owning one query row's scores.
//     The softmax statistics of that row then live in the lane (and its
//     partner lane+32), and O^T = V^T P^T (V^T from LDS as A, P^T straight
//     from the score registers as B) leaves the output row in the same lane:
//     no shuffles besides one max exchange between the two half-waves.
//   * Software pipeline inside each wave: the exponentials of block j are
//     interleaved with the score MFMAs of block j+1, and the row maximum of
//     block j+1 with the output MFMAs of block j, so the VALU and the MFMA
//     pipes work at the same time.
//   * Tree blocks apply the ancestor bitmask: each row's 64-bit word of the
//     block travels with the block's K/V tiles; a tree block no row of the
//     workgroup can see is skipped.
//   * Online softmax in base 2 with a lazy rescale: the running maximum is
//     only moved when a block's maximum exceeds it by more than 2^8, which
//     keeps every exponent bounded while leaving the arithmetic exact.  Row
//     sums use v_dot2 on the same bf16 probabilities the MFMA consumes.
//   * K and V tiles go straight from HBM into LDS (buffer_load ... lds, 16
//     bytes a lane) through a 4-stage ring, three blocks ahead; no registers
//     are spent on the prefetch.  For contiguous prefixes and tree blocks the
//     block position lives in the buffer descriptor (scalar work only), whose
//     record count also zero-fills rows past the end.  One copy instruction
//     fills 1 KiB of LDS; block n of a tile holds rows n, n+16, n+32, n+48,
//     and the blocks are padded (16 bytes for K, 64 for V) so that both the K
//     operand reads (ds_read_b128) and the V operand reads hit distinct
//     banks, while every operand address is one base register plus an
//     immediate.  V stays row-major: ds_read_b64_tr_b16 hands each lane four
//     consecutive keys of one head-dim column, which is exactly the V^T
//     operand layout.
//   * Each piece of a row cut in several writes (O / l, log-sum-exp)
//     partials in fp32, 256 rows per work item; a merge kernel combines the
//     pieces of a row with LSE weights.  A row in one piece writes the final
//     output directly.
//   * Serving batches: trees may be packed with a different node count per
//     sequence (rows node_off[b] .. node_off[b+1]-1), and prefix lengths may
//     come from device memory.  The host plans the pieces and the grid from
//     per-sequence prefix bounds; each workgroup reads the real length, and
//     pieces past it exit (the merge reads the same length), so one captured
//     launch serves any lengths up to the bounds.
#include "jf_internal.h"

#include <algorithm>
#include <queue>
#include <type_traits>
#include <vector>

namespace jf {
namespace {

constexpr int kKB = 64;                  // keys per block
constexpr int kNW = 8;                   // waves per workgroup (two per SIMD)
constexpr int kTQ = 32 * kNW;            // query rows per workgroup
constexpr int kD = 128;                  // head dim of the bf16 path
constexpr int kRow = kD * 2;             // bytes per K or V row
constexpr int kKBlk = 4 * kRow + 16;     // LDS block of 4 K rows (n, n+16, n+32, n+48)
constexpr int kVBlk = 4 * kRow + 64;     // LDS block of 4 V rows
constexpr int kKTile = 16 * kKBlk;
constexpr int kVTile = 16 * kVBlk;
constexpr int kMTile = kTQ * 8;          // one 64-bit visibility word per query row
constexpr int kStage = kKTile + kVTile + kMTile;
constexpr int kNS = 4;                   // stages of the copy ring (three blocks in flight)
constexpr int kCpw = 16 / kNW;           // K (and V) LDS blocks each wave fills per key block
constexpr int kOps = 2 * kCpw + 1;       // memory operations per wave per key block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.f;

struct AttnArgs {
    const uint16_t *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const uint64_t *mask;
    const int32_t *block_table;
    const int32_t *prefix_dev;   // device prefix lengths, or null (the bounds are the lengths)
    void *out;
    float *lse;
    float *part_o;         // piece partials O / l, fp32 [items * kTQ, kD]
    float *part_lse;       // [items * kTQ]
    int32_t *status;
    uint32_t q_bytes, tree_bytes, cache_bytes, mask_bytes;
    int64_t num_pages;
    int page_mode;  // 1: one page per sequence; 2: power-of-two pages >= 16; 0: other
    int page_size, page_shift, max_pages, B, Hq, Hkv, G, W, total_items;
    int L;                           // longest piece (64-key blocks) of a row
    int D;                           // head dim in memory: 128, or 64 (computed as 128, upper half zero)
    float scale, c2, lazy_raw;
    float k_scale, v_scale, c2k;     // FP8 caches: value = code * scale; c2k = c2 * k_scale
    int cap[kMaxBatch];              // planned prefix bound of each sequence
    int node_off[kMaxBatch + 1];     // tree rows of sequence b: node_off[b] .. node_off[b+1]-1
    int item_start[kMaxBatch + 1];   // first work item of the sequence at dispatch position p
    uint8_t seq_order[kMaxBatch];    // sequence at dispatch position p
};

constexpr int kPageLds = 2048;     // page ids of one piece staged in LDS

__device__ __forceinline__ int div_up(int x, int y) { return (x + y - 1) / y; }

// A row of sequence b has nbc = ceil(cap / 64) + ceil(n / 64) key blocks at
// its planned (bound) length, cut into np = ceil(nbc / L) pieces: np - 1 of
// ceil(nbc / np) blocks and a last, shorter one (which holds the tree blocks,
// whose masking makes them the dearer ones).  Piece k starts at
// min(k ceil(nbc / np), nbc); the last piece is never empty.
__device__ __forceinline__ int piece_start(int k, int nbc, int np) {
    return min(k * div_up(nbc, np), nbc);
}

// Workgroups are dealt round-robin over the XCDs by hardware id.  Deal
// blocks of kXcdRun consecutive work items instead: the items of one block
// (query tiles and KV heads of one piece, which share keys) meet in one XCD's
// L2, and each XCD still takes its items in dispatch (longest-first) order.
// Ids past the last whole round of blocks map to themselves.
constexpr int kXcdRun = 8;
__host__ __device__ __forceinline__ int xcd_interleave(int bid, int n) {
    constexpr int kRound = kNumXcd * kXcdRun;
    if (bid >= n / kRound * kRound) return bid;
    const int xcd = bid % kNumXcd, local = bid / kNumXcd;
    return ((local / kXcdRun) * kNumXcd + xcd) * kXcdRun + local % kXcdRun;
}

// the dispatch position of work item `item`: the last p with item_start[p] <= item
__device__ __forceinline__ int find_pos(const AttnArgs &a, int item) {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a.item_start[mid] <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Prefix length of sequence b: the device value when given, clamped to the
// planned bound [0, cap] (bad = true when it had to be clamped).
__device__ __forceinline__ int prefix_of(const AttnArgs &a, int b, bool &bad) {
    const int cap = a.cap[b];
    if (!a.prefix_dev) return cap;
    const int p = a.prefix_dev[b];
    if (p < 0 || p > cap) {
        bad = true;
        return p < 0 ? 0 : cap;
    }
    return p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) { return make_rsrc(p, bytes); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte offset of (key row, 16-byte chunk) of block kb in its buffer, or kOob.
// Prefix rows go through the piece's page ids in LDS; tree rows index the
// nodes' own K/V.  An out-of-range page id reads as zeros and is flagged.
template <int kDm>
__device__ __forceinline__ uint32_t row_offset(const AttnArgs &a, const int *pages, int page0,
                                               int64_t node0, int n, int g, int P, int nPB, int kb,
                                               int row, int chunk, bool &bad) {
    if (chunk * 8 >= kDm) return kOob;                // past the head dim: reads as zeros
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
        return ((((uint32_t)page * a.page_size + slot) * a.Hkv + g) * kDm + chunk * 8) * 2u;
    }
    const int j = (kb - nPB) * kKB + row;
    if (j >= n) return kOob;
    return ((((uint32_t)node0 + j) * a.Hkv + g) * kDm + chunk * 8) * 2u;
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
    __amdgpu_buffer_rsrc_t r_kc, r_vc, r_m;  // whole prefix cache (paged layouts), mask buffer
    const uint16_t *kc0, *vc0;               // one-page layout: KV head g of prefix row 0
    const uint16_t *kt0, *vt0;               // KV head g of tree row 0 of the sequence
    int64_t node0;                           // first tree row of the sequence
    int b, g, P, nPB, n, page0, lane, wave;  // n: the sequence's tree nodes
    const uint8_t *kc8, *vc8;                // FP8 one-page layout: KV head g of prefix row 0
    uint32_t rowb8;                          // FP8 bytes between consecutive prefix keys
    bool pzero;                              // one-page layout with a bad page id: zeros
    uint32_t rowb;                           // bytes between consecutive keys
    uint32_t vrow;                           // lane's offset of its first copy in a block
    uint32_t mrow;                           // lane's mask dword offset (kOob: none)
    bool chunk_ok;                           // the lane's 16-byte chunk lies inside the head dim
};

// A pointer known to be the same in every lane, moved to scalar registers.
__device__ __forceinline__ const uint16_t *uniform_ptr(const uint16_t *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint16_t *)(((uint64_t)hi << 32) | lo);
}

// This lane's eight 16-byte query fragments (k-steps t = 0..7 at +32 t bytes).
// Plain buffer-load builtins: the compiler then knows the registers are
// written when the loads return and waits before any read of them (a spill
// or a copy included); the kernel also waits for them explicitly before the
// first block copy.
// Fragments t >= tq lie past the head dim and read as zeros.
__device__ __forceinline__ void load_q(u32x4 (&d)[kD / 16], __amdgpu_buffer_rsrc_t r, uint32_t voff, int tq) {
#pragma unroll
    for (int t = 0; t < kD / 16; ++t)
        d[t] = __builtin_amdgcn_raw_buffer_load_b128(r, t < tq ? voff + 32u * t : kOob, 0, 0);
}

// 4 bytes per lane HBM -> LDS: lane L's dword lands at lds + 4 L.
__device__ __forceinline__ void copy4s(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff,
                                       uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}

// Start the copy of block kb into stage `dst` (asynchronous, kOps memory
// operations per wave): K and V tiles -- wave w fills LDS blocks 2w and 2w+1
// of each, lane L copying row n + 16*(L/16), 16-byte chunk L%16 -- and the
// visibility words of the workgroup's 256 query rows (zeros for prefix
// blocks), thread t copying dword t%2 of row t/2.
template <bool kPaged, int kDm>
__device__ __forceinline__ void issue_block(const AttnArgs &a, const SplitCtx &c, const int *pages,
                                            uint32_t dst, int kb, bool &bad) {
    const bool tree = kb >= c.nPB;
    const uint32_t dk = __builtin_amdgcn_readfirstlane(dst + kCpw * c.wave * kKBlk);
    const uint32_t dv = __builtin_amdgcn_readfirstlane(dst + kKTile + kCpw * c.wave * kVBlk);
    const uint32_t dm = __builtin_amdgcn_readfirstlane(dst + kKTile + kVTile + c.wave * 256);
    if (!kPaged || tree) {
        // the block's rows are contiguous keys: position in the descriptor,
        // rows past the end of the prefix (or tree) read as zeros
        const uint16_t *kp, *vp;
        int rows;
        if (tree) {
            const int j0 = (kb - c.nPB) * kKB;
            kp = c.kt0 + (int64_t)j0 * a.Hkv * kDm;
            vp = c.vt0 + (int64_t)j0 * a.Hkv * kDm;
            rows = min(kKB, c.n - j0);
        } else {
            const int p0 = kb * kKB;
            kp = c.kc0 + (int64_t)p0 * a.Hkv * kDm;
            vp = c.vc0 + (int64_t)p0 * a.Hkv * kDm;
            rows = c.pzero ? 0 : min(kKB, c.P - p0);
        }
        // every value here is wave-uniform; say so, so that the descriptors live in SGPRs
        const uint32_t nbytes = __builtin_amdgcn_readfirstlane((uint32_t)rows * c.rowb);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(uniform_ptr(kp), nbytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(uniform_ptr(vp), nbytes);
#pragma unroll
        for (int i = 0; i < kCpw; ++i) copy16(rk, dk + i * kKBlk, c.chunk_ok ? c.vrow + i * c.rowb : kOob);
#pragma unroll
        for (int i = 0; i < kCpw; ++i) copy16(rv, dv + i * kVBlk, c.chunk_ok ? c.vrow + i * c.rowb : kOob);
    } else {
        // paged layouts: every group of 16 rows sits in one page (page_mode 2)
        // or every row is looked up (page_mode 0)
        const int sub = c.lane >> 4, ch = c.lane & 15;
        uint32_t off[kCpw];
        if (a.page_mode == 2) {
            const int pos = kb * kKB + 16 * sub;
            const int lim = c.P - kb * kKB;
            uint32_t vbase = kOob;
            if (16 * sub < lim && c.chunk_ok) {
                const int page = pages[(pos >> a.page_shift) - c.page0];
                if (page >= 0 && page < a.num_pages)
                    vbase = ((((uint32_t)page * a.page_size + (pos & (a.page_size - 1))) * a.Hkv + c.g) * kDm +
                             ch * 8) * 2u;
                else
                    bad = true;
            }
#pragma unroll
            for (int i = 0; i < kCpw; ++i) {
                const int n = kCpw * c.wave + i;
                off[i] = (16 * sub + n < lim && vbase != kOob) ? vbase + n * c.rowb : kOob;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kCpw; ++i)
                off[i] = row_offset<kDm>(a, pages, c.page0, c.node0, c.n, c.g, c.P, c.nPB, kb,
                                    kCpw * c.wave + i + 16 * sub, ch, bad);
        }
#pragma unroll
        for (int i = 0; i < kCpw; ++i) copy16(c.r_kc, dk + i * kKBlk, off[i]);
#pragma unroll
        for (int i = 0; i < kCpw; ++i) copy16(c.r_vc, dv + i * kVBlk, off[i]);
    }
    copy4s(c.r_m, dm, tree ? c.mrow : kOob, tree ? (uint32_t)(kb - c.nPB) * 8u : 0u);
}

template <bool B>
struct Flag { static constexpr bool value = B; };

struct SoftmaxState {
    f32x16 o[kD / 32];
    float m, l;
};

// Wait until at most n memory operations of this wave are outstanding, then
// barrier (n is a multiple of kOps up to (kNS - 2) * kOps).
__device__ __forceinline__ void ring_wait(int n) {
    if (n >= 2 * kOps) ring_barrier<2 * kOps>();
    else if (n >= kOps) ring_barrier<kOps>();
    else ring_barrier<0>();
}

// A row's statistics live in lanes l and l + 32: combine them with one
// v_permlane32_swap (lanes l and l ^ 32 exchange in registers; no LDS trip).
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Register i of a half-wave's score tile holds key 4*(2*(i/4) + half) + i%4
// (+32 for the second tile).
__device__ __forceinline__ uint32_t half_bits(uint64_t vis, int half) {
    uint64_t x = (vis >> (4 * half)) & 0x0F0F0F0F0F0F0F0Full;
    x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
    x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
    return (uint32_t)(x | (x >> 16));
}

// Barrier that publishes LDS writes only: unlike __syncthreads it does not
// wait for outstanding global loads (the query fragments are in flight while
// the set-up runs).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// kPaged = false: every prefix is one page (page_mode 1); true: page_mode 0 or 2.
// kDm: the head dim of q, k and v in memory, 128 or 64; at 64 the kernel
// computes at 128 with the upper half of every row read as zeros (the scores
// are unchanged) and writes only the first 64 output columns.
// kFp8: the prefix cache holds E4M3 codes; each prefix block is loaded into
// registers one block ahead, converted exactly to bf16 and written into the
// same LDS layout the bf16 copies produce (tree blocks are bf16 and copied
// as usual).  Scores of prefix keys are scaled by k_scale through the
// exponent coefficient and the block maximum; the output accumulator holds
// prefix values in code units until the piece's first tree block (or the
// end), where it is multiplied by v_scale once.
template <bool kPaged, bool kFp8, int kDm>
__global__ __launch_bounds__(kNW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_tree_attn_split(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char ring[kNS][kStage];
    __shared__ int s_pages[kPageLds];
    __shared__ uint32_t s_used;
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets wave math stay scalar
    const int half = lane >> 5, l32 = lane & 31;

    // ---- work item: (piece, KV head, query tile) of one sequence ----
    const int item = xcd_interleave(blockIdx.x, a.total_items);
    const int pos = __builtin_amdgcn_readfirstlane(find_pos(a, item));
    const int b = __builtin_amdgcn_readfirstlane((int)a.seq_order[pos]);
    const int64_t node0 = a.node_off[b];
    const int n = __builtin_amdgcn_readfirstlane(a.node_off[b + 1] - a.node_off[b]);
    const int R = n * a.G;                                   // query rows of the sequence
    const int n_qt = div_up(R, kTQ);
    const int local = item - a.item_start[pos];
    const int qt = __builtin_amdgcn_readfirstlane(local % n_qt);
    const int g = __builtin_amdgcn_readfirstlane((local / n_qt) % a.Hkv);
    const int cidx = __builtin_amdgcn_readfirstlane(local / n_qt / a.Hkv);
    bool pbad = false;
    int P = __builtin_amdgcn_readfirstlane(prefix_of(a, b, pbad));
    const int nPB = (P + kKB - 1) / kKB;
    const int nTB = div_up(n, kKB);
    const int nB = nPB + nTB;                                // blocks of the real length
    const int nbc = div_up(a.cap[b], kKB) + nTB;             // blocks of the planned length
    const int np = div_up(nbc, a.L);                         // pieces of each row
    const int kb0 = __builtin_amdgcn_readfirstlane(piece_start(cidx, nbc, np));
    const int kb1c = __builtin_amdgcn_readfirstlane(piece_start(cidx + 1, nbc, np));
    if (kb0 >= nB) {
        // past the sequence's real length: nothing to do (the merge reads
        // the same length and skips this piece)
        if (pbad && tid == 0 && a.status) *a.status = JF_ERR_BAD_PREFIX;
        return;
    }
    const int kb1 = min(kb1c, nB);
    const bool single = cidx == 0 && kb1c >= nB;             // the only piece with keys
    const int64_t prow0 = (int64_t)item * kTQ;               // this item's partial rows

    SplitCtx c;
    c.r_kc = make_rsrc(a.k_cache, a.cache_bytes);
    c.r_vc = make_rsrc(a.v_cache, a.cache_bytes);
    c.r_m = make_rsrc(a.mask, a.mask_bytes);
    c.b = b; c.g = g; c.P = P; c.nPB = nPB; c.n = n; c.node0 = node0; c.lane = lane; c.wave = wave;
    c.rowb = (uint32_t)a.Hkv * kDm * 2;
    c.vrow = (uint32_t)(kCpw * wave + 16 * (lane >> 4)) * c.rowb + (uint32_t)(lane & 15) * 16u;
    c.chunk_ok = (lane & 15) * 8 < kDm;
    c.kt0 = uniform_ptr(a.k_tree + (node0 * a.Hkv + g) * kDm);
    c.vt0 = uniform_ptr(a.v_tree + (node0 * a.Hkv + g) * kDm);
    c.kc0 = a.k_cache;
    c.vc0 = a.v_cache;
    c.kc8 = (const uint8_t *)a.k_cache;
    c.vc8 = (const uint8_t *)a.v_cache;
    c.rowb8 = (uint32_t)a.Hkv * kDm;
    c.pzero = false;
    // ---- this lane's query row and mask dword ----
    const int r = qt * kTQ + wave * 32 + l32;
    const bool row_ok = r < R;
    const int node = row_ok ? r / a.G : 0;
    const int hq = g * a.G + (row_ok ? r % a.G : 0);
    {
        const int rm = qt * kTQ + (tid >> 1);
        c.mrow = rm < R ? (uint32_t)(((node0 + rm / a.G) * a.W) * 8 + (tid & 1) * 4) : kOob;
    }

    if (tid == 0) { s_used = 0u; s_bad = 0; }
    lds_barrier();

    // ---- page ids of this piece's prefix range ----
    c.page0 = 0;
    {
        const int pos0 = kb0 * kKB;
        const int pos1 = min(kb1 * kKB, P);
        if (pos1 > pos0) {
            const int32_t *bt = a.block_table + (int64_t)b * a.max_pages;
            if (!kPaged) {
                // one page per sequence: a bad id reads as zeros and is flagged
                const int page = __builtin_amdgcn_readfirstlane(bt[0]);
                if (page >= 0 && page < a.num_pages) {
                    const int64_t e0 = ((int64_t)page * a.page_size * a.Hkv + g) * kDm;
                    if constexpr (kFp8) {
                        c.kc8 = (const uint8_t *)a.k_cache + e0;
                        c.vc8 = (const uint8_t *)a.v_cache + e0;
                    } else {
                        c.kc0 = uniform_ptr(a.k_cache + e0);
                        c.vc0 = uniform_ptr(a.v_cache + e0);
                    }
                } else {
                    c.pzero = true;     // the prefix reads as zero keys and values
                    if (tid == 0) s_bad = 1;
                }
            } else {
                int pend;
                if (a.page_shift >= 0) {
                    c.page0 = pos0 >> a.page_shift;
                    pend = ((pos1 - 1) >> a.page_shift) + 1;
                } else {
                    c.page0 = pos0 / a.page_size;
                    pend = (pos1 - 1) / a.page_size + 1;
                }
                for (int i = tid; i < pend - c.page0; i += kNW * kWave) s_pages[i] = bt[c.page0 + i];
            }
        }
    }

    // ---- queries (Q^T fragments in registers), issued before the mask scan
    // so that their latency overlaps that work, and waited for before the
    // first block copy (the compiler cannot count the copies, so a wait it
    // placed itself would also wait for every copy in flight).  They come
    // after the page-table reads above, whose own waits would otherwise also
    // wait for them.
    u32x4 qraw[kD / 16];
    {
        const __amdgpu_buffer_rsrc_t r_q = make_rsrc(a.q, a.q_bytes);
        const uint32_t qoff = row_ok ? (uint32_t)((((node0 + node) * a.Hq + hq) * kDm + half * 8) * 2) : kOob;
        load_q(qraw, r_q, qoff, kDm / 16);
    }
    // ---- which tree blocks of this piece does any row of the tile see? ----
    lds_barrier();   // s_pages / s_bad written above
    if (kb1 > nPB && tid < kTQ) {
        const int rr = qt * kTQ + tid;
        if (rr < R) {
            const uint64_t *mr = a.mask + (node0 + rr / a.G) * a.W;
            uint32_t bits = 0;
            for (int kb = max(kb0, nPB); kb < kb1; ++kb)
                if (mr[kb - nPB] != 0ull) bits |= 1u << (kb - nPB);
            if (bits) atomicOr(&s_used, bits);
        }
    }
    lds_barrier();
    const uint32_t used = __builtin_amdgcn_readfirstlane(s_used);   // uniform: block choice stays scalar
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));            // vmcnt(0): the queries have landed
    auto next_vis = [&](int kb) {        // first visible block >= kb (kb1 if none)
        while (kb < kb1 && kb >= nPB && !((used >> (kb - nPB)) & 1u)) ++kb;
        return kb;
    };
    if (next_vis(kb0) >= kb1) {
        // no row of the tile sees a key of this piece: zero rows, lse = -inf;
        // the whole workgroup leaves here with nothing in flight
        if (row_ok) {
            if (single) {
                const int64_t orow = (node0 + node) * a.Hq + hq;
                uint16_t *op = (uint16_t *)a.out + orow * kDm + half * 4;
                if (a.lse && half == 0) a.lse[orow] = -INFINITY;
#pragma unroll
                for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq)
                        if (d * 32 + gq * 8 < kDm) *(u32x2 *)(op + d * 32 + gq * 8) = u32x2{0u, 0u};
            } else {
                const int64_t prow = prow0 + wave * 32 + l32;
                float *op = a.part_o + prow * kD + half * 4;
                if (half == 0) a.part_lse[prow] = -INFINITY;
#pragma unroll
                for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) *(f32x4 *)(op + d * 32 + gq * 8) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (tid == 0 && a.status) {
            if (s_bad) *a.status = JF_ERR_BAD_PAGE;
            if (pbad) *a.status = JF_ERR_BAD_PREFIX;
        }
        __builtin_amdgcn_s_waitcnt(0);   // the query loads have returned
        return;
    }

    SoftmaxState S;
#pragma unroll
    for (int d = 0; d < kD / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) S.o[d][i] = 0.f;
    S.m = -INFINITY;
    S.l = 0.f;
    bool bad = false;

    const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_t *)&ring[0][0];
    auto stage_of = [&](int j) { return (const lds_t *)&ring[j % kNS][0]; };

    // visible blocks in order: v(0), v(1), ... ; block v(j) goes to stage j % kNS.
    // Issue order: the query fragments (above), blocks 0 .. kNS-2, so that
    // waiting for block 0 leaves the later blocks in flight.
    int kb_iss = next_vis(kb0);         // next block to issue
    int n_iss = 0;                      // blocks issued so far
    if constexpr (!kFp8) {
        if (kb_iss < kb1) {
            issue_block<kPaged, kDm>(a, c, s_pages, ring0, kb_iss, bad);
            kb_iss = next_vis(kb_iss + 1);
            n_iss = 1;
        }
        for (; n_iss < kNS - 1 && kb_iss < kb1; ++n_iss) {
            issue_block<kPaged, kDm>(a, c, s_pages, ring0 + (n_iss % kNS) * kStage, kb_iss, bad);
            kb_iss = next_vis(kb_iss + 1);
        }
    }
    bf16x8 qf[kD / 16];                 // set from qraw after the first wait

    // ---- per-block pieces ----
    const int koff = k_lds(l32) + half * 16;                             // row l32, chunk half
    auto qk = [&](const lds_t *st, f32x16 &s0, f32x16 &s1) {            // S^T = K Q^T, with no other work
#pragma unroll
        for (int i = 0; i < 16; ++i) { s0[i] = 0.f; s1[i] = 0.f; }
        const lds_t *kb_ = st + koff;
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) {
            const bf16x8 k0 = *(const __attribute__((address_space(3))) bf16x8 *)(kb_ + t * 32);
            const bf16x8 k1 = *(const __attribute__((address_space(3))) bf16x8 *)(kb_ + 2 * kRow + t * 32);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[t], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[t], s1, 0, 0, 0);
        }
    };
    // visibility of a block's scores: tree blocks (ancestor words) and the prefix tail
    auto apply_mask = [&](const lds_t *st, int kb, f32x16 &s0, f32x16 &s1) {
        const bool is_tree = kb >= nPB;
        const bool tail = !is_tree && (kb + 1) * kKB > P;
        if (is_tree || tail) {
            uint64_t vis;
            if (is_tree) {
                const int left = n - (kb - nPB) * kKB;
                const uint64_t word = *(const __attribute__((address_space(3))) uint64_t *)(
                    st + kKTile + kVTile + (wave * 32 + l32) * 8);
                vis = word & (left >= 64 ? ~0ull : ((1ull << left) - 1ull));
            } else {
                vis = (1ull << (P - kb * kKB)) - 1ull;           // 0 < P - kb*64 < 64
            }
            const uint32_t m = half_bits(vis, half);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s0[i] = ((m >> i) & 1u) ? s0[i] : -INFINITY;
                s1[i] = ((m >> (16 + i)) & 1u) ? s1[i] : -INFINITY;
            }
        }
    };
    auto row_max = [&](const f32x16 &s0, const f32x16 &s1) -> float {
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(fmaxf(mx, s0[i]), s1[i]);
        return max_halves(mx);
    };
    // move the running maximum when the block's maximum exceeds it by > 2^8
    auto rescale = [&](float mx) {
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
    };

    // V^T operand reads (see the layout note at the top of the file)
    const int grp = l32 >> 4, gi = lane & 15, q4 = gi & 3, e4 = gi >> 2;
    const int vlane = kKTile + (4 * half + e4) * kVBlk + (grp * 16 + 4 * q4) * 2;
    auto vread = [&](const lds_t *st, int idx) -> bf16x8 {
        const int d = idx >> 2, stp = idx & 3;
        const lds_t *pa = st + vlane + stp * kRow + d * 64;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)pa);
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(pa + 8 * kVBlk));
        u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
        u32x4 w = {lw[0], lw[1], hw[0], hw[1]};
        return as_bf16x8(w);
    };

    // One pipelined step: finish block j (scores sc, maximum already folded
    // into S.m) while computing the scores sn of block j+1 (if has_next).
    //   region A: the 16 score MFMAs of block j+1 | exps of keys 0-31 of block j
    //             (slot t: k-step t of both key halves, so that the two
    //             accumulation chains of a wave interleave)
    //   region B: O += V^T P^T for keys 0-31      | exps of keys 32-63
    //             O += V^T P^T for keys 32-63     | row maximum of block j+1
    // Each slot pairs MFMAs with a matching amount of VALU work (an exp runs
    // at a quarter of the VALU rate).  Empty asm statements at every slot
    // boundary pass the slot's MFMA results and VALU results through, and the
    // scores later slots read, so no optimisation can move work between
    // slots.
    // cj: exponent coefficient of block j's raw scores (c2, or c2 * k_scale
    // for an FP8 prefix block)
    auto step = [&](auto next_tag, const lds_t *stj, const lds_t *stn, int kbn,
                    f32x16 &sc0, f32x16 &sc1, f32x16 &sn0, f32x16 &sn1, float cj) -> float {
        constexpr bool has_next = decltype(next_tag)::value;
        const float nb = S.m == -INFINITY ? 0.f : -S.m * a.c2;
        float ls[2] = {0.f, 0.f};                  // two partial row sums: shorter dependency chains
        u32x4 pw[4];
        // exps of registers i, i+1 of tile sx as one bf16 pair; the row sum
        // uses the same bf16 probabilities as the MFMA
        auto exp_pair = [&](const f32x16 &sx, int i) -> uint32_t {
            const float e0 = __builtin_amdgcn_exp2f(fmaf(sx[i], cj, nb));
            const float e1 = __builtin_amdgcn_exp2f(fmaf(sx[i + 1], cj, nb));
            const uint32_t w = pack_bf16x2(e0, e1);
            float &acc = ls[(i >> 1) & 1];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                                  __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
            return w;
        };
        const lds_t *kb_ = stn + koff;
        // K operand of k-step t for key rows 0-31 (h = 0) or 32-63 (h = 1)
        auto kread = [&](int h, int t) {
            return *(const __attribute__((address_space(3))) bf16x8 *)(kb_ + h * 2 * kRow + t * 32);
        };
        // K operands of slot t: k-step t of both key halves (two independent
        // accumulation chains per slot); read two slots ahead
        bf16x8 kr[3][2];
        auto kload = [&](int t, bf16x8 (&dst)[2]) {
            dst[0] = kread(0, t);
            dst[1] = kread(1, t);
        };
        if constexpr (has_next) {
#pragma unroll
            for (int i = 0; i < 16; ++i) { sn0[i] = 0.f; sn1[i] = 0.f; }
            kload(0, kr[0]);
            kload(1, kr[1]);
        }
        // ---- region A: slot t = k-step t of both key halves of block j+1 + two exps of sc0 ----
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (has_next) {
                if (t + 2 < 8) kload(t + 2, kr[(t + 2) % 3]);
                sn0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[t % 3][0], qf[t], sn0, 0, 0, 0);
                sn1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[t % 3][1], qf[t], sn1, 0, 0, 0);
            }
            uint32_t w = exp_pair(sc0, 2 * t);               // registers 2t, 2t+1 of sc0
            if constexpr (has_next) {
                asm volatile("" : "+v"(sn0), "+v"(sn1), "+v"(w));
            } else {
                asm volatile("" : "+v"(w));
            }
            if (t < 7) asm volatile("" : "+v"(sc0));
            pw[t >> 2][t & 3] = w;                            // P^T operand q holds registers 8q .. 8q+7
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (has_next) apply_mask(stn, kbn, sn0, sn1);
        bf16x8 p[4];
        p[0] = as_bf16x8(pw[0]);
        p[1] = as_bf16x8(pw[1]);
        // ---- region B: slot m = one output MFMA + (two exps of sc1 | row max) ----
        float mxn = -INFINITY, mxn1 = -INFINITY;   // row maximum of block j+1, one chain per key half
        // V^T operand of slot m (d = m%4, k-substep kk = m/4) is idx 4d + kk; read two slots ahead
        bf16x8 vr[3];
        vr[0] = vread(stj, 0);
        vr[1] = vread(stj, 4);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int kk = m >> 2, d = m & 3;
            if (m + 2 < 16) vr[(m + 2) % 3] = vread(stj, 4 * ((m + 2) & 3) + ((m + 2) >> 2));
            if (m == 8) {
                p[2] = as_bf16x8(pw[2]);
                p[3] = as_bf16x8(pw[3]);
            }
            S.o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[m % 3], p[kk], S.o[d], 0, 0, 0);
            if (m < 8) {
                uint32_t w = exp_pair(sc1, 2 * m);           // registers 2m, 2m+1 of sc1
                asm volatile("" : "+v"(S.o[d]), "+v"(w));
                if (m < 7) asm volatile("" : "+v"(sc1));
                pw[2 + (m >> 2)][m & 3] = w;
            } else if constexpr (has_next) {
                const int i = 2 * (m - 8);                   // registers i, i+1 of both tiles
                mxn = fmaxf(fmaxf(mxn, sn0[i]), sn0[i + 1]);
                mxn1 = fmaxf(fmaxf(mxn1, sn1[i]), sn1[i + 1]);
                asm volatile("" : "+v"(S.o[d]), "+v"(mxn), "+v"(mxn1));
            } else {
                asm volatile("" : "+v"(S.o[d]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        S.l += ls[0] + ls[1];
        mxn = fmaxf(mxn, mxn1);
        return has_next ? max_halves(mxn) : -INFINITY;
    };

    // ---- main loop over the visible blocks ----
    int kb_cur = next_vis(kb0);
    f32x16 sa0, sa1, sb0, sb1;
    float mx_cur = -INFINITY;
    int j = 0;
    bool o_codes = kFp8;                // FP8: O holds prefix values in code units
    auto to_values = [&]() {            // O from code units to values (once)
        if (kFp8 && o_codes) {
#pragma unroll
            for (int d = 0; d < kD / 32; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) S.o[d][i] *= a.v_scale;
            o_codes = false;
        }
    };
    if constexpr (!kFp8) {
        const int n_vis_first = n_iss;      // blocks in flight before the first wait
        if (kb_cur < kb1) {
            ring_wait((n_vis_first - 1) * kOps);          // block 0 has landed
            asm volatile("" : "+v"(qraw[0]), "+v"(qraw[1]), "+v"(qraw[2]), "+v"(qraw[3]),
                              "+v"(qraw[4]), "+v"(qraw[5]), "+v"(qraw[6]), "+v"(qraw[7]));
#pragma unroll
            for (int t = 0; t < kD / 16; ++t) qf[t] = as_bf16x8(qraw[t]);
            qk(stage_of(0), sa0, sa1);
            apply_mask(stage_of(0), kb_cur, sa0, sa1);
            mx_cur = row_max(sa0, sa1);
        }
        // block j with a visible successor kb_nxt (which has landed after the wait)
        auto iter_next = [&](f32x16 &sc0, f32x16 &sc1, f32x16 &sn0, f32x16 &sn1, int kb_nxt) {
            ring_wait((n_iss - (j + 2)) * kOps);            // blocks issued after j+1 stay in flight
            if (kb_iss < kb1) {                             // the stage of block j-1 is free
                issue_block<kPaged, kDm>(a, c, s_pages, ring0 + (n_iss % kNS) * kStage, kb_iss, bad);
                kb_iss = next_vis(kb_iss + 1);
                ++n_iss;
            }
            rescale(mx_cur);
            mx_cur = step(Flag<true>{}, stage_of(j), stage_of(j + 1), kb_nxt, sc0, sc1, sn0, sn1, a.c2);
            kb_cur = kb_nxt;
            ++j;
        };
        // the last visible block (it landed before the previous step)
        auto iter_last = [&](f32x16 &sc0, f32x16 &sc1) {
            rescale(mx_cur);
            step(Flag<false>{}, stage_of(j), stage_of(j), kb_cur, sc0, sc1, sc0, sc1, a.c2);
        };
        if (kb_cur < kb1) {
            // the loop only runs blocks with a successor (the last block's step is
            // outside it, which keeps the loop's register pressure down)
            bool in_b = false;                              // the last block's scores sit in sb
            for (;;) {
                int kn = next_vis(kb_cur + 1);
                if (kn >= kb1) break;
                iter_next(sa0, sa1, sb0, sb1, kn);
                kn = next_vis(kb_cur + 1);
                if (kn >= kb1) { in_b = true; break; }
                iter_next(sb0, sb1, sa0, sa1, kn);
            }
            if (in_b) iter_last(sb0, sb1);
            else iter_last(sa0, sa1);
        }
    } else {
        // FP8 prefix blocks, one block in flight.  Thread t moves 16 codes
        // (head dims 16 (t % 8) .. +15) of key row t / 8 of the K and V tiles.
        const int r8 = tid >> 3, c8 = tid & 7;
        __amdgpu_buffer_rsrc_t rk8, rv8;
        if constexpr (!kPaged) {
            const uint32_t nbytes = c.pzero ? 0u : (uint32_t)P * c.rowb8;
            rk8 = make_rsrc(c.kc8, nbytes);
            rv8 = make_rsrc(c.vc8, nbytes);
        } else {
            rk8 = make_rsrc(a.k_cache, a.cache_bytes);
            rv8 = make_rsrc(a.v_cache, a.cache_bytes);
        }
        u32x4 k8 = {0u, 0u, 0u, 0u}, v8 = {0u, 0u, 0u, 0u};
        auto issue8 = [&](int kb, int slot) {
            if (kb >= nPB) {                              // tree block: bf16 copies as usual
                issue_block<kPaged, kDm>(a, c, s_pages, ring0 + slot * kStage, kb, bad);
                return;
            }
            const int pos = kb * kKB + r8;
            uint32_t off = kOob;
            if (pos < P && c8 * 16 < kDm) {
                if constexpr (!kPaged) {
                    off = (uint32_t)pos * c.rowb8 + c8 * 16u;
                } else {
                    int pg, slot_in;
                    if (a.page_shift >= 0) {
                        pg = pos >> a.page_shift;
                        slot_in = pos & (a.page_size - 1);
                    } else {
                        pg = pos / a.page_size;
                        slot_in = pos - pg * a.page_size;
                    }
                    const int page = s_pages[pg - c.page0];
                    if (page >= 0 && page < a.num_pages)
                        off = (((uint32_t)page * a.page_size + slot_in) * a.Hkv + g) * kDm + c8 * 16u;
                    else
                        bad = true;
                }
            }
            k8 = __builtin_amdgcn_raw_buffer_load_b128(rk8, off, 0, 0);
            v8 = __builtin_amdgcn_raw_buffer_load_b128(rv8, off, 0, 0);
        };
        // wait for this wave's loads of block kb, then (a prefix block) write
        // its codes as bf16 into stage `slot` (E4M3 -> bf16 is exact)
        auto commit8 = [&](int kb, int slot) {
            __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));   // vmcnt(0)
            if (kb >= nPB) return;
            lds_t *st = (lds_t *)&ring[slot][0];
            auto cvt16 = [](const u32x4 &x, u32x4 &lo, u32x4 &hi) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t e01 = __builtin_bit_cast(uint32_t,
                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, false));
                    const uint32_t e23 = __builtin_bit_cast(uint32_t,
                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], 1.0f, true));
                    if (w < 2) { lo[2 * w] = e01; lo[2 * w + 1] = e23; }
                    else { hi[2 * (w - 2)] = e01; hi[2 * (w - 2) + 1] = e23; }
                }
            };
            u32x4 lo, hi;
            cvt16(k8, lo, hi);
            lds_t *kp = st + k_lds(r8) + c8 * 32;
            *(__attribute__((address_space(3))) u32x4 *)kp = lo;
            *(__attribute__((address_space(3))) u32x4 *)(kp + 16) = hi;
            cvt16(v8, lo, hi);
            lds_t *vp = st + kKTile + v_lds(r8) + c8 * 32;
            *(__attribute__((address_space(3))) u32x4 *)vp = lo;
            *(__attribute__((address_space(3))) u32x4 *)(vp + 16) = hi;
        };
        auto scaled_max = [&](float mx, int kb) { return kb < nPB ? mx * a.k_scale : mx; };
        auto coef = [&](int kb) { return kb < nPB ? a.c2k : a.c2; };
        if (kb_cur < kb1) {
            issue8(kb_cur, 0);
            commit8(kb_cur, 0);
            lds_barrier();
            asm volatile("" : "+v"(qraw[0]), "+v"(qraw[1]), "+v"(qraw[2]), "+v"(qraw[3]),
                              "+v"(qraw[4]), "+v"(qraw[5]), "+v"(qraw[6]), "+v"(qraw[7]));
#pragma unroll
            for (int t = 0; t < kD / 16; ++t) qf[t] = as_bf16x8(qraw[t]);
            const int kn = next_vis(kb_cur + 1);
            if (kn < kb1) issue8(kn, 1);
            qk(stage_of(0), sa0, sa1);
            apply_mask(stage_of(0), kb_cur, sa0, sa1);
            mx_cur = scaled_max(row_max(sa0, sa1), kb_cur);
        }
        auto iter_next = [&](f32x16 &sc0, f32x16 &sc1, f32x16 &sn0, f32x16 &sn1, int kb_nxt) {
            commit8(kb_nxt, (j + 1) % kNS);               // block j+1 into its stage
            lds_barrier();                                // ... visible to every wave
            const int kn = next_vis(kb_nxt + 1);
            if (kn < kb1) issue8(kn, (j + 2) % kNS);      // the stage of block j-2 is free
            rescale(mx_cur);
            if (kb_cur >= nPB) to_values();
            const float mx = step(Flag<true>{}, stage_of(j), stage_of(j + 1), kb_nxt, sc0, sc1, sn0, sn1,
                                  coef(kb_cur));
            mx_cur = scaled_max(mx, kb_nxt);
            kb_cur = kb_nxt;
            ++j;
        };
        auto iter_last = [&](f32x16 &sc0, f32x16 &sc1) {
            rescale(mx_cur);
            if (kb_cur >= nPB) to_values();
            step(Flag<false>{}, stage_of(j), stage_of(j), kb_cur, sc0, sc1, sc0, sc1, coef(kb_cur));
        };
        if (kb_cur < kb1) {
            bool in_b = false;
            for (;;) {
                int kn = next_vis(kb_cur + 1);
                if (kn >= kb1) break;
                iter_next(sa0, sa1, sb0, sb1, kn);
                kn = next_vis(kb_cur + 1);
                if (kn >= kb1) { in_b = true; break; }
                iter_next(sb0, sb1, sa0, sa1, kn);
            }
            if (in_b) iter_last(sb0, sb1);
            else iter_last(sa0, sa1);
        }
        to_values();                                      // a piece of prefix blocks only
    }

    if (bad) s_bad = 1;  // benign race: every writer stores 1
    float l_run = sum_halves(S.l);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse_v = l_run > 0.f ? S.m * a.scale + logf(l_run) : -INFINITY;
    // The wave's 32 output rows are stored row-contiguous: each lane leaves
    // its 4-column parts in LDS (the ring is idle once every copy has landed
    // and every wave is past its last step), then the wave writes 16-byte
    // chunks, 1 KiB per store instruction.  (A lane's own parts would
    // scatter 8 or 16 bytes over 32 rows per store instruction.)  The only
    // piece with keys writes the bf16 output; otherwise the fp32 partials of
    // the work item's rows.
    ring_barrier<0>();
    if (single) {
        constexpr int kOutRow = kRow + 16;              // padded row: rows fall on shifted banks
        lds_t *ob = (lds_t *)&ring[0][0] + wave * 32 * kOutRow;
#pragma unroll
        for (int d = 0; d < kD / 32; ++d)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(S.o[d][gq * 4 + 0] * inv, S.o[d][gq * 4 + 1] * inv);
                w[1] = pack_bf16x2(S.o[d][gq * 4 + 2] * inv, S.o[d][gq * 4 + 3] * inv);
                *(__attribute__((address_space(3))) u32x2 *)(ob + l32 * kOutRow + (d * 32 + gq * 8 + half * 4) * 2) = w;
            }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int cc = 0; cc < 32 * (kRow / 16) / kWave; ++cc) {
            const int idx = cc * kWave + lane, row = idx >> 4, ch = idx & 15;
            const int rr = qt * kTQ + wave * 32 + row;
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(ob + row * kOutRow + ch * 16);
            if (rr < R && ch * 8 < kDm) {
                const int64_t orow = (node0 + rr / a.G) * a.Hq + g * a.G + rr % a.G;
                *(u32x4 *)((uint16_t *)a.out + orow * kDm + ch * 8) = v;
            }
        }
        if (row_ok && half == 0 && a.lse) a.lse[(node0 + node) * a.Hq + hq] = lse_v;
    } else {
        constexpr int kPRow = kD * 4 + 16;              // padded fp32 row
        lds_t *ob = (lds_t *)&ring[0][0] + wave * 32 * kPRow;
#pragma unroll
        for (int d = 0; d < kD / 32; ++d)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 w = {S.o[d][gq * 4 + 0] * inv, S.o[d][gq * 4 + 1] * inv,
                                 S.o[d][gq * 4 + 2] * inv, S.o[d][gq * 4 + 3] * inv};
                *(__attribute__((address_space(3))) f32x4 *)(ob + l32 * kPRow + (d * 32 + gq * 8 + half * 4) * 4) = w;
            }
        __builtin_amdgcn_wave_barrier();
        float *pbase = a.part_o + (prow0 + wave * 32) * kD;
#pragma unroll
        for (int cc = 0; cc < 32 * (kD * 4 / 16) / kWave; ++cc) {
            const int idx = cc * kWave + lane, row = idx >> 5, ch = idx & 31;
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(ob + row * kPRow + ch * 16);
            if (qt * kTQ + wave * 32 + row < R) *(u32x4 *)(pbase + row * kD + ch * 4) = v;
        }
        if (row_ok && half == 0) a.part_lse[prow0 + wave * 32 + l32] = lse_v;
    }
    if (tid == 0 && a.status) {
        if (s_bad) *a.status = JF_ERR_BAD_PAGE;
        if (pbad) *a.status = JF_ERR_BAD_PREFIX;
    }
}

// Combine the pieces of one row: O = sum_s w_s O_s / sum_s w_s with
// w_s = exp(lse_s - max lse); lse = max + log sum w_s.  Sixteen threads per
// row, eight output columns (two 16-byte loads per piece) each; one pass over
// the pieces, four at a time, rescaling when the running maximum moves.  The
// grid's y index is the dispatch position of the sequence; pieces that start
// past the real length have no keys and were not written (the split kernel
// reads the same length), and a row whose first piece holds every real block
// was written by the split kernel.
constexpr int kMergeTPR = kD / 8;        // threads per row
__global__ __launch_bounds__(256) void k_tree_attn_merge(AttnArgs a) {
    const int sub = threadIdx.x % kMergeTPR;
    const int pos = blockIdx.y;
    const int b = a.seq_order[pos];
    const int n = a.node_off[b + 1] - a.node_off[b];
    bool pbad = false;
    const int P = prefix_of(a, b, pbad);
    const int nB = div_up(P, kKB) + div_up(n, kKB);
    const int nbc = div_up(a.cap[b], kKB) + div_up(n, kKB);
    const int np = div_up(nbc, a.L);
    if (piece_start(1, nbc, np) >= nB) return;               // written by the split kernel
    const int in_seq = blockIdx.x * (256 / kMergeTPR) + threadIdx.x / kMergeTPR;
    if (in_seq >= n * a.Hq || sub * 8 >= a.D) return;    // (sub 0 writes the lse)
    const int64_t flat = (int64_t)a.node_off[b] * a.Hq + in_seq;
    const int hq = in_seq % a.Hq;
    const int node = in_seq / a.Hq;
    const int g = hq / a.G;
    const int r = node * a.G + hq % a.G;
    const int n_qt = div_up(n * a.G, kTQ);
    // piece c's work item: item_start[pos] + (c * Hkv + g) * n_qt + r / kTQ
    const int64_t row0 = ((int64_t)a.item_start[pos] + (int64_t)g * n_qt + r / kTQ) * kTQ + r % kTQ;
    const int64_t stride = (int64_t)a.Hkv * n_qt * kTQ;      // rows between consecutive pieces
    const float *po = a.part_o + row0 * kD + sub * 8;
    int nc = np;                                             // pieces with keys
    while (nc > 1 && piece_start(nc - 1, nbc, np) >= nB) --nc;
    float M = -INFINITY;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    constexpr int kGroup = 4;
    for (int c = 0; c < nc; c += kGroup) {
        float l[kGroup];
        f32x4 v0[kGroup], v1[kGroup];
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const bool ok = c + u < nc;
            l[u] = ok ? a.part_lse[row0 + (c + u) * stride] : -INFINITY;
            v0[u] = ok ? *(const f32x4 *)(po + (c + u) * stride * kD) : f32x4{0.f, 0.f, 0.f, 0.f};
            v1[u] = ok ? *(const f32x4 *)(po + (c + u) * stride * kD + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float mg = M;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) mg = fmaxf(mg, l[u]);
        if (mg == -INFINITY) continue;                       // nothing visible yet
        const float alpha = M == -INFINITY ? 0.f : __expf(M - mg);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        wsum *= alpha;
        M = mg;
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const float w = l[u] == -INFINITY ? 0.f : __expf(l[u] - M);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += w * v0[u][e];
                acc[4 + e] += w * v1[u][e];
            }
            wsum += w;
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *(u32x4 *)((uint16_t *)a.out + flat * a.D + sub * 8) = o;
    if (a.lse && sub == 0) a.lse[flat] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// fp32 path: one wavefront per (tree row, query head); keys are taken 64 at a
// time (one per lane), scores in fp32, online softmax with expf, each lane
// accumulating D/64 output columns.  Meant for small problems.  A bad page id
// reads as a zero key (score 0) with a zero value, as on the bf16 path.
struct AttnArgsF32 {
    const float *q, *k_tree, *v_tree;
    const uint64_t *mask;
    const float *k_cache, *v_cache;
    const int32_t *block_table;
    const int32_t *prefix_dev;
    float *out, *lse;
    int32_t *status;
    int64_t num_pages;
    int page_size, max_pages, B, Hq, Hkv, G, W, D;
    float scale;
    int cap[kMaxBatch];
    int node_off[kMaxBatch + 1];
};

constexpr int kF32MaxD = 128;

__global__ __launch_bounds__(256) void k_tree_attn_f32(AttnArgsF32 a) {
    __shared__ float sq[4][kF32MaxD];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t flat = (int64_t)blockIdx.x * 4 + wv;
    const int64_t total = (int64_t)a.node_off[a.B] * a.Hq;
    if (flat >= total) return;
    const int hq = (int)(flat % a.Hq);
    const int64_t t = flat / a.Hq;                // tree row
    int b = 0;
    {
        int hi = a.B - 1;
        while (b < hi) {
            const int mid = (b + hi + 1) >> 1;
            if (a.node_off[mid] <= t) b = mid; else hi = mid - 1;
        }
    }
    const int64_t node0 = a.node_off[b];
    const int n = a.node_off[b + 1] - a.node_off[b];
    const int node = (int)(t - node0);
    const int g = hq / a.G;
    const int D = a.D;
    bool pbad = false;
    int P = a.cap[b];
    if (a.prefix_dev) {
        const int pd = a.prefix_dev[b];
        if (pd < 0 || pd > P) pbad = true;
        P = pd < 0 ? 0 : (pd > P ? P : pd);
    }
    for (int d = lane; d < D; d += 64) sq[wv][d] = a.q[flat * D + d];
    __builtin_amdgcn_wave_barrier();
    const uint64_t *mrow = a.mask + t * a.W;
    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    bool bad = false;
    const int nkeys = P + n;
    for (int kc = 0; kc < nkeys; kc += 64) {
        const int key = kc + lane;
        bool valid = false;
        int64_t off = -1;                         // -1: a zero key and value
        const float *kbase = a.k_cache;
        if (key < P) {
            int64_t page = a.block_table[(int64_t)b * a.max_pages + key / a.page_size];
            valid = true;
            if (page >= 0 && page < a.num_pages)
                off = ((page * a.page_size + key % a.page_size) * a.Hkv + g) * (int64_t)D;
            else
                bad = true;
        } else if (key < nkeys) {
            const int j = key - P;
            valid = (mrow[j >> 6] >> (j & 63)) & 1ull;
            off = ((node0 + j) * a.Hkv + g) * (int64_t)D;
            kbase = a.k_tree;
        }
        float s = -INFINITY;
        if (valid) {
            float dot = 0.f;
            if (off >= 0) {
                const float *kr = kbase + off;
                for (int d = 0; d < D; ++d) dot = fmaf(sq[wv][d], kr[d], dot);
            }
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
        for (int jj = 0; jj < 64; ++jj) {
            const float pj = __shfl(p, jj);
            const int64_t oj = __shfl(off, jj);
            if (pj == 0.f || oj < 0) continue;    // uniform across the wave
            const bool tree_j = (kc + jj) >= P;
            const float *vr = (tree_j ? a.v_tree : a.v_cache) + oj;
            if (lane < D) acc0 = fmaf(pj, vr[lane], acc0);
            if (lane + 64 < D) acc1 = fmaf(pj, vr[lane + 64], acc1);
        }
        m = mn;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (lane < D) a.out[flat * D + lane] = acc0 * inv;
    if (lane + 64 < D) a.out[flat * D + lane + 64] = acc1 * inv;
    if (a.lse && lane == 0) a.lse[flat] = l > 0.f ? m + logf(l) : -INFINITY;
    if (a.status && lane == 0) {
        if (bad) *a.status = JF_ERR_BAD_PAGE;
        if (pbad) *a.status = JF_ERR_BAD_PREFIX;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Split planning from the prefix bounds.  Every (sequence, KV head, query
// tile) is a row of 64-key blocks.  The piece target is L = ceil(units /
// compute units) blocks (about one workgroup per compute unit's share; a
// workgroup fills a compute unit's LDS), never less than two; a row of nb
// blocks is cut into np = ceil(nb / L) pieces of ceil(nb / np) blocks (the
// last one shorter), so no piece exceeds L and a long row does not leave a
// tiny remainder.  Sequences are dispatched in decreasing piece size
// (longest first): the hardware hands each workgroup to the compute unit that
// frees first, and the short pieces of ragged batches then fill the gaps at
// the end.  When the pieces spill over one wave of workgroups, a few piece
// sizes are compared by a model of that dispatch (below).  A caller that runs
// other work beside the attention can plan it for fewer compute units.
void plan_tree_attn(AttnPlan &p, int B, int N, int Hq, int Hkv, int D, int page_size,
                    const int32_t *prefix_cap, const int32_t *node_off, jf_dtype dtype, int cus) {
    p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.D = D;
    p.page_size = page_size;
    p.G = Hq / Hkv;
    p.W = (N + 63) / 64;
    std::vector<int64_t> nb((size_t)B), rows((size_t)B);
    int64_t units = 0, max_blocks = 1, Pmax = 0;
    for (int b = 0; b < B; ++b) {
        p.cap[b] = prefix_cap[b];
        p.node_off[b] = node_off ? node_off[b] : b * N;
        const int64_t n = node_off ? node_off[b + 1] - node_off[b] : N;
        nb[b] = (prefix_cap[b] + kKB - 1) / kKB + (n + kKB - 1) / kKB;
        rows[b] = (int64_t)Hkv * ((n * p.G + kTQ - 1) / kTQ);
        units += nb[b] * rows[b];
        if (nb[b] > max_blocks) max_blocks = nb[b];
        if (prefix_cap[b] > Pmax) Pmax = prefix_cap[b];
    }
    p.node_off[B] = node_off ? node_off[B] : B * N;
    const int64_t target = cus > 0 && cus < num_cus() ? (int64_t)cus : (int64_t)num_cus();
    int64_t L = (units + target - 1) / target;
    if (L < 2) L = 2;
    // a piece's page ids must fit the LDS staging array
    int64_t Lmax = max_blocks;
    if (page_size < Pmax) {
        int64_t cap = ((int64_t)(kPageLds - 2) * page_size) / kKB;
        if (cap < 1) cap = 1;
        if (Lmax > cap) Lmax = cap;
    }
    if (L > Lmax) L = Lmax;
    if (dtype == JF_F32) L = max_blocks;                  // the fp32 path does not split

    // Pieces of at most Lc blocks: np[b] pieces of piece[b] blocks (the last
    // shorter), sequences in decreasing piece size (ties: lower sequence
    // first).  Returns the work item count.
    std::vector<int64_t> np((size_t)B), piece((size_t)B);
    std::vector<int> order((size_t)B);
    auto build = [&](int64_t Lc) {
        int64_t items = 0;
        for (int b = 0; b < B; ++b) {
            np[b] = (nb[b] + Lc - 1) / Lc;
            piece[b] = (nb[b] + np[b] - 1) / np[b];
            order[(size_t)b] = b;
            items += np[b] * rows[b];
        }
        std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return piece[x] > piece[y]; });
        return items;
    };
    const int64_t items0 = build(L);
    // More work items than compute units: the pieces after the first wave
    // may leave a long tail (just over one wave is the worst case).  A few
    // piece sizes are then compared by a model of the dispatch and the
    // shortest predicted span wins (ties: the larger pieces, fewer partials).
    // The model follows the launch: workgroup ids are dealt round-robin over
    // the XCDs and mapped to work items by xcd_interleave; each XCD hands its
    // items in id order to whichever of its compute units frees first; an
    // item costs a fixed overhead of 4 blocks plus its blocks.
    if (dtype != JF_F32 && items0 > target && items0 <= 16 * target) {
        std::vector<int64_t> cost;
        auto span_of = [&](int64_t Lc) {
            build(Lc);
            constexpr int64_t kOverhead = 4;
            cost.clear();
            for (int i = 0; i < B; ++i) {
                const int b = order[(size_t)i];
                for (int64_t k = 0; k < np[b]; ++k) {
                    const int64_t k0 = k * piece[b];
                    const int64_t size = (k0 + piece[b] < nb[b] ? piece[b] : nb[b] - k0) + kOverhead;
                    for (int64_t r = 0; r < rows[b]; ++r) cost.push_back(size);
                }
            }
            const int64_t n = (int64_t)cost.size();
            const int nq = target >= kNumXcd ? kNumXcd : 1;           // too few units to split: one pool
            typedef std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> Queue;
            std::vector<Queue> free_at((size_t)nq);
            for (int x = 0; x < nq; ++x)
                for (int64_t c = 0; c < target / nq + (x < target % nq ? 1 : 0); ++c) free_at[(size_t)x].push(0);
            int64_t span = 0;
            for (int64_t bid = 0; bid < n; ++bid) {
                Queue &q = free_at[(size_t)(bid % nq)];
                const int64_t t = q.top() + cost[(size_t)xcd_interleave((int)bid, (int)n)];
                q.pop();
                q.push(t);
                span = t > span ? t : span;
            }
            return span;
        };
        // the smallest piece size whose items fit in w waves (below L too:
        // smaller pieces that fill two or three waves completely can beat
        // larger ones that leave the last wave part empty)
        auto fit_waves = [&](int64_t w) {
            int64_t lo = 2, hi = Lmax;
            if (build(hi) > w * target) return (int64_t)-1;
            while (lo < hi) {
                const int64_t mid = (lo + hi) / 2;
                if (build(mid) <= w * target) hi = mid; else lo = mid + 1;
            }
            return lo;
        };
        // The model ignores the partials' traffic and the merge; a size other
        // than L is taken only when it predicts a span at least 10 % shorter
        // (measured on the serving batch of 32 ragged prefixes: L = 68
        // predicted 96, the chosen 46 predicted 80; 46 ran 3 % faster than 51,
        // the choice of a model with one pool of compute units, and 10-15 %
        // faster than 28-40 blocks).
        const int64_t span0 = span_of(L);
        std::vector<int64_t> cand = {(3 * L + 3) / 4, (L + 1) / 2};
        for (int64_t w = 1; w <= 3; ++w) {
            // w waves filled, and slightly larger pieces that leave a few
            // units of the last wave free for the longest rows' tails
            const int64_t c = fit_waves(w);
            if (c < 0) continue;
            for (int64_t d = 0; d <= 2; ++d) cand.push_back(c + d);
        }
        int64_t best_L = L, best = -1;
        for (int64_t c : cand) {
            if (c < 2 || c > Lmax || c == L) continue;
            const int64_t sp = span_of(c);
            if (best < 0 || sp < best || (sp == best && c > best_L)) { best = sp; best_L = c; }
        }
        if (best < 0 || 10 * best > 9 * span0) best_L = L;
        L = best_L;
        build(L);
    }
    p.L = (int)L;
    int64_t items = 0;
    for (int b = 0; b < B; ++b) items += np[b] * rows[b];
    // work item indices and the grid are 32-bit: refuse plans beyond 2^30 items
    p.fits = items <= ((int64_t)1 << 30);
    p.any_split = false;
    items = 0;
    for (int i = 0; i < B; ++i) {
        const int b = order[(size_t)i];
        p.seq_order[i] = (uint8_t)b;
        p.item_start[i] = p.fits ? (int)items : 0;
        if (np[b] > 1) p.any_split = true;
        items += np[b] * rows[b];
    }
    p.item_start[B] = p.fits ? (int)items : 0;
    p.total_items = p.fits ? (int)items : 0;
}

size_t tree_attn_workspace_bytes(const AttnPlan &p) {
    if (!p.any_split) return 0;
    const size_t rows = (size_t)p.total_items * kTQ;
    return rows * kD * sizeof(float) + rows * sizeof(float);
}

hipError_t launch_tree_attn_bf16(const AttnPlan &p, const void *q, const void *k_tree,
                                 const void *v_tree, const uint64_t *mask, const void *k_cache,
                                 const void *v_cache, int64_t num_pages, int page_size,
                                 const int32_t *block_table, int max_pages,
                                 const int32_t *prefix_dev, float scale, bool fp8, float k_scale,
                                 float v_scale, void *out, float *lse, void *workspace,
                                 int32_t *status, hipStream_t s) {
    AttnArgs a;
    a.q = (const uint16_t *)q;
    a.k_tree = (const uint16_t *)k_tree;
    a.v_tree = (const uint16_t *)v_tree;
    a.mask = mask;
    a.k_cache = (const uint16_t *)k_cache;
    a.v_cache = (const uint16_t *)v_cache;
    a.block_table = block_table;
    a.prefix_dev = prefix_dev;
    a.out = out;
    a.lse = lse;
    const size_t rows = (size_t)p.total_items * kTQ;
    a.part_o = p.any_split ? (float *)workspace : nullptr;
    a.part_lse = p.any_split ? (float *)((char *)workspace + rows * kD * sizeof(float)) : nullptr;
    a.status = status;
    const int64_t T = p.node_off[p.B];
    a.D = p.D;
    a.q_bytes = (uint32_t)(T * p.Hq * p.D * 2);
    a.tree_bytes = (uint32_t)(T * p.Hkv * p.D * 2);
    a.cache_bytes = (uint32_t)(num_pages * page_size * (int64_t)p.Hkv * p.D * (fp8 ? 1 : 2));
    a.mask_bytes = (uint32_t)(T * p.W * 8);
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
        for (int b = 0; b < p.B; ++b) Pmax = p.cap[b] > Pmax ? p.cap[b] : Pmax;
        a.page_mode = (max_pages == 1 && page_size >= Pmax) ? 1
                      : (a.page_shift >= 4 ? 2 : 0);
    }
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.W = p.W;
    a.L = p.L;
    a.total_items = p.total_items;
    a.scale = scale;
    a.c2 = scale * kLog2e;
    a.lazy_raw = kLazyLog2 / a.c2;
    a.k_scale = fp8 ? k_scale : 1.f;
    a.v_scale = fp8 ? v_scale : 1.f;
    a.c2k = a.c2 * a.k_scale;
    for (int b = 0; b < p.B; ++b) a.cap[b] = p.cap[b];
    for (int b = 0; b <= p.B; ++b) {
        a.node_off[b] = p.node_off[b];
        a.item_start[b] = p.item_start[b];
    }
    for (int i = 0; i < p.B; ++i) a.seq_order[i] = p.seq_order[i];
    const dim3 grid(p.total_items), block(kNW * kWave);
    auto launch = [&](auto dm) {
        constexpr int kDm = decltype(dm)::value;
        if (a.page_mode == 1) {
            if (fp8) hipLaunchKernelGGL((k_tree_attn_split<false, true, kDm>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_tree_attn_split<false, false, kDm>), grid, block, 0, s, a);
        } else {
            if (fp8) hipLaunchKernelGGL((k_tree_attn_split<true, true, kDm>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_tree_attn_split<true, false, kDm>), grid, block, 0, s, a);
        }
    };
    if (p.D == 64) launch(std::integral_constant<int, 64>{});
    else launch(std::integral_constant<int, kD>{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !p.any_split) return e;
    const int64_t per_seq = (int64_t)p.N * p.Hq;
    const int64_t rows_per_wg = 256 / kMergeTPR;
    hipLaunchKernelGGL(k_tree_attn_merge, dim3((unsigned)((per_seq + rows_per_wg - 1) / rows_per_wg), (unsigned)p.B),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tree_attn_f32(const AttnPlan &p, const float *q, const float *k_tree,
                                const float *v_tree, const uint64_t *mask, const float *k_cache,
                                const float *v_cache, int64_t num_pages, int page_size,
                                const int32_t *block_table, int max_pages, const int32_t *prefix_dev,
                                float scale, float *out, float *lse, int32_t *status,
                                hipStream_t s) {
    AttnArgsF32 a;
    a.q = q; a.k_tree = k_tree; a.v_tree = v_tree; a.mask = mask;
    a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.prefix_dev = prefix_dev;
    a.out = out; a.lse = lse; a.status = status;
    a.num_pages = num_pages; a.page_size = page_size; a.max_pages = max_pages;
    a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.W = p.W; a.D = p.D;
    a.scale = scale;
    for (int b = 0; b < p.B; ++b) a.cap[b] = p.cap[b];
    for (int b = 0; b <= p.B; ++b) a.node_off[b] = p.node_off[b];
    const int64_t total = (int64_t)p.node_off[p.B] * p.Hq;
    hipLaunchKernelGGL(k_tree_attn_f32, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace jf
