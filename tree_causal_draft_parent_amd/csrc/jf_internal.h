// jf_internal.h -- shared device types and launcher declarations of libjf.
// gfx950 only: wave64, MFMA bf16 32x32x16, 160 KiB LDS per CU, 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jf.h"

namespace jf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Consecutive workgroup ids are spread round-robin over the XCDs.  Map the
// hardware id so that the workgroups landing on one XCD get one contiguous
// range of logical ids: neighbours in logical order then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    int xcd = bid % kNumXcd, local = bid / kNumXcd;
    int q = n / kNumXcd, rem = n % kNumXcd;
    return xcd * q + (xcd < rem ? xcd : rem) + local;
}

typedef __attribute__((address_space(3))) char lds_t;

// Buffer resource over [p, p + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOob = 0xffffff00u;  // an offset past every buffer (reads as zeros)

// One 16-byte-per-lane copy HBM -> LDS: lane L's 16 bytes land at lds + 16 L
// (lds must be wave-uniform).  Issued as inline asm so that the compiler does
// not order later LDS reads of another stage behind it; completion is waited
// for explicitly with stage_barrier().
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(r) : "memory");
}

// Wait for this wave's outstanding memory operations, then barrier: every
// wave's copies into the current stage have landed and no wave still reads
// the other stage.  The wait is the s_waitcnt builtin (not asm) so that the
// compiler knows every older load is complete; the empty asm is a compiler
// fence for memory.
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima), then barrier.  Used by multi-stage copy rings where
// later stages' copies stay in flight.
template <int kN>
__device__ __forceinline__ void ring_barrier() {
    static_assert(kN >= 0 && kN < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kN & 0xf) | ((kN >> 4) << 14) | (0x7 << 4) | (0xf << 8));
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Device properties cached once per process and device.
int num_cus();

// ----- launchers (host) ------------------------------------------------------
constexpr int kMaxBatch = 256;

// node_off: HOST [B+1] packed node offsets (B <= kMaxBatch), or NULL for N
// nodes per sequence.
hipError_t launch_tree_mask(const int32_t *parent, const int32_t *node_off, int B, int N,
                            uint64_t *mask, int32_t *depth, int32_t *seq_status, hipStream_t s);

hipError_t launch_path_scores(const int32_t *parent, const float *logp, int B, int N, float *score,
                              int32_t *seq_status, hipStream_t s);

hipError_t launch_tree_accept(const int32_t *parent, const int32_t *token,
                              const int32_t *target_next, const int32_t *root_next, int B, int N,
                              int32_t *accept_len, int32_t *accept_node, int32_t *next_token,
                              int32_t *path, int32_t *seq_status, hipStream_t s);

hipError_t launch_tree_rope(void *q, void *k, const int32_t *depth, const int32_t *prefix_len,
                            int B, int N, int Hq, int Hkv, int D, double theta, jf_dtype dtype,
                            hipStream_t s);

hipError_t launch_rmsnorm(const void *x, int64_t rows, int H, int64_t ldx, const void *w, float eps,
                          jf_dtype dtype, void *y, hipStream_t s);

hipError_t launch_swiglu(const void *gu, int64_t M, int64_t I, int64_t ld, jf_dtype dtype, void *y,
                         hipStream_t s);

// One expansion step sorts every (node, rank) candidate of a sequence in LDS.
constexpr int kExpandMaxCands = 16384;
hipError_t launch_tree_expand(const float *score, const int32_t *depth, const int32_t *idx,
                              const float *val, const float *lse, const int32_t *parent,
                              const int32_t *token, int B, int N, int k, int M,
                              int max_depth, int32_t *new_parent, int32_t *new_token,
                              float *new_score, int32_t *new_depth, hipStream_t s);

struct AttnPlan {
    int B, N, Hq, Hkv, D, G, W;    // N: the largest tree; W = ceil(N / 64) mask words a row
    int L;               // longest piece of a row (64-key blocks)
    int page_size;
    int total_items;     // workgroups of the split kernel
    bool any_split;      // some row has more than one piece (by the bounds)
    bool fits;           // the work items fit 32-bit indices (else the call is refused)
    int cap[kMaxBatch];              // planned prefix bound of each sequence
    int node_off[kMaxBatch + 1];     // tree rows of sequence b: node_off[b] .. node_off[b+1]-1
    int item_start[kMaxBatch + 1];   // first work item of the sequence at dispatch position p
    uint8_t seq_order[kMaxBatch];    // sequence at dispatch position p (longest pieces first)
};
// prefix_cap: HOST [B] prefix bounds (the lengths themselves when no device
// lengths are given); node_off: HOST [B+1] packed tree rows or NULL (N a
// sequence); cus: compute units the split plan fills (<= 0: all).
void plan_tree_attn(AttnPlan &p, int B, int N, int Hq, int Hkv, int D, int page_size,
                    const int32_t *prefix_cap, const int32_t *node_off, jf_dtype dtype,
                    int cus = 0);
size_t tree_attn_workspace_bytes(const AttnPlan &p);

hipError_t launch_tree_attn_bf16(const AttnPlan &p, const void *q, const void *k_tree,
                                 const void *v_tree, const uint64_t *mask,
                                 const void *k_cache, const void *v_cache,
                                 int64_t num_pages, int page_size,
                                 const int32_t *block_table, int max_pages,
                                 const int32_t *prefix_dev, float scale, bool fp8,
                                 float k_scale, float v_scale,
                                 void *out, float *lse, void *workspace,
                                 int32_t *status, hipStream_t s);
hipError_t launch_tree_attn_f32(const AttnPlan &p, const float *q, const float *k_tree,
                                const float *v_tree, const uint64_t *mask,
                                const float *k_cache, const float *v_cache,
                                int64_t num_pages, int page_size,
                                const int32_t *block_table, int max_pages,
                                const int32_t *prefix_dev, float scale,
                                float *out, float *lse, int32_t *status,
                                hipStream_t s);

struct TopkPlan {
    int64_t R, V;
    int k;
    int chunks;        // splits of each row
    int64_t chunk_len; // elements per split (multiple of 512)
};
void plan_topk(TopkPlan &p, int64_t R, int64_t V, int k, jf_dtype dtype);
size_t topk_workspace_bytes(const TopkPlan &p);
hipError_t launch_topk(const TopkPlan &p, const void *logits, int64_t ld, jf_dtype dtype,
                       int32_t *idx, float *val, float *lse, void *workspace, hipStream_t s);
// The allocation-free top-k's static device scratch: its size, and its
// address on the current device (taken once per device).
constexpr size_t kTopkScratchBytes = JF_NODE_TOPK_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
hipError_t topk_scratch(void **ptr);

struct FusePlan {
    int64_t M, H_in, H_out;
    int k;
    int bm, bn;        // output tile
    int split_k;       // K slices (>1 uses the fp32 partial workspace)
    int64_t k_per_split;
};
// cus: compute units the split-K plan fills (<= 0: all of the device's)
void plan_fuse(FusePlan &p, int64_t M, int64_t H_in, int k, int64_t H_out, jf_dtype in_dtype,
               int cus = 0);
size_t fuse_workspace_bytes(const FusePlan &p);
hipError_t launch_fuse_bf16(const FusePlan &p, const void *const *x, int64_t ldx,
                            const void *w, void *y, jf_dtype out_dtype, void *workspace,
                            hipStream_t s);
hipError_t launch_fuse_f32(const FusePlan &p, const void *const *x, int64_t ldx,
                           const void *w, float *y, hipStream_t s);

}  // namespace jf
