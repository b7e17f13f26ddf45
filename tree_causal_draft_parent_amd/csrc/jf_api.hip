// jf_api.hip -- the extern "C" entry points of libjf: argument validation,
// planning and launches on the caller's stream.  Nothing here allocates or
// synchronises.  Every argument error returns before any HIP call, so the
// checks work on a machine without a GPU.
#include <math.h>
#include <string.h>

#include <atomic>

#include "jf_internal.h"

namespace jf {

// Compute units of the current device, cached per device.  Host threads may
// call concurrently: each slot is atomic, and racing first calls store the
// same value.
int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

static inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace jf

using namespace jf;

extern "C" {

const char *jf_status_string(int status) {
    switch (status) {
        case JF_OK: return "JF_OK";
        case JF_ERR_INVALID_ARG: return "JF_ERR_INVALID_ARG";
        case JF_ERR_UNSUPPORTED: return "JF_ERR_UNSUPPORTED";
        case JF_ERR_ALIGN: return "JF_ERR_ALIGN";
        case JF_ERR_WORKSPACE: return "JF_ERR_WORKSPACE";
        case JF_ERR_BAD_TREE: return "JF_ERR_BAD_TREE";
        case JF_ERR_BAD_PAGE: return "JF_ERR_BAD_PAGE";
        case JF_ERR_HIP: return "JF_ERR_HIP";
        case JF_ERR_BAD_PREFIX: return "JF_ERR_BAD_PREFIX";
        default: return "JF_ERR_UNKNOWN";
    }
}

int jf_abi_version(void) { return 6; }

// Packed node offsets: node_off[0] = 0, at least one node a sequence, at
// most N (the largest count, which sets the mask width).
static jf_status check_node_off(const int32_t *node_off, int32_t B, int32_t N) {
    if (!node_off) return JF_OK;
    if (B > kMaxBatch) return JF_ERR_UNSUPPORTED;
    if (node_off[0] != 0) return JF_ERR_INVALID_ARG;
    int32_t nmax = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t n = (int64_t)node_off[b + 1] - node_off[b];
        if (n < 1 || n > N) return JF_ERR_INVALID_ARG;
        if (n > nmax) nmax = (int32_t)n;
    }
    return nmax == N ? JF_OK : JF_ERR_INVALID_ARG;
}

jf_status jf_tree_mask_build(const int32_t *parent, const int32_t *node_off, int32_t B, int32_t N,
                             uint64_t *mask, int32_t *depth, int32_t *seq_status, void *stream) {
    if (!parent || !mask) return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || N > 4096) return JF_ERR_INVALID_ARG;
    jf_status st = check_node_off(node_off, B, N);
    if (st != JF_OK) return st;
    if (!aligned(parent, 4) || !aligned(mask, 8) || (depth && !aligned(depth, 4)) ||
        (seq_status && !aligned(seq_status, 4)))
        return JF_ERR_ALIGN;
    hipError_t e = launch_tree_mask(parent, node_off, B, N, mask, depth, seq_status,
                                    (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

// ---------------------------------------------------------------------------
static jf_status check_fuse(int32_t k, int64_t M, int64_t H_in, int64_t ldx, int64_t H_out,
                            jf_dtype in_dtype) {
    if (k < 1 || k > 8 || M < 1 || H_in < 1 || H_out < 1 || ldx < H_in) return JF_ERR_INVALID_ARG;
    if (in_dtype != JF_BF16 && in_dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (in_dtype == JF_BF16 && H_in % 64 != 0) return JF_ERR_UNSUPPORTED;
    if (M > (int64_t)1 << 30 || H_out > (int64_t)1 << 30) return JF_ERR_UNSUPPORTED;
    return JF_OK;
}

size_t jf_fuse_proj_workspace_size_cus(int64_t M, int64_t H_in, int32_t k, int64_t H_out,
                                       jf_dtype in_dtype, int32_t cus) {
    if (check_fuse(k, M, H_in, H_in, H_out, in_dtype) != JF_OK) return 0;
    FusePlan p;
    plan_fuse(p, M, H_in, k, H_out, in_dtype, cus);
    return fuse_workspace_bytes(p);
}

size_t jf_fuse_proj_workspace_size(int64_t M, int64_t H_in, int32_t k, int64_t H_out,
                                   jf_dtype in_dtype) {
    return jf_fuse_proj_workspace_size_cus(M, H_in, k, H_out, in_dtype, 0);
}

jf_status jf_fuse_proj(const void *const *x, int32_t k, int64_t M, int64_t H_in, int64_t ldx,
                       const void *w, int64_t H_out, jf_dtype in_dtype, void *y,
                       jf_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return jf_fuse_proj_cus(x, k, M, H_in, ldx, w, H_out, in_dtype, y, out_dtype, workspace,
                            workspace_bytes, 0, stream);
}

jf_status jf_fuse_proj_cus(const void *const *x, int32_t k, int64_t M, int64_t H_in, int64_t ldx,
                           const void *w, int64_t H_out, jf_dtype in_dtype, void *y,
                           jf_dtype out_dtype, void *workspace, size_t workspace_bytes, int32_t cus,
                           void *stream) {
    if (!x || !w || !y) return JF_ERR_INVALID_ARG;
    jf_status st = check_fuse(k, M, H_in, ldx, H_out, in_dtype);
    if (st != JF_OK) return st;
    for (int l = 0; l < k; ++l)
        if (!x[l]) return JF_ERR_INVALID_ARG;
    if (out_dtype != JF_F32 && out_dtype != JF_BF16) return JF_ERR_INVALID_ARG;
    if (in_dtype == JF_F32 && out_dtype != JF_F32) return JF_ERR_UNSUPPORTED;
    // bf16 operands are read as 16-byte vectors; the fp32 path reads scalars.
    const size_t a = in_dtype == JF_BF16 ? 16 : 4;
    for (int l = 0; l < k; ++l)
        if (!aligned(x[l], a)) return JF_ERR_ALIGN;
    if (!aligned(w, a) || !aligned(y, in_dtype == JF_BF16 ? (out_dtype == JF_BF16 ? 8 : 16) : 4))
        return JF_ERR_ALIGN;
    if (in_dtype == JF_BF16 && ldx % 8 != 0) return JF_ERR_ALIGN;
    if (in_dtype == JF_BF16) {
        // 32-bit buffer offsets with room for the K position: each operand < 3.75 GiB
        const int64_t lim = 0xf0000000LL;
        if (((M - 1) * ldx + H_in) * 2 > lim || H_out * (int64_t)k * H_in * 2 > lim)
            return JF_ERR_UNSUPPORTED;
    }
    FusePlan p;
    plan_fuse(p, M, H_in, k, H_out, in_dtype, cus);
    const size_t need = fuse_workspace_bytes(p);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return JF_ERR_WORKSPACE;
    hipError_t e = in_dtype == JF_BF16
                       ? launch_fuse_bf16(p, x, ldx, w, y, out_dtype, workspace, (hipStream_t)stream)
                       : launch_fuse_f32(p, x, ldx, w, (float *)y, (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

// ---------------------------------------------------------------------------
static jf_status check_attn_dims(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                 const int32_t *prefix_len, const int32_t *node_off,
                                 jf_dtype dtype) {
    if (!prefix_len) return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || D < 1) return JF_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (B > kMaxBatch || N > 1024) return JF_ERR_UNSUPPORTED;
    if (dtype == JF_BF16 && D != 128 && D != 64) return JF_ERR_UNSUPPORTED;
    if (dtype == JF_F32 && D > 128) return JF_ERR_UNSUPPORTED;
    for (int b = 0; b < B; ++b)
        if (prefix_len[b] < 0) return JF_ERR_INVALID_ARG;
    return check_node_off(node_off, B, N);
}

size_t jf_tree_attn_workspace_size_cus(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t page_size, const int32_t *prefix_len,
                                       const int32_t *node_off, jf_dtype dtype, int32_t cus) {
    if (check_attn_dims(B, N, Hq, Hkv, D, prefix_len, node_off, dtype) != JF_OK || page_size < 1)
        return 0;
    if (dtype == JF_F32) return 0;
    AttnPlan p;
    plan_tree_attn(p, B, N, Hq, Hkv, D, page_size, prefix_len, node_off, dtype, cus);
    return p.fits ? tree_attn_workspace_bytes(p) : 0;
}

size_t jf_tree_attn_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                   int32_t page_size, const int32_t *prefix_len,
                                   const int32_t *node_off, jf_dtype dtype) {
    return jf_tree_attn_workspace_size_cus(B, N, Hq, Hkv, D, page_size, prefix_len, node_off, dtype,
                                           0);
}

jf_status jf_tree_attn_fwd(const void *q, const void *k_tree, const void *v_tree,
                           const uint64_t *mask, const void *k_cache, const void *v_cache,
                           jf_dtype kv_dtype, float k_scale, float v_scale, int64_t num_pages,
                           int32_t page_size, const int32_t *block_table, int32_t max_pages,
                           const int32_t *prefix_len, const int32_t *prefix_len_dev,
                           const int32_t *node_off, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                           int32_t D, float scale, jf_dtype dtype, void *out, float *lse,
                           void *workspace, size_t workspace_bytes, int32_t *status,
                           void *stream) {
    return jf_tree_attn_fwd_cus(q, k_tree, v_tree, mask, k_cache, v_cache, kv_dtype, k_scale,
                                v_scale, num_pages, page_size, block_table, max_pages, prefix_len,
                                prefix_len_dev, node_off, B, N, Hq, Hkv, D, scale, dtype, out, lse,
                                workspace, workspace_bytes, status, 0, stream);
}

jf_status jf_tree_attn_fwd_cus(const void *q, const void *k_tree, const void *v_tree,
                               const uint64_t *mask, const void *k_cache, const void *v_cache,
                               jf_dtype kv_dtype, float k_scale, float v_scale, int64_t num_pages,
                               int32_t page_size, const int32_t *block_table, int32_t max_pages,
                               const int32_t *prefix_len, const int32_t *prefix_len_dev,
                               const int32_t *node_off, int32_t B, int32_t N, int32_t Hq,
                               int32_t Hkv, int32_t D, float scale, jf_dtype dtype, void *out,
                               float *lse, void *workspace, size_t workspace_bytes,
                               int32_t *status, int32_t cus, void *stream) {
    if (!q || !k_tree || !v_tree || !mask || !k_cache || !v_cache || !block_table || !out)
        return JF_ERR_INVALID_ARG;
    jf_status st = check_attn_dims(B, N, Hq, Hkv, D, prefix_len, node_off, dtype);
    if (st != JF_OK) return st;
    if (kv_dtype != JF_F32 && kv_dtype != JF_BF16 && kv_dtype != JF_FP8_E4M3)
        return JF_ERR_INVALID_ARG;
    const bool fp8 = kv_dtype == JF_FP8_E4M3;
    if (kv_dtype != dtype && !(fp8 && dtype == JF_BF16)) return JF_ERR_UNSUPPORTED;
    if (fp8 && !(k_scale > 0.f && v_scale > 0.f && k_scale < INFINITY && v_scale < INFINITY))
        return JF_ERR_INVALID_ARG;
    if (page_size < 1 || max_pages < 1 || num_pages < 0) return JF_ERR_INVALID_ARG;
    for (int b = 0; b < B; ++b)
        if ((int64_t)prefix_len[b] > (int64_t)max_pages * page_size) return JF_ERR_INVALID_ARG;
    const size_t al = 16;
    if (!aligned(q, al) || !aligned(k_tree, al) || !aligned(v_tree, al) || !aligned(k_cache, al) ||
        !aligned(v_cache, al) || !aligned(out, al) || !aligned(mask, 8) || !aligned(block_table, 4) ||
        (lse && !aligned(lse, 4)) || (status && !aligned(status, 4)) ||
        (prefix_len_dev && !aligned(prefix_len_dev, 4)))
        return JF_ERR_ALIGN;
    const int64_t T = node_off ? (int64_t)node_off[B] : (int64_t)B * N;
    if (dtype == JF_BF16) {
        // the bf16 kernel addresses each tensor with 32-bit buffer offsets
        const int64_t lim = 0xffffff00LL;
        if (num_pages * page_size * (int64_t)Hkv * D * (fp8 ? 1 : 2) > lim || T * Hq * D * 2 > lim ||
            T * Hkv * D * 2 > lim)
            return JF_ERR_UNSUPPORTED;
    }
    if (!(scale > 0.f)) scale = 1.f / sqrtf((float)D);
    AttnPlan p;
    plan_tree_attn(p, B, N, Hq, Hkv, D, page_size, prefix_len, node_off, dtype, cus);
    hipError_t e;
    if (dtype == JF_BF16) {
        if (!p.fits) return JF_ERR_UNSUPPORTED;
        const size_t need = tree_attn_workspace_bytes(p);
        if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
            return JF_ERR_WORKSPACE;
        e = launch_tree_attn_bf16(p, q, k_tree, v_tree, mask, k_cache, v_cache, num_pages, page_size,
                                  block_table, max_pages, prefix_len_dev, scale, fp8, k_scale,
                                  v_scale, out, lse, workspace, status, (hipStream_t)stream);
    } else {
        e = launch_tree_attn_f32(p, (const float *)q, (const float *)k_tree, (const float *)v_tree,
                                 mask, (const float *)k_cache, (const float *)v_cache, num_pages,
                                 page_size, block_table, max_pages, prefix_len_dev, scale,
                                 (float *)out, lse, status, (hipStream_t)stream);
    }
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

// ---------------------------------------------------------------------------
size_t jf_node_topk_workspace_size(int64_t R, int64_t V, int32_t k) {
    if (R < 1 || V < 1 || k < 1 || k > 64 || k > V || V > INT32_MAX) return 0;
    // the fp32 plan has the most slices; its workspace also fits the bf16 plan
    TopkPlan p, pb;
    plan_topk(p, R, V, k, JF_F32);
    plan_topk(pb, R, V, k, JF_BF16);
    if (p.chunks == 0 && pb.chunks == 0) return 0;
    size_t a = p.chunks > 0 ? topk_workspace_bytes(p) : 0, b = pb.chunks > 0 ? topk_workspace_bytes(pb) : 0;
    return a > b ? a : b;
}

jf_status jf_node_topk(const void *logits, int64_t R, int64_t V, int64_t ld, jf_dtype dtype,
                       int32_t k, int32_t *idx, float *val, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (!logits || !idx || !val) return JF_ERR_INVALID_ARG;
    if (R < 1 || V < 1 || ld < V || k < 1) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (k > 64 || k > V || V > INT32_MAX) return JF_ERR_UNSUPPORTED;
    if (R > (int64_t)1 << 30) return JF_ERR_UNSUPPORTED;
    if (!aligned(logits, 16) || ld % (dtype == JF_BF16 ? 8 : 4) != 0) return JF_ERR_ALIGN;
    if (!aligned(idx, 4) || !aligned(val, 4) || (lse && !aligned(lse, 4))) return JF_ERR_ALIGN;
    TopkPlan p;
    plan_topk(p, R, V, k, dtype);
    if (p.chunks == 0) return JF_ERR_UNSUPPORTED;   // V too large for k slices to merge
    const size_t need = topk_workspace_bytes(p);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return JF_ERR_WORKSPACE;
    hipError_t e = launch_topk(p, logits, ld, dtype, idx, val, lse, workspace, (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_node_topk_noalloc(const void *logits, int64_t R, int64_t V, int64_t ld,
                               jf_dtype dtype, int32_t k, int32_t *idx, float *val, float *lse,
                               void *stream) {
    if (!logits || !idx || !val) return JF_ERR_INVALID_ARG;
    if (R < 1 || V < 1 || ld < V || k < 1) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (k > 64 || k > V || V > INT32_MAX) return JF_ERR_UNSUPPORTED;
    if (R > (int64_t)1 << 30) return JF_ERR_UNSUPPORTED;
    if (!aligned(logits, 16) || ld % (dtype == JF_BF16 ? 8 : 4) != 0) return JF_ERR_ALIGN;
    if (!aligned(idx, 4) || !aligned(val, 4) || (lse && !aligned(lse, 4))) return JF_ERR_ALIGN;
    TopkPlan p;
    plan_topk(p, R, V, k, dtype);
    if (p.chunks == 0) return JF_ERR_UNSUPPORTED;
    if (topk_workspace_bytes(p) > kTopkScratchBytes) return JF_ERR_WORKSPACE;
    void *scratch_ptr = nullptr;
    if (topk_scratch(&scratch_ptr) != hipSuccess) return JF_ERR_HIP;
    hipError_t e = launch_topk(p, logits, ld, dtype, idx, val, lse, scratch_ptr, (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

// ---------------------------------------------------------------------------
jf_status jf_path_scores(const int32_t *parent, const float *logp, int32_t B, int32_t N,
                         float *score, int32_t *seq_status, void *stream) {
    if (!parent || !logp || !score) return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || N > 4096) return JF_ERR_INVALID_ARG;
    if (!aligned(parent, 4) || !aligned(logp, 4) || !aligned(score, 4) ||
        (seq_status && !aligned(seq_status, 4)))
        return JF_ERR_ALIGN;
    hipError_t e = launch_path_scores(parent, logp, B, N, score, seq_status, (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_swiglu(const void *gu, int64_t M, int64_t I, int64_t ld, jf_dtype dtype, void *y,
                    void *stream) {
    if (!gu || !y) return JF_ERR_INVALID_ARG;
    if (M < 1 || I < 1 || ld < 2 * I) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    const size_t e = dtype == JF_BF16 ? 2 : 4;
    if (!aligned(gu, e) || !aligned(y, e)) return JF_ERR_ALIGN;
    hipError_t err = launch_swiglu(gu, M, I, ld, dtype, y, (hipStream_t)stream);
    return err == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_rmsnorm(const void *x, int64_t rows, int64_t H, int64_t ldx, const void *w, float eps,
                     jf_dtype dtype, void *y, void *stream) {
    if (!x || !y) return JF_ERR_INVALID_ARG;
    if (rows < 1 || H < 1 || ldx < H || !(eps >= 0.f)) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (H > INT32_MAX || rows > ((int64_t)INT32_MAX) * 4) return JF_ERR_UNSUPPORTED;
    if (x == y && ldx != H) return JF_ERR_INVALID_ARG;     // in place needs dense rows
    const size_t e = dtype == JF_BF16 ? 2 : 4;
    if (!aligned(x, e) || !aligned(y, e) || (w && !aligned(w, e))) return JF_ERR_ALIGN;
    hipError_t err = launch_rmsnorm(x, rows, (int)H, ldx, w, eps, dtype, y, (hipStream_t)stream);
    return err == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_tree_rope(void *q, void *k, const int32_t *depth, const int32_t *prefix_len,
                       int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D, double theta,
                       jf_dtype dtype, void *stream) {
    if (!q || !depth || !prefix_len) return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || Hq < 1 || (k && Hkv < 1) || D < 2 || D % 2 != 0) return JF_ERR_INVALID_ARG;
    if (dtype != JF_BF16 && dtype != JF_F32) return JF_ERR_INVALID_ARG;
    if (D > 256) return JF_ERR_UNSUPPORTED;
    if ((int64_t)B * N > INT32_MAX) return JF_ERR_UNSUPPORTED;
    const size_t e = dtype == JF_BF16 ? 2 : 4;
    if (!aligned(q, e) || (k && !aligned(k, e)) || !aligned(depth, 4) || !aligned(prefix_len, 4))
        return JF_ERR_ALIGN;
    if (!(theta > 0.0)) theta = 1e6;
    hipError_t err = launch_tree_rope(q, k, depth, prefix_len, B, N, Hq, Hkv, D, theta, dtype,
                                      (hipStream_t)stream);
    return err == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_tree_accept(const int32_t *parent, const int32_t *token, const int32_t *target_next,
                         const int32_t *root_next, int32_t B, int32_t N, int32_t *accept_len,
                         int32_t *accept_node, int32_t *next_token, int32_t *path,
                         int32_t *seq_status, void *stream) {
    if (!parent || !token || !target_next || !root_next || !accept_len || !accept_node ||
        !next_token)
        return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || N > 4096) return JF_ERR_INVALID_ARG;
    const void *ptrs[] = {parent, token, target_next, root_next, accept_len, accept_node,
                          next_token, path, seq_status};
    for (const void *q : ptrs)
        if (q && !aligned(q, 4)) return JF_ERR_ALIGN;
    hipError_t e = launch_tree_accept(parent, token, target_next, root_next, B, N, accept_len,
                                      accept_node, next_token, path, seq_status,
                                      (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

jf_status jf_tree_expand(const float *score, const int32_t *depth, const int32_t *idx,
                         const float *val, const float *lse, const int32_t *parent,
                         const int32_t *token, int32_t B, int32_t N, int32_t k,
                         int32_t M, int32_t max_depth, int32_t *new_parent, int32_t *new_token,
                         float *new_score, int32_t *new_depth, void *stream) {
    if (!score || !depth || !idx || !val || !lse || !parent || !token || !new_parent ||
        !new_token || !new_score || !new_depth)
        return JF_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || k < 1 || M < 1) return JF_ERR_INVALID_ARG;
    if ((int64_t)N * k > kExpandMaxCands) return JF_ERR_UNSUPPORTED;
    const void *ptrs[] = {score, depth, idx, val, lse, parent, token, new_parent, new_token,
                          new_score, new_depth};
    for (const void *q : ptrs)
        if (!aligned(q, 4)) return JF_ERR_ALIGN;
    hipError_t e = launch_tree_expand(score, depth, idx, val, lse, parent, token, B, N, k, M,
                                      max_depth, new_parent, new_token, new_score, new_depth,
                                      (hipStream_t)stream);
    return e == hipSuccess ? JF_OK : JF_ERR_HIP;
}

}  // extern "C"
