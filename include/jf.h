/*
 * jf.h -- C ABI of the MI355X (gfx950) tree-causal draft-head hot path.
 *
 * One forward pass of a causal parallel draft head scores every node of a
 * candidate token tree at once.  Each node attends to the shared prefix and to
 * its own ancestors in the tree, never to siblings or descendants (JetFlow
 * blog page, "What JetFlow Does Differently"), over hidden states fused from
 * several frozen target-model layers (abstract, on every page).  The per-node
 * draft distributions multiply along a branch into that branch's probability
 * (same section), so every node needs its own top candidates and its
 * normaliser.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is DEVICE memory owned by the caller, unless the
 *     argument says "host".  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and is asynchronous.
 *   - Tensors are dense row-major in the stated shape, 16-byte aligned.
 *   - Argument errors are returned synchronously and launch nothing.  Data
 *     errors that only the device can see (a parent array that is not a
 *     forest, a page id out of range) are written to caller-provided device
 *     words, described per call.
 *   - Calls are re-entrant: there is no mutable global state beyond a cached
 *     device-property query.  Concurrent calls need distinct workspaces.
 *   - bf16 is IEEE binary32 truncated to its upper 16 bits (round to nearest
 *     even on conversion); accumulation is always fp32.
 */
#ifndef JF_H
#define JF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JF_OK = 0,
    JF_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, inconsistent dims */
    JF_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head dim, dtype mix, k) */
    JF_ERR_ALIGN = 3,        /* pointer or leading dimension not 16-byte aligned */
    JF_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the size query */
    JF_ERR_BAD_TREE = 5,     /* device-side only: parent array is not a forest */
    JF_ERR_BAD_PAGE = 6,     /* device-side only: block-table entry out of range */
    JF_ERR_HIP = 7,          /* the HIP runtime refused a launch */
    JF_ERR_BAD_PREFIX = 8    /* device-side only: a device prefix length outside [0, bound] */
} jf_status;

/* JF_FP8_E4M3: OCP FP8 E4M3 ("fn": no infinities, max 448), one byte per
 * element, for prefix K/V caches only (with a per-tensor scale). */
typedef enum { JF_F32 = 0, JF_BF16 = 1, JF_FP8_E4M3 = 2 } jf_dtype;

/* Human-readable name of a status code (static storage). */
const char *jf_status_string(int status);

/* ABI version, bumped on any signature change. */
int jf_abi_version(void);  /* 6 */

/* --------------------------------------------------------------------------
 * jf_tree_mask_build -- ancestor bitmask of every tree node.
 *
 * Realises the visibility rule (a node sees the prefix and its ancestors;
 * JetFlow blog page, "What JetFlow Does Differently") as data: node i's row
 * has bit j set iff j is an ancestor of i, the node itself included.
 * parent[i] is the index of node i's parent within its sequence, or -1 when
 * node i hangs directly off the prefix end (several such roots are allowed).
 * Node ids need not be in creation order.
 *
 * Tree layout (shared with jf_tree_attn_fwd):
 *   node_off == NULL: every sequence has N nodes; sequence b owns rows
 *              b*N .. b*N+N-1 of parent, mask and depth.
 *   node_off   HOST [B+1] int32 (packed trees of different sizes, as a
 *              serving batch carries): sequence b owns rows node_off[b] ..
 *              node_off[b+1]-1, with n_b = node_off[b+1] - node_off[b] >= 1
 *              nodes and parents local to the sequence; node_off[0] = 0,
 *              N = the largest n_b, B <= 256.
 *
 *   parent     [T] int32, T = B*N or node_off[B].
 *   mask       [T, W] uint64, W = ceil(N / 64): bit (j % 64) of word j / 64
 *              of a node's row <=> j in anc(node).  Bits for j >= n_b are zero.
 *   depth      [T] int32, |anc(i)| (1 for a prefix child), or NULL.
 *   seq_status [B] int32 or NULL: -1 when sequence b is a forest, otherwise
 *              the smallest local index i whose walk to the prefix meets a
 *              parent outside [-1, n_b) or does not end within n_b steps (a
 *              cycle).  Rows of such nodes are zero and their depth is 0.
 *              Written on every call.
 *   B >= 1, 1 <= N <= 4096.
 * ------------------------------------------------------------------------ */
jf_status jf_tree_mask_build(const int32_t *parent, const int32_t *node_off,
                             int32_t B, int32_t N, uint64_t *mask,
                             int32_t *depth, int32_t *seq_status, void *stream);

/* --------------------------------------------------------------------------
 * jf_fuse_proj -- projection of hidden states fused from several layers.
 *
 * The pages train the draft head "over fused hidden states" of the frozen
 * target (abstract; JetFlow blog page, "What JetFlow Does Differently") but
 * do not give the fusion operator.  Reading taken here: concatenate the k
 * layers' states and apply one bias-free linear map,
 *     y[m, o] = sum_l sum_c x_l[m, c] * w[o, l*H_in + c].
 *
 *   x        HOST array of k DEVICE pointers; x[l] is [M, H_in] with row
 *            stride ldx elements (ldx >= H_in).
 *   w        [H_out, k*H_in] (row o = weights of output o; torch Linear).
 *   y        [M, H_out] of out_dtype.
 *   in_dtype JF_BF16 (MFMA, fp32 accumulation) or JF_F32 (fp32 FMA).
 *   out_dtype JF_F32 or JF_BF16 (bf16 inputs) / JF_F32 (fp32 inputs).
 *   1 <= k <= 8; H_in % 64 == 0 for bf16; ldx % 8 == 0 for bf16.
 *   Alignment: bf16 x and w 16 bytes, y 16 (fp32 out) or 8 (bf16 out);
 *   fp32 inputs need only 4-byte alignment.  bf16: each x[l] and w must
 *   span less than 3.75 GiB (32-bit buffer offsets), else JF_ERR_UNSUPPORTED.
 *   workspace: jf_fuse_proj_workspace_size() bytes (may be 0 -> NULL ok).
 * ------------------------------------------------------------------------ */
size_t jf_fuse_proj_workspace_size(int64_t M, int64_t H_in, int32_t k,
                                   int64_t H_out, jf_dtype in_dtype);
jf_status jf_fuse_proj(const void *const *x, int32_t k, int64_t M,
                       int64_t H_in, int64_t ldx, const void *w, int64_t H_out,
                       jf_dtype in_dtype, void *y, jf_dtype out_dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------------------------------
 * jf_fuse_proj_cus / jf_fuse_proj_workspace_size_cus -- the same projection
 * (same citation and arguments as above), with the K split planned for `cus`
 * compute units instead of all of the device's (cus <= 0 or above the
 * device's count: all).  For a caller that runs other work beside the
 * projection on another stream: fewer K slices leave compute units to that
 * work and write fewer fp32 partials.  The workspace size must come from
 * jf_fuse_proj_workspace_size_cus with the same cus.  Results agree with
 * jf_fuse_proj to the rounding of the fp32 slice sums.
 * ------------------------------------------------------------------------ */
size_t jf_fuse_proj_workspace_size_cus(int64_t M, int64_t H_in, int32_t k,
                                       int64_t H_out, jf_dtype in_dtype,
                                       int32_t cus);
jf_status jf_fuse_proj_cus(const void *const *x, int32_t k, int64_t M,
                           int64_t H_in, int64_t ldx, const void *w,
                           int64_t H_out, jf_dtype in_dtype, void *y,
                           jf_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, int32_t cus, void *stream);

/* --------------------------------------------------------------------------
 * jf_tree_attn_fwd -- tree-causal attention of all draft nodes in one pass.
 *
 * For sequence b, tree node i and query head h (KV head g = h / (Hq/Hkv)):
 * keys are the P_b prefix positions followed by the tree nodes j with
 * j in anc(i) (JetFlow blog page, "What JetFlow Does Differently";
 * "block-level causal attention", arxivlens methodology and the arXiv page's
 * section 1).  s_t = scale * <q, k_t>,
 *     out = sum_t softmax(s)_t v_t,   lse = log sum_t exp(s_t).
 * Trees are laid out as for jf_tree_mask_build (N nodes a sequence, or
 * packed with node_off); T = B*N or node_off[B] tree rows.
 *
 *   q           [T, Hq, D]          dtype
 *   k_tree/v_tree [T, Hkv, D]       dtype (the tree nodes' own keys/values)
 *   mask        [T, ceil(N/64)]     from jf_tree_mask_build
 *   k_cache/v_cache [num_pages, page_size, Hkv, D] kv_dtype: prefix pages.
 *   kv_dtype    dtype, or JF_FP8_E4M3 with dtype JF_BF16: the cache holds
 *               E4M3 codes and a key's (value's) element is its decoded code
 *               times k_scale (v_scale); the scales are ignored otherwise.
 *   block_table [B, max_pages] int32 (device): page of prefix position p of
 *               sequence b is block_table[b][p / page_size], slot
 *               p % page_size.  A contiguous prefix is one page per sequence
 *               (page_size >= max P_b, block_table[b][0] = b).
 *   prefix_len  HOST [B] int32 >= 0: the prefix lengths, or, when
 *               prefix_len_dev is given, their upper bounds.  The key splits
 *               and the launch are planned from these host values.
 *   prefix_len_dev DEVICE [B] int32 or NULL: the prefix lengths, read by the
 *               kernels; each must lie in [0, prefix_len[b]] (one captured
 *               launch then serves any lengths up to the bounds).  A value
 *               outside is clamped into the range and status is set.
 *   node_off    HOST [B+1] int32 or NULL: packed trees (jf_tree_mask_build).
 *   scale       softmax scale; <= 0 selects 1/sqrt(D).
 *   out         [T, Hq, D] dtype;  lse [T, Hq] fp32 or NULL.
 *   status      one device int32 or NULL, never cleared by the library (zero
 *               it once beforehand): set to JF_ERR_BAD_PAGE when a needed
 *               block-table entry is outside [0, num_pages) (that prefix
 *               position then reads as a zero key with a zero value: score 0,
 *               counted in the normaliser), or to JF_ERR_BAD_PREFIX for a
 *               device prefix length outside its bound.
 *   dtype       JF_BF16: D == 128 or 64, MFMA path over row pieces with fp32
 *               partials (D = 64 is computed at 128 with the upper half of
 *               q, k and v read as zeros);  JF_F32: D <= 128, plain fp32 path
 *               (small problems).
 *   Limits: 1 <= B <= 256, 1 <= N <= 1024, Hq % Hkv == 0; on the bf16
 *   path each of q, k_tree, k_cache (and their value twins) must be smaller
 *   than 4 GiB - 256 bytes (32-bit buffer offsets), else JF_ERR_UNSUPPORTED;
 *   so is a plan of more than 2^30 work items (prefix bounds of billions of
 *   tokens).
 *   workspace:  jf_tree_attn_workspace_size() bytes with the same arguments.
 * ------------------------------------------------------------------------ */
size_t jf_tree_attn_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t page_size,
                                   const int32_t *prefix_len,
                                   const int32_t *node_off, jf_dtype dtype);
jf_status jf_tree_attn_fwd(const void *q, const void *k_tree,
                           const void *v_tree, const uint64_t *mask,
                           const void *k_cache, const void *v_cache,
                           jf_dtype kv_dtype, float k_scale, float v_scale,
                           int64_t num_pages, int32_t page_size,
                           const int32_t *block_table, int32_t max_pages,
                           const int32_t *prefix_len,
                           const int32_t *prefix_len_dev,
                           const int32_t *node_off, int32_t B, int32_t N,
                           int32_t Hq, int32_t Hkv, int32_t D, float scale,
                           jf_dtype dtype, void *out, float *lse,
                           void *workspace, size_t workspace_bytes,
                           int32_t *status, void *stream);

/* --------------------------------------------------------------------------
 * jf_tree_attn_fwd_cus / jf_tree_attn_workspace_size_cus -- the same
 * computation (same citation and arguments as above), with the key splits
 * planned for `cus` compute units instead of all of the device's (cus <= 0
 * or above the device's count: all).  For a caller that runs other work
 * beside the attention on another stream: fewer, longer splits leave compute
 * units to that work and write fewer partial results.  The workspace size
 * must come from jf_tree_attn_workspace_size_cus with the same cus.  Results
 * agree with jf_tree_attn_fwd to the rounding of the split combination.
 * ------------------------------------------------------------------------ */
size_t jf_tree_attn_workspace_size_cus(int32_t B, int32_t N, int32_t Hq,
                                       int32_t Hkv, int32_t D, int32_t page_size,
                                       const int32_t *prefix_len,
                                       const int32_t *node_off, jf_dtype dtype,
                                       int32_t cus);
jf_status jf_tree_attn_fwd_cus(const void *q, const void *k_tree,
                               const void *v_tree, const uint64_t *mask,
                               const void *k_cache, const void *v_cache,
                               jf_dtype kv_dtype, float k_scale, float v_scale,
                               int64_t num_pages, int32_t page_size,
                               const int32_t *block_table, int32_t max_pages,
                               const int32_t *prefix_len,
                               const int32_t *prefix_len_dev,
                               const int32_t *node_off, int32_t B, int32_t N,
                               int32_t Hq, int32_t Hkv, int32_t D, float scale,
                               jf_dtype dtype, void *out, float *lse,
                               void *workspace, size_t workspace_bytes,
                               int32_t *status, int32_t cus, void *stream);

/* --------------------------------------------------------------------------
 * jf_node_topk -- the k best candidates of every node's draft distribution.
 *
 * A tree grows by expanding nodes with their most likely next tokens, and a
 * branch's probability is the product of its per-node conditionals (JetFlow
 * blog page, "What JetFlow Does Differently"), so each row needs its top-k
 * logits and its log-normaliser.
 *
 *   logits [R, V] dtype with row stride ld (elements; ld >= V, ld % 8 == 0
 *          for bf16, % 4 == 0 for fp32).  NaN is not a supported value.
 *   idx    [R, k] int32: indices ordered by value descending, ties by the
 *          lower index; -0 and +0 are equal.
 *   val    [R, k] fp32: the selected values.
 *   lse    [R] fp32 or NULL: log sum_v exp(logits[r, v]).
 *   1 <= k <= 64, k <= V, and ceil(V / S) * k <= 4096 with S = 9728 (bf16)
 *   or 4864 (fp32): V up to 311296 at k = 64 for fp32, about 4.9 million at
 *   k = 8 for bf16; else JF_ERR_UNSUPPORTED.
 *   workspace: jf_node_topk_workspace_size() bytes.
 * ------------------------------------------------------------------------ */
size_t jf_node_topk_workspace_size(int64_t R, int64_t V, int32_t k);
jf_status jf_node_topk(const void *logits, int64_t R, int64_t V, int64_t ld,
                       jf_dtype dtype, int32_t k, int32_t *idx, float *val,
                       float *lse, void *workspace, size_t workspace_bytes,
                       void *stream);

/* --------------------------------------------------------------------------
 * jf_node_topk_noalloc -- jf_node_topk (same arguments and results) for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace and
 * allocates nothing: its scratch is a static device array of
 * JF_NODE_TOPK_SCRATCH_BYTES per GPU, held by each GPU the library runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there).  A size whose jf_node_topk_workspace_size(R, V, k)
 * exceeds that limit returns JF_ERR_WORKSPACE and launches nothing.  All
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (different streams, or one stream of another process sharing the library
 * instance) race and must not be issued.  The array keeps the last call's
 * contents; no part of it has to start at zero.
 * ------------------------------------------------------------------------ */
#define JF_NODE_TOPK_SCRATCH_BYTES ((size_t)4 << 20)
jf_status jf_node_topk_noalloc(const void *logits, int64_t R, int64_t V,
                               int64_t ld, jf_dtype dtype, int32_t k,
                               int32_t *idx, float *val, float *lse,
                               void *stream);

/* --------------------------------------------------------------------------
 * jf_path_scores -- path log-probability of every draft-tree node.
 *
 * A branch's draft probability is the product of the conditionals of the
 * nodes along it (JetFlow blog page, "What JetFlow Does Differently"), so
 * with logp[i] the conditional log-probability of node i's own token given
 * its ancestors,
 *     score[i] = sum of logp[a] over a in anc(i)   (i itself included).
 * The sum runs from the node up to the prefix in fp64 and is rounded once to
 * fp32, so the result does not depend on the launch shape.
 *
 *   parent     [B, N] int32, as for jf_tree_mask_build.
 *   logp       [B, N] fp32.
 *   score      [B, N] fp32 out; 0 for nodes of a bad walk.
 *   seq_status [B] int32 or NULL: as for jf_tree_mask_build.
 *   B >= 1, 1 <= N <= 4096.
 * ------------------------------------------------------------------------ */
jf_status jf_path_scores(const int32_t *parent, const float *logp, int32_t B,
                         int32_t N, float *score, int32_t *seq_status,
                         void *stream);

/* --------------------------------------------------------------------------
 * jf_tree_expand -- one budgeted best-first expansion step of the tree.
 *
 * The tree grows with each node's most likely next tokens, ranked by the
 * product of conditionals along the branch (JetFlow blog page, "What JetFlow
 * Does Differently"), under a node budget (the 16- and 256-token draft
 * budgets of the "Empirical Results" section).  The pages do not print the
 * expansion rule (their Algorithm 1 is absent); reading taken: per sequence
 * the candidates are the pairs (p, r), node p's r-th top token, with score
 *     s(p, r) = score[p] + (val[p][r] - lse[p])
 * (two fp32 roundings, in that order), eligible when
 * 1 <= depth[p] < max_depth and node p has no child carrying idx[p][r] yet
 * (the step grows the tree as it stands; a second child with the same token
 * would be the same branch twice).  The M best eligible candidates in the
 * order (s descending, p ascending, r ascending) become the new nodes,
 * written in that order: new_parent = p, new_token = idx[p][r], new_score = s
 * (a zero written as +0; -0 and +0 tie), new_depth = depth[p] + 1.  Slots
 * beyond the eligible count read parent -2, token -1, score -inf, depth 0.
 *
 *   score  [B, N] fp32 path scores of the current nodes (jf_path_scores).
 *   depth  [B, N] int32 (jf_tree_mask_build).
 *   idx    [B, N, k] int32, val [B, N, k] fp32, lse [B, N] fp32: the
 *          per-node top-k lists and log-normalisers (jf_node_topk); a
 *          node's listed tokens are distinct (as jf_node_topk returns them).
 *   parent [B, N] int32, token [B, N] int32: the tree being grown; node j
 *          is a child of parent[j] (-1: of the prefix) carrying token[j].
 *          A parent outside [0, N) excludes nothing.
 *   new_parent, new_token, new_depth [B, M] int32; new_score [B, M] fp32.
 *   B >= 1, N >= 1, 1 <= k, N * k <= 16384, M >= 1; NaN scores, values or
 *   normalisers are not supported.
 * ------------------------------------------------------------------------ */
jf_status jf_tree_expand(const float *score, const int32_t *depth,
                         const int32_t *idx, const float *val, const float *lse,
                         const int32_t *parent, const int32_t *token,
                         int32_t B, int32_t N, int32_t k, int32_t M,
                         int32_t max_depth, int32_t *new_parent,
                         int32_t *new_token, float *new_score,
                         int32_t *new_depth, void *stream);

/* --------------------------------------------------------------------------
 * jf_swiglu -- gated MLP activation.
 *
 * The Qwen3 models the pages draft for (abstract) gate their MLP with SiLU:
 *     y[m][c] = silu(gu[m][c]) * gu[m][I + c],  silu(g) = g / (1 + exp(-g)),
 * the gate projection in the first I columns of gu, the up projection in
 * the last I (e.g. one jf_fuse_proj call with the two weights stacked).
 * fp32 arithmetic; bf16 storage rounds to nearest even.
 *
 *   gu  [M, 2I] dtype with row stride ld elements (ld >= 2I).
 *   y   [M, I] dtype, dense; must not overlap gu.
 * ------------------------------------------------------------------------ */
jf_status jf_swiglu(const void *gu, int64_t M, int64_t I, int64_t ld,
                    jf_dtype dtype, void *y, void *stream);

/* --------------------------------------------------------------------------
 * jf_rmsnorm -- root-mean-square normalisation of rows.
 *
 * The Qwen3 models the pages draft for (abstract) normalise a layer's hidden
 * state, and per head its queries and keys, by the root mean square:
 *     y[r][c] = x[r][c] / sqrt(mean_c(x[r][c]^2) + eps) * w[c].
 * The sum of squares is accumulated in fp64, the inverse root rounded once
 * to fp32, the products formed in fp32 (bf16 storage rounds to nearest even).
 *
 *   x    [rows, H] dtype, row stride ldx elements (ldx >= H).
 *   w    [H] dtype or NULL (no weight).
 *   eps  >= 0, added to the mean square inside the root.
 *   y    [rows, H] dtype, dense; may be x itself when ldx == H (in place).
 *   Per-head normalisation of q [B, N, Hq, D] is rows = B*N*Hq, H = D.
 * ------------------------------------------------------------------------ */
jf_status jf_rmsnorm(const void *x, int64_t rows, int64_t H, int64_t ldx,
                     const void *w, float eps, jf_dtype dtype, void *y,
                     void *stream);

/* --------------------------------------------------------------------------
 * jf_tree_rope -- rotary position embedding of the tree nodes, in place.
 *
 * The pages draft for Qwen3 target models (abstract), which rotate queries
 * and keys by position (rotary embedding, RoFormer).  A node's position is
 * prefix_len[b] + depth[b][i] - 1, the position of ordinary decoding along
 * its branch (a prefix child sits right after the last prefix token).
 * Pairs (j, j + D/2) as in the Qwen3 models:
 *     a = pos * theta^(-2j/D),  x[j] <- x[j] cos a - x[j+D/2] sin a,
 *                               x[j+D/2] <- x[j+D/2] cos a + x[j] sin a.
 * Angles are formed in fp64, the rotation in fp32 (bf16 storage rounds to
 * nearest even).  Nodes of depth < 1 are left unchanged.
 *
 *   q          [B, N, Hq, D] dtype, rotated in place.
 *   k          [B, N, Hkv, D] dtype or NULL, rotated in place.
 *   depth      [B, N] int32 (jf_tree_mask_build).
 *   prefix_len [B] int32, DEVICE memory.
 *   theta      rotary base; <= 0 selects 1e6 (the Qwen3 models' base).
 *   D even, 2 <= D <= 256.
 * ------------------------------------------------------------------------ */
jf_status jf_tree_rope(void *q, void *k, const int32_t *depth,
                       const int32_t *prefix_len, int32_t B, int32_t N,
                       int32_t Hq, int32_t Hkv, int32_t D, double theta,
                       jf_dtype dtype, void *stream);

/* --------------------------------------------------------------------------
 * jf_tree_accept -- greedy verification: the longest accepted path.
 *
 * The target model checks the whole drafted tree in one parallel pass and
 * accepts a prefix of the proposal; a larger budget pays off only through a
 * longer accepted prefix (JetFlow blog page, introduction and "The
 * Causality-Efficiency Dilemma").  The pages do not spell out the rule;
 * reading taken (greedy verification): node i is accepted when
 * token[i] == target_next[parent(i)] (root_next for parent -1) and all its
 * ancestors are accepted.  The deepest accepted node wins (ties to the
 * lower index).  The target's next tokens come from its logits, e.g. from
 * jf_node_topk with k = 1 over the verification pass's rows.
 *
 *   parent      [B, N] int32, as for jf_tree_mask_build.
 *   token       [B, N] int32: each node's drafted token.
 *   target_next [B, N] int32: the target's next token after each node.
 *   root_next   [B] int32: the target's next token after the prefix.
 *   accept_len  [B] int32: depth of the deepest accepted node (0: none).
 *   accept_node [B] int32: that node, or -1.
 *   next_token  [B] int32: target_next[accept_node], or root_next[b] when
 *               nothing is accepted.
 *   path        [B, N] int32 or NULL: the accepted nodes from the prefix
 *               down (the first accept_len entries), then -1.
 *   seq_status  [B] int32 or NULL: as for jf_tree_mask_build; a sequence
 *               that is not a forest accepts nothing.
 *   B >= 1, 1 <= N <= 4096.
 * ------------------------------------------------------------------------ */
jf_status jf_tree_accept(const int32_t *parent, const int32_t *token,
                         const int32_t *target_next, const int32_t *root_next,
                         int32_t B, int32_t N, int32_t *accept_len,
                         int32_t *accept_node, int32_t *next_token,
                         int32_t *path, int32_t *seq_status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* JF_H */
