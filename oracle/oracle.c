/*
 * oracle.c -- plain fp64 CPU oracle of the tree-causal draft-head hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark do.  It shares no code,
 * header, table or helper with the HIP kernels.
 *
 * Every function is the textbook definition written out in double precision
 * over inputs that the caller has already widened exactly to double (bf16 and
 * float32 values are exactly representable).  OpenMP only splits independent
 * output rows across threads; no blocking, fusion or reordering of any sum.
 *
 * Sources (the JetFlow/JetSpec pages):
 *   - tree-causal visibility: JetFlow blog page, "What JetFlow Does
 *     Differently": a node sees the original prefix and its ancestors in the
 *     tree, never its siblings or descendants.
 *   - branch-wise factorisation (why per-node distributions are needed): same
 *     section, the path probability as a product of conditionals along the
 *     branch.
 *   - hidden-state fusion from several frozen target layers: abstract (all
 *     pages) and the same blog section; the pages do not give the fusion op.
 *
 * Readings where the pages are silent (listed with reasons in the design
 * notes): a node is its own ancestor; parent -1 means "child of the prefix
 * end"; softmax scale defaults to 1/sqrt(D); query head h reads KV head
 * h / (Hq/Hkv); the fusion is concatenation followed by one bias-free linear
 * map; top-k order is value descending then index ascending, -0 == +0; a path
 * score is the sum of the conditional log-probabilities along the branch, and
 * one expansion step keeps the M best one-token extensions of the tree that
 * are not already in it;
 * verification is greedy (a node is accepted when its token is the target's
 * next token after its parent) and keeps the deepest fully accepted node.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_INVALID 1
#define OR_BAD_TREE 5
#define OR_BAD_PAGE 6

/* ---------------------------------------------------------------------------
 * Ancestor sets.
 *
 * anc(i) = {i} u anc(parent(i)), with parent -1 ending the walk at the prefix.
 * Row i of the mask holds bit j (word j/64, bit j%64) iff j is in anc(i);
 * depth(i) = |anc(i)|.  A row is bad when its walk meets a parent outside
 * [-1, n_b) or does not end within n_b steps (a cycle, including
 * parent(i) == i).
 * Layout: sequence b owns rows node_off[b] .. node_off[b+1]-1 of parent [T],
 * mask [T, W] and depth [T], with n_b = node_off[b+1] - node_off[b] nodes and
 * parents given as indices local to the sequence; W = ceil(N / 64) for the
 * largest count N.  node_off == NULL means n_b = N for every b (rows b*N+i).
 * Returns OR_BAD_TREE and the smallest row of a bad node, or OR_OK.
 * ------------------------------------------------------------------------- */
int oracle_tree_mask(const int32_t *parent, const int64_t *node_off, int64_t B, int64_t N,
                     uint64_t *mask, int32_t *depth, int64_t *first_bad)
{
    int64_t W = (N + 63) / 64;
    int64_t bad = -1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t off = node_off ? node_off[b] : b * N;
        const int64_t n = node_off ? node_off[b + 1] - node_off[b] : N;
        for (int64_t i = 0; i < n; ++i) {
            uint64_t *row = mask + (off + i) * W;
            for (int64_t w = 0; w < W; ++w) row[w] = 0;
            int64_t j = i, steps = 0;
            int ok = 1;
            while (j != -1) {
                if (j < -1 || j >= n || steps >= n) { ok = 0; break; }
                row[j / 64] |= (uint64_t)1 << (j % 64);
                steps += 1;
                j = parent[off + j];
            }
            if (depth) depth[off + i] = ok ? (int32_t)steps : 0;
            if (!ok && bad < 0) bad = off + i;
        }
    }
    if (first_bad) *first_bad = bad;
    return bad < 0 ? OR_OK : OR_BAD_TREE;
}

/* Membership of j in anc(i), by walking the parent chain (no mask involved). */
static int is_ancestor(const int32_t *par, int64_t N, int64_t i, int64_t j)
{
    int64_t k = i, steps = 0;
    while (k != -1 && k >= 0 && k < N && steps <= N) {
        if (k == j) return 1;
        k = par[k];
        steps += 1;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Fused projection: y[m, o] = sum_l sum_c x_l[m, c] * w[o, l*H_in + c].
 * x is [k, M, H_in] (the k fused layers stacked), w is [H_out, k*H_in]
 * (row o holds the weights of output o, the torch Linear layout).
 * ------------------------------------------------------------------------- */
void oracle_fuse_proj(const double *x, int64_t k, int64_t M, int64_t H_in,
                      const double *w, int64_t H_out, double *y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t o = 0; o < H_out; ++o) {
            double acc = 0.0;
            for (int64_t l = 0; l < k; ++l) {
                const double *xr = x + (l * M + m) * H_in;
                const double *wr = w + o * (k * H_in) + l * H_in;
                for (int64_t c = 0; c < H_in; ++c) acc += xr[c] * wr[c];
            }
            y[m * H_out + o] = acc;
        }
    }
}

/* Same, for a list of output rows only (rows[r] = m); y is [n_rows, H_out]. */
void oracle_fuse_proj_rows(const double *x, int64_t k, int64_t M, int64_t H_in,
                           const double *w, int64_t H_out, const int64_t *rows,
                           int64_t n_rows, double *y)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t o = 0; o < H_out; ++o) {
            int64_t m = rows[r];
            double acc = 0.0;
            for (int64_t l = 0; l < k; ++l) {
                const double *xr = x + (l * M + m) * H_in;
                const double *wr = w + o * (k * H_in) + l * H_in;
                for (int64_t c = 0; c < H_in; ++c) acc += xr[c] * wr[c];
            }
            y[r * H_out + o] = acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Tree attention for one query row (b, i, h).
 *
 * Visible keys, in this order: prefix positions p = 0 .. P_b-1 of sequence b
 * (page block_table[b][p / page_size], slot p % page_size), then every tree
 * node j of sequence b with j in anc(i), in increasing j.
 * s_t = scale * <q, k_t>;  M = max s_t;  w_t = exp(s_t - M);  Z = sum w_t;
 * out = sum_t w_t v_t / Z;  lse = M + log Z.
 * A prefix position whose page id is outside [0, num_pages) reads as a zero
 * key with a zero value (score 0, still counted in Z: the library's contract
 * for a bad block-table entry) and the row reports OR_BAD_PAGE.
 * Tree rows: sequence b owns rows node_off[b] .. node_off[b+1]-1 of q
 * [T, Hq, D], k_tree / v_tree [T, Hkv, D] and parent [T] (parents local to
 * the sequence); node_off == NULL means N rows per sequence (b*N + i).
 * ------------------------------------------------------------------------- */
typedef struct {
    const double *q, *k_tree, *v_tree, *k_cache, *v_cache;
    const int32_t *parent, *block_table, *prefix_len;
    const int64_t *node_off;
    int64_t max_pages, B, N, Hq, Hkv, D, page_size, num_pages;
    double scale;
} attn_args;

static const double kZeroRow[1024];

static int attn_row(const attn_args *a, int64_t b, int64_t i, int64_t h,
                    double *out, double *lse_out, double *s_buf,
                    const double **v_buf)
{
    const int64_t D = a->D, Hkv = a->Hkv, G = a->Hq / a->Hkv;
    const int64_t g = h / G;
    const int64_t off = a->node_off ? a->node_off[b] : b * a->N;
    const int64_t n = a->node_off ? a->node_off[b + 1] - a->node_off[b] : a->N;
    const double *qv = a->q + ((off + i) * a->Hq + h) * D;
    const int64_t P = a->prefix_len[b];
    int status = OR_OK;
    int64_t nk = 0;
    for (int64_t p = 0; p < P; ++p) {
        int64_t page = a->block_table[b * a->max_pages + p / a->page_size];
        if (page < 0 || page >= a->num_pages) {
            status = OR_BAD_PAGE;             /* zero key, zero value */
            s_buf[nk] = 0.0;
            v_buf[nk] = kZeroRow;
            nk += 1;
            continue;
        }
        int64_t slot = p % a->page_size;
        const double *kv = a->k_cache + ((page * a->page_size + slot) * Hkv + g) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qv[d] * kv[d];
        s_buf[nk] = a->scale * dot;
        v_buf[nk] = a->v_cache + ((page * a->page_size + slot) * Hkv + g) * D;
        nk += 1;
    }
    const int32_t *par = a->parent + off;
    for (int64_t j = 0; j < n; ++j) {
        if (!is_ancestor(par, n, i, j)) continue;
        const double *kv = a->k_tree + ((off + j) * Hkv + g) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qv[d] * kv[d];
        s_buf[nk] = a->scale * dot;
        v_buf[nk] = a->v_tree + ((off + j) * Hkv + g) * D;
        nk += 1;
    }
    double M = -INFINITY;
    for (int64_t t = 0; t < nk; ++t) if (s_buf[t] > M) M = s_buf[t];
    double Z = 0.0;
    for (int64_t t = 0; t < nk; ++t) { s_buf[t] = exp(s_buf[t] - M); Z += s_buf[t]; }
    /* out[d] = (sum over t, in increasing t, of w_t v_t[d]) / Z; the value
     * rows are walked one at a time (each out[d] still sums in t order) */
    for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
    for (int64_t t = 0; t < nk; ++t) {
        const double w = s_buf[t];
        const double *vt = v_buf[t];
        for (int64_t d = 0; d < D; ++d) out[d] += w * vt[d];
    }
    for (int64_t d = 0; d < D; ++d) out[d] = out[d] / Z;
    if (lse_out) *lse_out = M + log(Z);
    return status;
}

/* All rows (rows == NULL: out is [T, Hq, D], lse [T, Hq]) or a list of flat
 * row ids r = t*Hq + h over the tree rows t (out is [n_rows, D], lse
 * [n_rows]).  Every row is computed; the status is OR_BAD_PAGE when some row
 * met a bad page id. */
int oracle_tree_attn(const double *q, const double *k_tree, const double *v_tree,
                     const int32_t *parent, const double *k_cache,
                     const double *v_cache, const int32_t *block_table,
                     int64_t max_pages, const int32_t *prefix_len,
                     const int64_t *node_off, int64_t B,
                     int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                     int64_t page_size, int64_t num_pages, double scale,
                     const int64_t *rows, int64_t n_rows, double *out,
                     double *lse)
{
    if (B < 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D > 1024 || Hq % Hkv != 0 ||
        page_size <= 0)
        return OR_INVALID;
    attn_args a = {q, k_tree, v_tree, k_cache, v_cache, parent, block_table,
                   prefix_len, node_off, max_pages, B, N, Hq, Hkv, D, page_size, num_pages,
                   scale};
    int64_t Pmax = 0, nmax = 0;
    for (int64_t b = 0; b < B; ++b) {
        if (prefix_len[b] > Pmax) Pmax = prefix_len[b];
        const int64_t n = node_off ? node_off[b + 1] - node_off[b] : N;
        if (n > nmax) nmax = n;
    }
    const int64_t T = node_off ? node_off[B] : B * N;
    const int64_t total = rows ? n_rows : T * Hq;
    int status = OR_OK;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(Pmax + nmax + 1));
        const double **v_buf = (const double **)malloc(sizeof(double *) * (size_t)(Pmax + nmax + 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < total; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            const int64_t h = flat % Hq, t = flat / Hq;
            /* the sequence owning tree row t */
            int64_t b = node_off ? 0 : t / N;
            if (node_off) while (b + 1 < B && node_off[b + 1] <= t) ++b;
            const int64_t i = t - (node_off ? node_off[b] : b * N);
            int st = attn_row(&a, b, i, h, out + r * D, lse ? lse + r : NULL, s_buf, v_buf);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
            }
        }
        free(s_buf);
        free(v_buf);
    }
    return status;
}

/* ---------------------------------------------------------------------------
 * Per-row top-k of the draft logits and the row log-sum-exp.
 *
 * Order: value descending, then index ascending (-0 == +0 as doubles compare;
 * -inf is an ordinary value; NaN is not a supported input).  Pick t is the
 * largest element that comes strictly after pick t-1 in that order.
 * val is the picked value itself; lse = M + log sum exp(x - M), M = row max.
 * ------------------------------------------------------------------------- */
void oracle_topk(const double *logits, int64_t R, int64_t V, int64_t k,
                 int32_t *idx, double *val, double *lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        const double *x = logits + r * V;
        double prev_v = INFINITY;
        int64_t prev_i = -1;
        for (int64_t t = 0; t < k; ++t) {
            int64_t best = -1;
            double bv = 0.0;
            for (int64_t v = 0; v < V; ++v) {
                double xv = x[v];
                int after_prev = (t == 0) || (xv < prev_v) || (xv == prev_v && v > prev_i);
                if (!after_prev) continue;
                if (best < 0 || xv > bv) { best = v; bv = xv; }
            }
            idx[r * k + t] = (int32_t)best;
            val[r * k + t] = bv;
            prev_v = bv;
            prev_i = best;
        }
        if (lse) {
            double M = -INFINITY;
            for (int64_t v = 0; v < V; ++v) if (x[v] > M) M = x[v];
            if (M == -INFINITY) {
                lse[r] = -INFINITY;
            } else {
                double Z = 0.0;
                for (int64_t v = 0; v < V; ++v) Z += exp(x[v] - M);
                lse[r] = M + log(Z);
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Path scores.
 *
 * A branch's draft probability is the product of the conditionals along it
 * (JetFlow blog page, "What JetFlow Does Differently").  With logp(a) the
 * conditional log-probability of node a's own token given its ancestors, the
 * log-probability of the path from the prefix to node i is
 *     score(i) = sum of logp(a) over a in anc(i).
 * Bad rows (as in oracle_tree_mask) get score 0.  Returns OR_BAD_TREE and the
 * smallest flat index of a bad row, or OR_OK.
 * ------------------------------------------------------------------------- */
int oracle_path_scores(const int32_t *parent, const double *logp, int64_t B, int64_t N,
                       double *score, int64_t *first_bad)
{
    int64_t bad = -1;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < N; ++i) {
            double sum = 0.0;
            int64_t j = i, steps = 0;
            int ok = 1;
            while (j != -1) {
                if (j < -1 || j >= N || steps >= N) { ok = 0; break; }
                sum += logp[b * N + j];
                j = parent[b * N + j];
                ++steps;
            }
            score[b * N + i] = ok ? sum : 0.0;
            if (!ok && bad < 0) bad = b * N + i;
        }
    }
    if (first_bad) *first_bad = bad;
    return bad >= 0 ? OR_BAD_TREE : OR_OK;
}

/* ---------------------------------------------------------------------------
 * Budgeted best-first expansion by one level.
 *
 * The candidates of sequence b are the pairs (p, r): node p's r-th best next
 * token idx[p][r] (from the per-node top-k), whose path score is the parent's
 * path score plus the child's conditional log-probability, the log-softmax
 * of p's row at that token:
 *     s(p, r) = score[p] + (val[p][r] - lse[p]).
 * A candidate is eligible when 1 <= depth[p], depth[p] + 1 <= max_depth, and
 * node p does not already have a child carrying token idx[p][r]: the step
 * grows the tree as it stands, and a second child with the same token would
 * be the same branch twice.  The tree's children are read from parent[] and
 * token[] (node j is a child of parent[j] carrying token[j]; parents outside
 * [0, N) name no node and exclude nothing).
 * With a budget of M new nodes, best-first expansion takes the M best
 * eligible candidates in the order (s descending, p ascending, r ascending),
 * written in that order: new parent p, token, s, depth depth[p] + 1.  Slots
 * left over (fewer eligible candidates than M) read parent -2, token -1,
 * score -inf, depth 0.  The scores decide which candidates survive, so they
 * are computed in float32 with the two roundings in the order written (the
 * precision the selection is made in); inputs are float32.  -0 and +0 are the
 * same score (ties go by p, r) and a zero score is written as +0.
 * ------------------------------------------------------------------------- */
typedef struct { float s; int32_t p, r; } cand_t;

static int cand_cmp(const void *x, const void *y)
{
    const cand_t *a = (const cand_t *)x, *b = (const cand_t *)y;
    if (a->s != b->s) return a->s > b->s ? -1 : 1;
    if (a->p != b->p) return a->p < b->p ? -1 : 1;
    return a->r < b->r ? -1 : (a->r > b->r);
}

/* Does node p of sequence b already have a child carrying token t? */
static int has_child_with_token(const int32_t *parent, const int32_t *token, int64_t b,
                                int64_t N, int64_t p, int32_t t)
{
    for (int64_t j = 0; j < N; ++j)
        if (parent[b * N + j] == p && token[b * N + j] == t) return 1;
    return 0;
}

int oracle_tree_expand(const float *score, const int32_t *depth, const int32_t *idx,
                       const float *val, const float *lse, const int32_t *parent,
                       const int32_t *token, int64_t B, int64_t N, int64_t k,
                       int64_t M, int64_t max_depth, int32_t *new_parent, int32_t *new_token,
                       float *new_score, int32_t *new_depth)
{
    if (B < 1 || N < 1 || k < 1 || M < 1) return OR_INVALID;
    cand_t *c = (cand_t *)malloc((size_t)(N * k) * sizeof(cand_t));
    if (!c) return OR_INVALID;
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = 0;
        for (int64_t p = 0; p < N; ++p) {
            const int32_t d = depth[b * N + p];
            if (d < 1 || (int64_t)d + 1 > max_depth) continue;
            for (int64_t r = 0; r < k; ++r) {
                const int64_t e = (b * N + p) * k + r;
                if (has_child_with_token(parent, token, b, N, p, idx[e])) continue;
                volatile float t = val[e] - lse[b * N + p];     /* rounded to float */
                volatile float sc = score[b * N + p] + t;        /* rounded to float */
                c[n].s = sc;
                c[n].p = (int32_t)p;
                c[n].r = (int32_t)r;
                ++n;
            }
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        for (int64_t m = 0; m < M; ++m) {
            const int64_t o = b * M + m;
            if (m < n) {
                const int64_t e = (b * N + c[m].p) * k + c[m].r;
                new_parent[o] = c[m].p;
                new_token[o] = idx[e];
                new_score[o] = c[m].s == 0.0f ? 0.0f : c[m].s;   /* -0 written as +0 */
                new_depth[o] = depth[b * N + c[m].p] + 1;
            } else {
                new_parent[o] = -2;
                new_token[o] = -1;
                new_score[o] = -INFINITY;
                new_depth[o] = 0;
            }
        }
    }
    free(c);
    return OR_OK;
}

/* ---------------------------------------------------------------------------
 * Gated MLP activation.
 *
 * The Qwen3 models the pages draft for (abstract) gate their MLP with SiLU:
 *     y[m][c] = silu(gu[m][c]) * gu[m][I + c],  silu(g) = g / (1 + exp(-g)),
 * where gu [M, 2I] holds the gate projection in its first I columns and the
 * up projection in its last I (one projection with the two weights stacked).
 * ------------------------------------------------------------------------- */
void oracle_swiglu(const double *gu, int64_t M, int64_t I, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t c = 0; c < I; ++c) {
            const double g = gu[m * 2 * I + c], u = gu[m * 2 * I + I + c];
            y[m * I + c] = g / (1.0 + exp(-g)) * u;
        }
}

/* ---------------------------------------------------------------------------
 * Root-mean-square normalisation of rows.
 *
 * The Qwen3 models the pages draft for (abstract) normalise hidden states,
 * and per head their queries and keys, by the root mean square:
 *     y[r][c] = x[r][c] / sqrt(mean_c(x[r][c]^2) + eps) * w[c]
 * (w = 1 when absent).  x and y [rows, H] (x rows ld apart).
 * ------------------------------------------------------------------------- */
void oracle_rmsnorm(const double *x, int64_t rows, int64_t H, int64_t ld, const double *w,
                    double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * ld;
        double ss = 0.0;
        for (int64_t c = 0; c < H; ++c) ss += xr[c] * xr[c];
        const double inv = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t c = 0; c < H; ++c) y[r * H + c] = xr[c] * inv * (w ? w[c] : 1.0);
    }
}

/* ---------------------------------------------------------------------------
 * Rotary position embedding of the tree nodes' queries and keys.
 *
 * The pages draft with Qwen3 target models (abstract), which rotate queries
 * and keys by their positions (rotary embedding, RoFormer).  A tree node's
 * position is the prefix length plus its depth minus one: a node hanging off
 * the prefix end sits right after the last prefix token, and every node of
 * a branch sits one step after its parent, as in ordinary decoding of that
 * branch.  Pairing as in the Qwen3 models (component d with d + D/2):
 *     a = pos * theta^(-2j/D),  j < D/2
 *     out[j]       = x[j] cos a - x[j + D/2] sin a
 *     out[j + D/2] = x[j + D/2] cos a + x[j] sin a
 * Nodes of depth < 1 (bad rows of the mask builder) are left unchanged.
 * x [B, N, H, D] in place; depth [B, N]; prefix_len [B].
 * ------------------------------------------------------------------------- */
void oracle_tree_rope(double *x, const int32_t *depth, const int32_t *prefix_len, int64_t B,
                      int64_t N, int64_t H, int64_t D, double theta)
{
    const int64_t half = D / 2;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < N; ++i) {
            const int32_t d = depth[b * N + i];
            if (d < 1) continue;
            const double pos = (double)prefix_len[b] + (double)d - 1.0;
            for (int64_t h = 0; h < H; ++h) {
                double *row = x + ((b * N + i) * H + h) * D;
                for (int64_t j = 0; j < half; ++j) {
                    const double a = pos * pow(theta, -2.0 * (double)j / (double)D);
                    const double c = cos(a), sn = sin(a);
                    const double x0 = row[j], x1 = row[j + half];
                    row[j] = x0 * c - x1 * sn;
                    row[j + half] = x1 * c + x0 * sn;
                }
            }
        }
}

/* ---------------------------------------------------------------------------
 * Greedy verification of a drafted tree: the longest accepted path.
 *
 * The target checks the whole tree in one parallel pass and accepts a prefix
 * of the proposal, so a larger budget pays off only through a longer
 * accepted prefix (JetFlow blog page, "The Causality-Efficiency Dilemma" and
 * its introduction).  Reading taken (greedy verification; the pages do not
 * spell out the rule): with pred(-1) = root_next[b], the target's next token
 * after the prefix, and pred(j) = target_next[b][j], its next token after
 * node j, node i is accepted when token[i] == pred(parent(i)) and every
 * ancestor of i is accepted.  The answer is the deepest accepted node (depth
 * = |anc(i)|; ties to the lower index), its depth as the accepted length, the
 * nodes of its path from the prefix down to it, and the target's token after
 * it (after the prefix when nothing is accepted).  A sequence whose parent
 * array is not a forest (as in oracle_tree_mask) reports its smallest bad
 * node and accepts nothing.
 *
 *   accept_len [B], accept_node [B] (-1: none), next_token [B],
 *   path [B, N] (the first accept_len entries, the rest -1),
 *   bad_node [B] (-1 for a forest).
 * ------------------------------------------------------------------------- */
int oracle_tree_accept(const int32_t *parent, const int32_t *token, const int32_t *target_next,
                       const int32_t *root_next, int64_t B, int64_t N, int32_t *accept_len,
                       int32_t *accept_node, int32_t *next_token, int32_t *path,
                       int32_t *bad_node)
{
    if (B < 1 || N < 1) return OR_INVALID;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t *par = parent + b * N;
        const int32_t *tok = token + b * N;
        const int32_t *nxt = target_next + b * N;
        int64_t bad = -1, best = -1, best_depth = 0;
        for (int64_t i = 0; i < N && bad < 0; ++i) {
            /* walk i -> prefix: every node on the way must be accepted */
            int64_t j = i, steps = 0;
            int ok = 1;
            while (j != -1) {
                if (j < -1 || j >= N || steps >= N) { bad = i; break; }
                const int64_t pj = par[j];
                const int32_t pred = pj == -1 ? root_next[b]
                                   : (pj >= 0 && pj < N ? nxt[pj] : -1);
                if (tok[j] != pred) ok = 0;
                j = pj;
                ++steps;
            }
            if (bad >= 0) break;
            if (ok && steps > best_depth) { best = i; best_depth = steps; }
        }
        for (int64_t i = 0; i < N; ++i) path[b * N + i] = -1;
        bad_node[b] = (int32_t)bad;
        if (bad >= 0) { best = -1; best_depth = 0; }
        accept_node[b] = (int32_t)best;
        accept_len[b] = (int32_t)best_depth;
        next_token[b] = best >= 0 ? nxt[best] : root_next[b];
        for (int64_t j = best, d = best_depth - 1; j != -1 && d >= 0; j = par[j], --d)
            path[b * N + d] = (int32_t)j;
    }
    return OR_OK;
}

/* Threads an OpenMP region of this library uses (for reporting). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of later OpenMP regions (n >= 1); used to time the
   oracle on one core beside the all-core figure. */
void oracle_set_num_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }
