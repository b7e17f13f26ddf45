"""fp64 CPU oracle of the tree-causal draft-head hot path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark may use it; the product path (the HIP library and its binding)
never imports it.  It shares no code with the HIP path.

Thin ctypes wrappers over ``oracle.c`` (built with gcc into
``oracle/liboracle.so``).  Inputs are numpy arrays already widened exactly to
float64; see ``oracle.c`` for the definitions and the passages they follow.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
  tree_mask  -- pinned: hand-derived golden fixture, chain/star closed forms,
                set recursion, bad-tree cases.
  tree_attn  -- pinned: chain == causal attention (library SDPA), star ==
                prefix+self attention, path-by-path brute force, hand-computed
                golden example, q=0 / lone-root closed forms, GQA head map via
                library SDPA with grouped heads, perturbation invariance.
  fuse_proj  -- pinned: numpy matmul of the concatenation, identity selector.
  topk       -- pinned: numpy lexsort brute force, all-equal rows, signed
                zeros, -inf, scipy logsumexp.
  path_scores -- pinned: hand-derived golden forest, chain == numpy cumsum,
                star == inputs, recursion on random forests, relabelling.
  tree_expand -- pinned: hand-derived golden step, numpy lexsort brute force
                over float32 scores, depth cap, budget, ties, signed zeros.
  swiglu     -- pinned: hand-derived golden values, silu(0) = 0, the odd
                part silu(g) - silu(-g) = g, the large-|g| limits, the
                logistic curve written as a tanh.
  rmsnorm    -- pinned: hand-derived golden rows, constant rows, unit RMS of
                the output at eps = 0, scale invariance, the weight as a
                per-column factor.
  tree_rope  -- pinned: hand-derived golden rotation (D = 4), position 0 is
                the identity, pair norms kept, rotations compose by adding
                positions, scores depend only on the position difference,
                a chain's positions are P, P+1, ...
  tree_accept -- pinned: hand-derived golden tree, top-down greedy-decoding
                simulation on trees with distinct sibling tokens, chain / star
                / nothing-accepted closed cases, duplicate siblings, bad trees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")
_lib = None

OK, INVALID, BAD_TREE, BAD_PAGE = 0, 1, 5, 6


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_tree_mask.argtypes = [P, P, I64, I64, P, P, P]
    lib.oracle_tree_mask.restype = ctypes.c_int
    lib.oracle_fuse_proj.argtypes = [P, I64, I64, I64, P, I64, P]
    lib.oracle_fuse_proj.restype = None
    lib.oracle_fuse_proj_rows.argtypes = [P, I64, I64, I64, P, I64, P, I64, P]
    lib.oracle_fuse_proj_rows.restype = None
    lib.oracle_tree_attn.argtypes = [P, P, P, P, P, P, P, I64, P, P, I64, I64, I64, I64, I64,
                                     I64, I64, ctypes.c_double, P, I64, P, P]
    lib.oracle_tree_attn.restype = ctypes.c_int
    lib.oracle_topk.argtypes = [P, I64, I64, I64, P, P, P]
    lib.oracle_topk.restype = None
    lib.oracle_path_scores.argtypes = [P, P, I64, I64, P, P]
    lib.oracle_path_scores.restype = ctypes.c_int
    lib.oracle_tree_expand.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, P, P, P, P]
    lib.oracle_tree_expand.restype = ctypes.c_int
    lib.oracle_tree_accept.argtypes = [P, P, P, P, I64, I64, P, P, P, P, P]
    lib.oracle_tree_accept.restype = ctypes.c_int
    lib.oracle_tree_rope.argtypes = [P, P, P, I64, I64, I64, I64, ctypes.c_double]
    lib.oracle_tree_rope.restype = None
    lib.oracle_rmsnorm.argtypes = [P, I64, I64, I64, P, ctypes.c_double, P]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_swiglu.argtypes = [P, I64, I64, P]
    lib.oracle_swiglu.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def tree_mask(parent: np.ndarray, node_off=None):
    """Ancestor bitmask, depth, status, first bad row.

    Uniform trees: parent [B, N] -> mask [B, N, ceil(N/64)] uint64, depth [B, N].
    Packed trees: parent [T] with node_off [B+1] (sequence b owns rows
    node_off[b] .. node_off[b+1]-1, parents local to it) -> mask [T, W] with
    W = ceil(max count / 64), depth [T]."""
    parent = _c(parent, np.int32)
    if node_off is None:
        B, N = parent.shape
        no, T = None, B * N
    else:
        no = _c(node_off, np.int64)
        B, T = no.shape[0] - 1, parent.shape[0]
        assert no[0] == 0 and no[-1] == T and np.all(np.diff(no) >= 1)
        N = int(np.max(np.diff(no)))
    W = (N + 63) // 64
    mask = np.zeros((T, W), dtype=np.uint64)
    depth = np.zeros((T,), dtype=np.int32)
    bad = np.zeros(1, dtype=np.int64)
    st = _load().oracle_tree_mask(_p(parent), _p(no) if no is not None else None, B, N, _p(mask),
                                  _p(depth), _p(bad))
    if no is None:
        mask, depth = mask.reshape(B, N, W), depth.reshape(B, N)
    return mask, depth, int(st), int(bad[0])


def fuse_proj(x: np.ndarray, w: np.ndarray, rows=None) -> np.ndarray:
    """x [k, M, H_in] float64, w [H_out, k*H_in] float64 -> y [M or len(rows), H_out]."""
    x = _c(x, np.float64)
    w = _c(w, np.float64)
    k, M, H_in = x.shape
    H_out = w.shape[0]
    assert w.shape == (H_out, k * H_in)
    lib = _load()
    if rows is None:
        y = np.empty((M, H_out), dtype=np.float64)
        lib.oracle_fuse_proj(_p(x), k, M, H_in, _p(w), H_out, _p(y))
    else:
        rows = _c(rows, np.int64)
        y = np.empty((rows.shape[0], H_out), dtype=np.float64)
        lib.oracle_fuse_proj_rows(_p(x), k, M, H_in, _p(w), H_out, _p(rows), rows.shape[0], _p(y))
    return y


def fp8_e4m3_to_f64(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (the "fn" variant: no infinities), times a
    per-tensor scale, in float64.  Sign bit 7; exponent bits 6..3 with bias 7;
    mantissa bits 2..0.  Exponent 0: subnormal m/8 * 2^-6; exponent 15 with
    mantissa 7: NaN; otherwise (1 + m/8) * 2^(e - 7)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sgn * mag * float(scale)


def tree_attn(*, q, k_tree, v_tree, parent, k_cache, v_cache, block_table, prefix_len,
              page_size, scale=None, rows=None, node_off=None, bad_page_ok=False):
    """Tree attention in float64.

    Uniform trees: q [B,N,Hq,D], k_tree/v_tree [B,N,Hkv,D], parent [B,N].
    Packed trees (node_off [B+1] given): q [T,Hq,D], k_tree/v_tree [T,Hkv,D],
    parent [T] with parents local to each sequence.
    k_cache/v_cache [num_pages,page_size,Hkv,D] (all float64), block_table
    [B,max_pages] int32, prefix_len [B] int32.
    Returns (out, lse): shaped like q and q without D, or [n_rows,D] and
    [n_rows] for rows = flat ids t*Hq+h over the tree rows t.  A bad page id
    raises unless bad_page_ok, which returns (out, lse, bad) with that
    position read as a zero key and a zero value.
    """
    q = _c(q, np.float64)
    k_tree = _c(k_tree, np.float64)
    v_tree = _c(v_tree, np.float64)
    k_cache = _c(k_cache, np.float64)
    v_cache = _c(v_cache, np.float64)
    parent = _c(parent, np.int32)
    block_table = _c(block_table, np.int32)
    prefix_len = _c(prefix_len, np.int32)
    if node_off is None:
        B, N, Hq, D = q.shape
        Hkv = k_tree.shape[2]
        no, T = None, B * N
    else:
        no = _c(node_off, np.int64)
        B, (T, Hq, D) = no.shape[0] - 1, q.shape
        Hkv = k_tree.shape[1]
        assert no[0] == 0 and no[-1] == T and np.all(np.diff(no) >= 1) and parent.shape == (T,)
        N = int(np.max(np.diff(no)))
    num_pages = k_cache.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        out = np.empty(q.shape, dtype=np.float64)
        lse = np.empty(q.shape[:-1], dtype=np.float64)
        rp, nr = None, 0
    else:
        rows = _c(rows, np.int64)
        out = np.empty((rows.shape[0], D), dtype=np.float64)
        lse = np.empty((rows.shape[0],), dtype=np.float64)
        rp, nr = _p(rows), rows.shape[0]
    st = _load().oracle_tree_attn(
        _p(q), _p(k_tree), _p(v_tree), _p(parent), _p(k_cache), _p(v_cache),
        _p(block_table), block_table.shape[1], _p(prefix_len), _p(no) if no is not None else None,
        B, N, Hq, Hkv, D, page_size, num_pages, float(scale), rp, nr, _p(out), _p(lse))
    if bad_page_ok and st in (OK, BAD_PAGE):
        return out, lse, st == BAD_PAGE
    if st != OK:
        raise ValueError(f"oracle_tree_attn status {st}")
    return out, lse


def topk(logits: np.ndarray, k: int, with_lse: bool = True):
    """Top-k (value desc, index asc) of each row of float64 logits [R, V]."""
    logits = _c(logits, np.float64)
    R, V = logits.shape
    idx = np.empty((R, k), dtype=np.int32)
    val = np.empty((R, k), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64) if with_lse else None
    _load().oracle_topk(_p(logits), R, V, k, _p(idx), _p(val), _p(lse))
    return idx, val, lse


def path_scores(parent: np.ndarray, logp: np.ndarray):
    """Path log-probability [B, N] float64 (sum of logp over anc(i)), status, first bad row."""
    parent = _c(parent, np.int32)
    logp = _c(logp, np.float64)
    B, N = parent.shape
    score = np.zeros((B, N), dtype=np.float64)
    bad = np.zeros(1, dtype=np.int64)
    st = _load().oracle_path_scores(_p(parent), _p(logp), B, N, _p(score), _p(bad))
    return score, int(st), int(bad[0])


def tree_expand(score: np.ndarray, depth: np.ndarray, idx: np.ndarray, val: np.ndarray,
                lse: np.ndarray, M: int, max_depth: int, parent: np.ndarray, token: np.ndarray):
    """One best-first expansion step of the trees (parent, token) [B, N]: the M
    best (node, rank) candidates of each sequence that are not already a child
    of their node -> new parent, token, score (float32), depth, each [B, M]."""
    score = _c(score, np.float32)
    depth = _c(depth, np.int32)
    idx = _c(idx, np.int32)
    val = _c(val, np.float32)
    lse = _c(lse, np.float32)
    parent = _c(parent, np.int32)
    token = _c(token, np.int32)
    B, N = score.shape
    k = idx.shape[-1]
    assert idx.shape == (B, N, k) and val.shape == (B, N, k) and lse.shape == (B, N)
    assert parent.shape == (B, N) and token.shape == (B, N)
    outp = np.zeros((B, M), dtype=np.int32)
    outt = np.zeros((B, M), dtype=np.int32)
    outs = np.zeros((B, M), dtype=np.float32)
    outd = np.zeros((B, M), dtype=np.int32)
    st = _load().oracle_tree_expand(_p(score), _p(depth), _p(idx), _p(val), _p(lse), _p(parent),
                                    _p(token), B, N, k, M, max_depth, _p(outp), _p(outt), _p(outs),
                                    _p(outd))
    if st != 0:
        raise ValueError(f"oracle_tree_expand: status {st}")
    return outp, outt, outs, outd


def tree_accept(parent: np.ndarray, token: np.ndarray, target_next: np.ndarray,
                root_next: np.ndarray):
    """Greedy verification of a drafted tree: (accept_len [B], accept_node [B],
    next_token [B], path [B, N], bad_node [B])."""
    parent = _c(parent, np.int32)
    token = _c(token, np.int32)
    target_next = _c(target_next, np.int32)
    root_next = _c(root_next, np.int32)
    B, N = parent.shape
    assert token.shape == (B, N) and target_next.shape == (B, N) and root_next.shape == (B,)
    alen = np.zeros(B, np.int32)
    anode = np.zeros(B, np.int32)
    ntok = np.zeros(B, np.int32)
    path = np.zeros((B, N), np.int32)
    bad = np.zeros(B, np.int32)
    st = _load().oracle_tree_accept(_p(parent), _p(token), _p(target_next), _p(root_next), B, N,
                                    _p(alen), _p(anode), _p(ntok), _p(path), _p(bad))
    if st != 0:
        raise ValueError(f"oracle_tree_accept: status {st}")
    return alen, anode, ntok, path, bad


def swiglu(gu: np.ndarray) -> np.ndarray:
    """silu(gate) * up from gu [M, 2I] (gate columns first) -> [M, I] float64."""
    gu = _c(gu, np.float64)
    M, I2 = gu.shape
    assert I2 % 2 == 0
    y = np.empty((M, I2 // 2), dtype=np.float64)
    _load().oracle_swiglu(_p(gu), M, I2 // 2, _p(y))
    return y


def rmsnorm(x: np.ndarray, w=None, eps: float = 1e-6) -> np.ndarray:
    """Rows of x [rows, H] (float64) divided by their root mean square
    (+ eps inside the root), times w [H] when given."""
    x = _c(x, np.float64)
    rows, H = x.shape
    wv = None if w is None else _c(w, np.float64)
    y = np.empty((rows, H), dtype=np.float64)
    _load().oracle_rmsnorm(_p(x), rows, H, H, _p(wv), float(eps), _p(y))
    return y


def tree_rope(x: np.ndarray, depth: np.ndarray, prefix_len, theta: float = 1e6) -> np.ndarray:
    """Rotary embedding of x [B, N, H, D] (float64 copy returned) at positions
    prefix_len[b] + depth[b, i] - 1; depth < 1 leaves a node unchanged."""
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    depth = _c(depth, np.int32)
    pl = _c(np.asarray(prefix_len), np.int32)
    B, N, H, D = x.shape
    assert D % 2 == 0 and depth.shape == (B, N) and pl.shape == (B,)
    _load().oracle_tree_rope(_p(x), _p(depth), _p(pl), B, N, H, D, float(theta))
    return x


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count for the oracle's later parallel loops (at least 1)."""
    _load().oracle_set_num_threads(int(n))
