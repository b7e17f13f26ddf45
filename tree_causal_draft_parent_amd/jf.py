"""Python binding of libjf (include/jf.h): argument marshalling only.

Each function has the C entry point's name, takes torch tensors that live on
the GPU, passes their device pointers and sizes to the C ABI, and raises
``JfError`` on a non-OK status.  Outputs and workspaces that the caller does
not pass are allocated with torch (PyTorch is the memory and stream provider);
every step of the computation runs in the HIP kernels of libjf.  There is no
fallback: if libjf.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjf.so")

JF_OK, JF_ERR_INVALID_ARG, JF_ERR_UNSUPPORTED, JF_ERR_ALIGN = 0, 1, 2, 3
JF_ERR_WORKSPACE, JF_ERR_BAD_TREE, JF_ERR_BAD_PAGE, JF_ERR_HIP = 4, 5, 6, 7
JF_ERR_BAD_PREFIX = 8
JF_F32, JF_BF16, JF_FP8_E4M3 = 0, 1, 2

EXPORTS = ("jf_status_string", "jf_abi_version", "jf_tree_mask_build",
           "jf_fuse_proj_workspace_size", "jf_fuse_proj", "jf_fuse_proj_workspace_size_cus",
           "jf_fuse_proj_cus", "jf_tree_attn_workspace_size",
           "jf_tree_attn_fwd", "jf_tree_attn_workspace_size_cus", "jf_tree_attn_fwd_cus",
           "jf_node_topk_workspace_size", "jf_node_topk", "jf_node_topk_noalloc", "jf_path_scores",
           "jf_tree_expand", "jf_tree_accept", "jf_tree_rope", "jf_rmsnorm", "jf_swiglu")

_lib = None


class JfError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


def lib():
    """Load libjf.so (built by tree_causal_draft_parent_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tree_causal_draft_parent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.jf_status_string.argtypes = [ctypes.c_int]
    L.jf_status_string.restype = ctypes.c_char_p
    L.jf_abi_version.argtypes = []
    L.jf_abi_version.restype = ctypes.c_int
    L.jf_tree_mask_build.argtypes = [P, P, I32, I32, P, P, P, P]
    L.jf_tree_mask_build.restype = ctypes.c_int
    L.jf_fuse_proj_workspace_size.argtypes = [I64, I64, I32, I64, ctypes.c_int]
    L.jf_fuse_proj_workspace_size.restype = SZ
    L.jf_fuse_proj.argtypes = [P, I32, I64, I64, I64, P, I64, ctypes.c_int, P, ctypes.c_int,
                               P, SZ, P]
    L.jf_fuse_proj.restype = ctypes.c_int
    L.jf_fuse_proj_workspace_size_cus.argtypes = [I64, I64, I32, I64, ctypes.c_int, I32]
    L.jf_fuse_proj_workspace_size_cus.restype = SZ
    L.jf_fuse_proj_cus.argtypes = [P, I32, I64, I64, I64, P, I64, ctypes.c_int, P, ctypes.c_int,
                                   P, SZ, I32, P]
    L.jf_fuse_proj_cus.restype = ctypes.c_int
    F = ctypes.c_float
    L.jf_tree_attn_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, P, P, ctypes.c_int]
    L.jf_tree_attn_workspace_size.restype = SZ
    L.jf_tree_attn_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, F, F, I64, I32, P, I32, P, P, P,
                                   I32, I32, I32, I32, I32, F, ctypes.c_int, P, P, P, SZ, P, P]
    L.jf_tree_attn_fwd.restype = ctypes.c_int
    L.jf_tree_attn_workspace_size_cus.argtypes = [I32, I32, I32, I32, I32, I32, P, P, ctypes.c_int,
                                                  I32]
    L.jf_tree_attn_workspace_size_cus.restype = SZ
    L.jf_tree_attn_fwd_cus.argtypes = [P, P, P, P, P, P, ctypes.c_int, F, F, I64, I32, P, I32, P, P,
                                       P, I32, I32, I32, I32, I32, F, ctypes.c_int, P, P, P, SZ, P,
                                       I32, P]
    L.jf_tree_attn_fwd_cus.restype = ctypes.c_int
    L.jf_node_topk_workspace_size.argtypes = [I64, I64, I32]
    L.jf_node_topk_workspace_size.restype = SZ
    L.jf_node_topk.argtypes = [P, I64, I64, I64, ctypes.c_int, I32, P, P, P, P, SZ, P]
    L.jf_node_topk.restype = ctypes.c_int
    L.jf_node_topk_noalloc.argtypes = [P, I64, I64, I64, ctypes.c_int, I32, P, P, P, P]
    L.jf_node_topk_noalloc.restype = ctypes.c_int
    L.jf_path_scores.argtypes = [P, P, I32, I32, P, P, P]
    L.jf_path_scores.restype = ctypes.c_int
    L.jf_tree_expand.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P]
    L.jf_tree_expand.restype = ctypes.c_int
    L.jf_tree_accept.argtypes = [P, P, P, P, I32, I32, P, P, P, P, P, P]
    L.jf_tree_accept.restype = ctypes.c_int
    L.jf_tree_rope.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, ctypes.c_double, ctypes.c_int, P]
    L.jf_tree_rope.restype = ctypes.c_int
    L.jf_rmsnorm.argtypes = [P, I64, I64, I64, P, ctypes.c_float, ctypes.c_int, P, P]
    L.jf_rmsnorm.restype = ctypes.c_int
    L.jf_swiglu.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P]
    L.jf_swiglu.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().jf_status_string(int(status)).decode()


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return JF_BF16
    if t.dtype == torch.float32:
        return JF_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn: str, st: int):
    if st != JF_OK:
        raise JfError(fn, st)


def _contig(name: str, t: torch.Tensor):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
def _node_off(node_off):
    """Host int32 [B+1] packed node offsets (or None), and the largest count."""
    if node_off is None:
        return None, 0
    no = _host_i32(node_off)
    return no, int(np.max(np.diff(no)))


def jf_tree_mask_build(parent: torch.Tensor, mask: Optional[torch.Tensor] = None,
                       depth: Optional[torch.Tensor] = None,
                       seq_status: Optional[torch.Tensor] = None, node_off=None, stream=None):
    """Uniform trees: parent [B, N] int32 -> (mask [B, N, ceil(N/64)] uint64
    (as int64), depth [B, N], seq_status [B]).  Packed trees: parent [T] with
    host node_off [B+1] -> (mask [T, W], depth [T], seq_status [B]) with W =
    ceil(largest count / 64).  On the parent's device."""
    _contig("parent", parent)
    no, nmax = _node_off(node_off)
    if no is None:
        B, N = parent.shape
        rows = (B, N)
    else:
        B, N = len(no) - 1, nmax
        rows = (parent.shape[0],)
    W = (N + 63) // 64
    dev = parent.device
    if mask is None:
        mask = torch.empty(rows + (W,), dtype=torch.int64, device=dev)
    if depth is None:
        depth = torch.empty(rows, dtype=torch.int32, device=dev)
    if seq_status is None:
        seq_status = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib().jf_tree_mask_build(_p(parent), None if no is None else no.ctypes.data_as(ctypes.c_void_p),
                                  B, N, _p(mask), _p(depth), _p(seq_status), _stream(stream))
    _check("jf_tree_mask_build", st)
    return mask, depth, seq_status


def jf_fuse_proj_workspace_size(M: int, H_in: int, k: int, H_out: int, in_dtype: int,
                                cus: int = 0) -> int:
    """cus > 0: the plan of jf_fuse_proj(..., cus=cus) (see jf_fuse_proj_cus)."""
    if cus > 0:
        return int(lib().jf_fuse_proj_workspace_size_cus(M, H_in, k, H_out, in_dtype, cus))
    return int(lib().jf_fuse_proj_workspace_size(M, H_in, k, H_out, in_dtype))


def jf_fuse_proj(xs: Sequence[torch.Tensor], w: torch.Tensor, out_dtype=torch.float32,
                 y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None, cus: int = 0):
    """y[m, o] = sum_l xs[l][m, :] . w[o, l*H_in:(l+1)*H_in]  (xs[l]: [M, H_in], rows may be
    strided; w: [H_out, k*H_in]).  cus > 0 plans the K split for that many
    compute units (jf_fuse_proj_cus); the workspace must then be sized with
    the same cus."""
    k = len(xs)
    M, H_in = xs[0].shape
    ldx = xs[0].stride(0)
    for x in xs:
        if x.shape != (M, H_in) or x.stride(1) != 1 or x.stride(0) != ldx or x.dtype != xs[0].dtype:
            raise ValueError("fused inputs must share shape, dtype and row stride")
    _contig("w", w)
    H_out = w.shape[0]
    in_code = _dtype_code(xs[0])
    if y is None:
        y = torch.empty((M, H_out), dtype=out_dtype, device=w.device)
    out_code = _dtype_code(y)
    need = jf_fuse_proj_workspace_size(M, H_in, k, H_out, in_code, cus)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    arr = (ctypes.c_void_p * k)(*[x.data_ptr() for x in xs])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if cus > 0:
        st = lib().jf_fuse_proj_cus(arr, k, M, H_in, ldx, _p(w), H_out, in_code, _p(y), out_code,
                                    _p(workspace), ws_bytes, int(cus), _stream(stream))
    else:
        st = lib().jf_fuse_proj(arr, k, M, H_in, ldx, _p(w), H_out, in_code, _p(y), out_code,
                                _p(workspace), ws_bytes, _stream(stream))
    _check("jf_fuse_proj", st)
    return y


def _host_i32(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def jf_tree_attn_workspace_size(B: int, N: int, Hq: int, Hkv: int, D: int, page_size: int,
                                prefix_len, dtype: int, cus: int = 0, node_off=None) -> int:
    """cus > 0: the plan of jf_tree_attn_fwd(..., cus=cus) (see jf_tree_attn_fwd_cus)."""
    pl = _host_i32(prefix_len)
    no, _ = _node_off(node_off)
    nop = None if no is None else no.ctypes.data_as(ctypes.c_void_p)
    if cus > 0:
        return int(lib().jf_tree_attn_workspace_size_cus(B, N, Hq, Hkv, D, page_size,
                                                         pl.ctypes.data_as(ctypes.c_void_p), nop,
                                                         dtype, cus))
    return int(lib().jf_tree_attn_workspace_size(B, N, Hq, Hkv, D, page_size,
                                                 pl.ctypes.data_as(ctypes.c_void_p), nop, dtype))


def _kv_code(t: torch.Tensor) -> int:
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return JF_FP8_E4M3
    return _dtype_code(t)


def jf_tree_attn_fwd(q, k_tree, v_tree, mask, k_cache, v_cache, block_table, prefix_len,
                     scale: float = 0.0, out=None, lse=None, with_lse: bool = True,
                     workspace=None, status=None, stream=None, cus: int = 0,
                     prefix_len_dev=None, node_off=None, k_scale: float = 1.0,
                     v_scale: float = 1.0):
    """Tree attention.  Uniform trees: q [B,N,Hq,D], k_tree/v_tree [B,N,Hkv,D];
    packed trees (host node_off [B+1]): q [T,Hq,D], k_tree/v_tree [T,Hkv,D].
    mask from jf_tree_mask_build; k_cache/v_cache [num_pages, page_size, Hkv, D]
    of q's dtype, or E4M3 codes (uint8 / float8_e4m3fn) with per-tensor scales
    k_scale / v_scale; block_table [B, max_pages] int32 (device); prefix_len
    host ints [B]: the lengths, or their upper bounds when prefix_len_dev (a
    device int32 [B] tensor) gives the lengths.  cus > 0 plans the key splits
    for that many compute units (jf_tree_attn_fwd_cus); the workspace must
    then be sized with the same cus.  status: a device int32 word for data
    errors (bad page id, device prefix length outside its bound)."""
    for n, t in (("q", q), ("k_tree", k_tree), ("v_tree", v_tree), ("mask", mask),
                 ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table)):
        _contig(n, t)
    no, nmax = _node_off(node_off)
    if no is None:
        B, N, Hq, D = q.shape
        Hkv = k_tree.shape[2]
    else:
        B, N = len(no) - 1, nmax
        _, Hq, D = q.shape
        Hkv = k_tree.shape[1]
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    dt = _dtype_code(q)
    kv = _kv_code(k_cache)
    pl = _host_i32(prefix_len)
    if prefix_len_dev is not None:
        _contig("prefix_len_dev", prefix_len_dev)
        if prefix_len_dev.dtype != torch.int32 or prefix_len_dev.shape != (B,):
            raise ValueError("prefix_len_dev must be a device int32 [B] tensor")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and with_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    need = jf_tree_attn_workspace_size(B, N, Hq, Hkv, D, page_size, pl, dt, cus, no)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    nop = None if no is None else no.ctypes.data_as(ctypes.c_void_p)
    args = [_p(q), _p(k_tree), _p(v_tree), _p(mask), _p(k_cache), _p(v_cache), kv, float(k_scale),
            float(v_scale), num_pages, page_size, _p(block_table), max_pages,
            pl.ctypes.data_as(ctypes.c_void_p), _p(prefix_len_dev), nop, B, N, Hq, Hkv, D,
            float(scale), dt, _p(out), _p(lse), _p(workspace), ws_bytes, _p(status)]
    if cus > 0:
        st = lib().jf_tree_attn_fwd_cus(*args, int(cus), _stream(stream))
    else:
        st = lib().jf_tree_attn_fwd(*args, _stream(stream))
    _check("jf_tree_attn_fwd", st)
    return out, lse


def jf_node_topk_workspace_size(R: int, V: int, k: int) -> int:
    return int(lib().jf_node_topk_workspace_size(R, V, k))


def jf_node_topk(logits: torch.Tensor, k: int, with_lse: bool = True, idx=None, val=None,
                 lse=None, workspace=None, stream=None):
    """logits [R, V] (row stride may exceed V) -> idx [R, k] int32, val [R, k] fp32, lse [R]."""
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    R, V = logits.shape
    ld = logits.stride(0)
    dev = logits.device
    if idx is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=dev)
    if val is None:
        val = torch.empty((R, k), dtype=torch.float32, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((R,), dtype=torch.float32, device=dev)
    need = jf_node_topk_workspace_size(R, V, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().jf_node_topk(_p(logits), R, V, ld, _dtype_code(logits), k, _p(idx), _p(val), _p(lse),
                            _p(workspace), ws_bytes, _stream(stream))
    _check("jf_node_topk", st)
    return idx, val, lse


# JF_NODE_TOPK_SCRATCH_BYTES of include/jf.h
NODE_TOPK_SCRATCH_BYTES = 4 << 20


def jf_node_topk_noalloc(logits: torch.Tensor, k: int, idx: torch.Tensor, val: torch.Tensor,
                         lse: Optional[torch.Tensor] = None, stream=None):
    """jf_node_topk without a workspace: the library's static per-GPU scratch
    (calls that overlap on one GPU race).  The outputs are the caller's:
    idx [R, k] int32, val [R, k] fp32, lse [R] fp32 or None."""
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    R, V = logits.shape
    for n, t, dt in (("idx", idx, torch.int32), ("val", val, torch.float32)):
        _contig(n, t)
        if t.shape != (R, k) or t.dtype != dt:
            raise ValueError(f"{n} must be [R, k] {dt}")
    if lse is not None and (lse.shape != (R,) or lse.dtype != torch.float32):
        raise ValueError("lse must be [R] float32")
    st = lib().jf_node_topk_noalloc(_p(logits), R, V, logits.stride(0), _dtype_code(logits), k,
                                    _p(idx), _p(val), _p(lse), _stream(stream))
    _check("jf_node_topk_noalloc", st)
    return idx, val, lse


def jf_path_scores(parent: torch.Tensor, logp: torch.Tensor, score=None, seq_status=None,
                   stream=None):
    """parent [B, N] int32, logp [B, N] fp32 -> (score [B, N] fp32, seq_status [B] int32):
    the sum of logp over each node's ancestors, itself included."""
    _contig("parent", parent)
    _contig("logp", logp)
    B, N = parent.shape
    if logp.shape != (B, N) or logp.dtype != torch.float32 or parent.dtype != torch.int32:
        raise ValueError("parent [B, N] int32 and logp [B, N] float32 expected")
    dev = parent.device
    if score is None:
        score = torch.empty((B, N), dtype=torch.float32, device=dev)
    if seq_status is None:
        seq_status = torch.empty((B,), dtype=torch.int32, device=dev)
    st = lib().jf_path_scores(_p(parent), _p(logp), B, N, _p(score), _p(seq_status),
                              _stream(stream))
    _check("jf_path_scores", st)
    return score, seq_status


def jf_tree_expand(score: torch.Tensor, depth: torch.Tensor, idx: torch.Tensor,
                   val: torch.Tensor, lse: torch.Tensor, parent: torch.Tensor,
                   token: torch.Tensor, M: int, max_depth: int, out=None, stream=None):
    """One best-first expansion step of the trees (parent, token) [B, N] int32:
    score [B, N] fp32, depth [B, N] int32, idx [B, N, k] int32, val [B, N, k]
    fp32, lse [B, N] fp32 -> the M best one-token extensions of each
    sequence's tree that are not already children, as (new_parent, new_token,
    new_score, new_depth), each [B, M]."""
    for n, t in (("score", score), ("depth", depth), ("idx", idx), ("val", val), ("lse", lse),
                 ("parent", parent), ("token", token)):
        _contig(n, t)
    B, N = score.shape
    k = idx.shape[-1]
    if (depth.shape != (B, N) or idx.shape != (B, N, k) or val.shape != (B, N, k)
            or lse.shape != (B, N) or parent.shape != (B, N) or token.shape != (B, N)):
        raise ValueError("inconsistent shapes")
    if (score.dtype != torch.float32 or val.dtype != torch.float32 or lse.dtype != torch.float32
            or depth.dtype != torch.int32 or idx.dtype != torch.int32
            or parent.dtype != torch.int32 or token.dtype != torch.int32):
        raise ValueError("score/val/lse float32 and depth/idx/parent/token int32 expected")
    dev = score.device
    if out is None:
        out = (torch.empty((B, M), dtype=torch.int32, device=dev),
               torch.empty((B, M), dtype=torch.int32, device=dev),
               torch.empty((B, M), dtype=torch.float32, device=dev),
               torch.empty((B, M), dtype=torch.int32, device=dev))
    np_, nt, ns, nd = out
    st = lib().jf_tree_expand(_p(score), _p(depth), _p(idx), _p(val), _p(lse), _p(parent),
                              _p(token), B, N, k, int(M), int(max_depth), _p(np_), _p(nt), _p(ns),
                              _p(nd), _stream(stream))
    _check("jf_tree_expand", st)
    return np_, nt, ns, nd


def jf_tree_accept(parent: torch.Tensor, token: torch.Tensor, target_next: torch.Tensor,
                   root_next: torch.Tensor, out=None, with_path: bool = True, stream=None):
    """Greedy verification: parent, token, target_next [B, N] int32 and
    root_next [B] int32 -> (accept_len [B], accept_node [B], next_token [B],
    path [B, N] or None, seq_status [B])."""
    for n, t in (("parent", parent), ("token", token), ("target_next", target_next),
                 ("root_next", root_next)):
        _contig(n, t)
        if t.dtype != torch.int32:
            raise ValueError(f"{n} must be int32")
    B, N = parent.shape
    if token.shape != (B, N) or target_next.shape != (B, N) or root_next.shape != (B,):
        raise ValueError("inconsistent shapes")
    dev = parent.device
    if out is None:
        out = (torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, N), dtype=torch.int32, device=dev) if with_path else None,
               torch.empty((B,), dtype=torch.int32, device=dev))
    alen, anode, ntok, path, st = out
    s = lib().jf_tree_accept(_p(parent), _p(token), _p(target_next), _p(root_next), B, N,
                             _p(alen), _p(anode), _p(ntok), _p(path), _p(st), _stream(stream))
    _check("jf_tree_accept", s)
    return alen, anode, ntok, path, st


def jf_tree_rope(q: torch.Tensor, k: Optional[torch.Tensor], depth: torch.Tensor,
                 prefix_len: torch.Tensor, theta: float = 0.0, stream=None):
    """Rotate q [B, N, Hq, D] (and k [B, N, Hkv, D]) in place at positions
    prefix_len[b] + depth[b, i] - 1 (prefix_len: device int32 [B])."""
    _contig("q", q)
    if k is not None:
        _contig("k", k)
        if k.dtype != q.dtype or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
            raise ValueError("k must match q in dtype, B, N and D")
    _contig("depth", depth)
    _contig("prefix_len", prefix_len)
    B, N, Hq, D = q.shape
    Hkv = 0 if k is None else k.shape[2]
    if depth.shape != (B, N) or depth.dtype != torch.int32 or prefix_len.shape != (B,) \
            or prefix_len.dtype != torch.int32:
        raise ValueError("depth [B, N] and prefix_len [B] int32 expected")
    st = lib().jf_tree_rope(_p(q), _p(k), _p(depth), _p(prefix_len), B, N, Hq, Hkv, D,
                            float(theta), _dtype_code(q), _stream(stream))
    _check("jf_tree_rope", st)
    return q, k


def jf_rmsnorm(x: torch.Tensor, w: Optional[torch.Tensor] = None, eps: float = 1e-6,
               y: Optional[torch.Tensor] = None, stream=None):
    """Rows of x (2-D, unit column stride; any leading row stride) divided by
    their root mean square, times w [H] when given -> y [rows, H] (y may be x
    when x is dense: in place)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, H = x.shape
    if w is not None:
        _contig("w", w)
        if w.shape != (H,) or w.dtype != x.dtype:
            raise ValueError("w must be [H] of x's dtype")
    if y is None:
        y = torch.empty((rows, H), dtype=x.dtype, device=x.device)
    _contig("y", y)
    st = lib().jf_rmsnorm(_p(x), rows, H, x.stride(0), _p(w), float(eps), _dtype_code(x), _p(y),
                          _stream(stream))
    _check("jf_rmsnorm", st)
    return y


def jf_swiglu(gu: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None):
    """silu(gate) * up from gu [M, 2I] (gate columns first; rows may be
    strided) -> y [M, I]."""
    if gu.dim() != 2 or gu.stride(1) != 1 or gu.shape[1] % 2:
        raise ValueError("gu must be [M, 2I] with contiguous rows")
    M, I = gu.shape[0], gu.shape[1] // 2
    if y is None:
        y = torch.empty((M, I), dtype=gu.dtype, device=gu.device)
    _contig("y", y)
    st = lib().jf_swiglu(_p(gu), M, I, gu.stride(0), _dtype_code(gu), _p(y), _stream(stream))
    _check("jf_swiglu", st)
    return y
