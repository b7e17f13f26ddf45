"""The C ABI on a machine without a GPU: the library loads, exports every
function include/jf.h declares, and rejects bad arguments before any HIP call
(no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from tree_causal_draft_parent_amd import jf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "jf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jf_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 20
    assert sorted(jf.EXPORTS) == names
    L = jf.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert jf.status_string(0) == "JF_OK"
    assert jf.status_string(5) == "JF_ERR_BAD_TREE"
    assert jf.lib().jf_abi_version() == 6
    assert jf.status_string(8) == "JF_ERR_BAD_PREFIX"


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x10001)


def test_mask_argument_errors():
    L = jf.lib()
    assert L.jf_tree_mask_build(None, None, 1, 4, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, None, 0, 4, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, None, 1, 0, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, None, 1, 5000, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, None, 1, 4, FAKE_ODD, None, None, None) == jf.JF_ERR_ALIGN
    # packed node offsets: start at 0, at least one node a sequence, N = the largest count
    off = lambda *v: np.array(v, np.int32).ctypes.data_as(ctypes.c_void_p)
    assert L.jf_tree_mask_build(FAKE, off(1, 3, 7), 2, 4, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, off(0, 3, 3), 2, 3, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, off(0, 3, 7), 2, 5, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_tree_mask_build(FAKE, off(0, 3, 9), 2, 4, FAKE, None, None, None) == jf.JF_ERR_INVALID_ARG
    big = np.arange(302, dtype=np.int32).ctypes.data_as(ctypes.c_void_p)
    assert L.jf_tree_mask_build(FAKE, big, 301, 1, FAKE, None, None, None) == jf.JF_ERR_UNSUPPORTED


def _attn(L, **kw):
    a = dict(q=FAKE, kt=FAKE, vt=FAKE, mask=FAKE, kc=FAKE, vc=FAKE, kv=None, ks=1.0, vs=1.0,
             num_pages=4, page_size=16, bt=FAKE, max_pages=4, pl=np.array([10, 20], np.int32),
             pdev=None, no=None, B=2, N=8, Hq=8, Hkv=2, D=128, scale=0.0, dtype=jf.JF_BF16,
             out=FAKE, lse=None, ws=None, ws_bytes=0, ps=None)
    a.update(kw)
    if a["kv"] is None:
        a["kv"] = a["dtype"]
    pl, no = a["pl"], a["no"]
    plp = None if pl is None else pl.ctypes.data_as(ctypes.c_void_p)
    nop = None if no is None else np.asarray(no, np.int32).ctypes.data_as(ctypes.c_void_p)
    return L.jf_tree_attn_fwd(a["q"], a["kt"], a["vt"], a["mask"], a["kc"], a["vc"], a["kv"], a["ks"],
                              a["vs"], a["num_pages"], a["page_size"], a["bt"], a["max_pages"], plp,
                              a["pdev"], nop, a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                              a["dtype"], a["out"], a["lse"], a["ws"], a["ws_bytes"], a["ps"], None)


def _ws(L, B, N, Hq, Hkv, D, page, pl, dtype, no=None, cus=None):
    plp = np.asarray(pl, np.int32).ctypes.data_as(ctypes.c_void_p)
    nop = None if no is None else np.asarray(no, np.int32).ctypes.data_as(ctypes.c_void_p)
    if cus is None:
        return L.jf_tree_attn_workspace_size(B, N, Hq, Hkv, D, page, plp, nop, dtype)
    return L.jf_tree_attn_workspace_size_cus(B, N, Hq, Hkv, D, page, plp, nop, dtype, cus)


def test_attn_argument_errors():
    L = jf.lib()
    assert _attn(L, q=None) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, pl=None) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, Hq=6, Hkv=4) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, D=96) == jf.JF_ERR_UNSUPPORTED          # bf16: D = 64 or 128
    assert _attn(L, D=64) != jf.JF_ERR_UNSUPPORTED
    assert _attn(L, D=256, dtype=jf.JF_F32) == jf.JF_ERR_UNSUPPORTED
    assert _attn(L, N=2000) == jf.JF_ERR_UNSUPPORTED
    assert _attn(L, B=300, pl=np.zeros(300, np.int32)) == jf.JF_ERR_UNSUPPORTED
    assert _attn(L, pl=np.array([10, -1], np.int32)) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, pl=np.array([10, 65], np.int32)) == jf.JF_ERR_INVALID_ARG  # > 4 pages of 16
    assert _attn(L, page_size=0) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, q=FAKE_ODD) == jf.JF_ERR_ALIGN
    assert _attn(L, pdev=FAKE_ODD) == jf.JF_ERR_ALIGN
    assert _attn(L, kv=9) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, kv=jf.JF_F32) == jf.JF_ERR_UNSUPPORTED       # the cache must match q or be FP8
    assert _attn(L, kv=jf.JF_FP8_E4M3, dtype=jf.JF_F32) == jf.JF_ERR_UNSUPPORTED
    assert _attn(L, kv=jf.JF_FP8_E4M3, ks=0.0) == jf.JF_ERR_INVALID_ARG       # scales must be > 0
    assert _attn(L, kv=jf.JF_FP8_E4M3, vs=-1.0) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, kv=jf.JF_FP8_E4M3, vs=float("inf")) == jf.JF_ERR_INVALID_ARG
    # packed trees: offsets from 0, every sequence has nodes, N is the largest count
    assert _attn(L, no=[0, 3, 11]) != jf.JF_ERR_INVALID_ARG      # counts 3 and 8
    assert _attn(L, no=[1, 3, 8]) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, no=[0, 0, 8]) == jf.JF_ERR_INVALID_ARG
    assert _attn(L, no=[0, 3, 7]) == jf.JF_ERR_INVALID_ARG       # largest count 4 != N = 8
    # this shape splits the keys, so a workspace is required
    pl = np.array([4096, 4096], np.int32)
    need = _ws(L, 2, 256, 32, 8, 128, 4096, pl, 1)
    assert need > 0
    assert _attn(L, pl=pl, N=256, Hq=32, Hkv=8, max_pages=1, page_size=4096,
                 ws=FAKE, ws_bytes=need - 1) == jf.JF_ERR_WORKSPACE


def test_workspace_sizes_are_host_side_and_consistent():
    L = jf.lib()
    a = _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 1)
    assert a % 4 == 0
    assert _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 0) == 0    # fp32 path: no splits
    assert _ws(L, 1, 256, 32, 7, 128, 4096, [4096], 1) == 0    # invalid -> 0
    assert L.jf_node_topk_workspace_size(256, 151936, 8) > 0
    assert L.jf_node_topk_workspace_size(4, 10, 65) == 0
    assert L.jf_fuse_proj_workspace_size(256, 4096, 3, 4096, 1) >= 0
    assert L.jf_fuse_proj_workspace_size(256, 100, 3, 4096, 1) == 0  # H_in % 64 != 0


def _attn_ws_bytes(items):
    rows = items * 256                      # fp32 O / l rows of 128 + one fp32 lse, per work item
    return rows * 128 * 4 + rows * 4


def test_attn_plan_for_fewer_compute_units():
    # the _cus entry points plan the key splits for fewer compute units: at
    # 4096 prefix tokens and 256 nodes (68 key blocks, 8 KV heads, 4 query
    # tiles) 192 units give splits of 12 blocks (6 a sequence) instead of 9
    # (8 a sequence), so the partials take 6/8 of the bytes
    L = jf.lib()
    full = _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 1)
    assert _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 1, cus=0) == full
    assert _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 1, cus=100000) == full
    assert full == _attn_ws_bytes(8 * 8 * 4)
    assert _ws(L, 1, 256, 32, 8, 128, 4096, [4096], 1, cus=192) == _attn_ws_bytes(6 * 8 * 4)
    assert _ws(L, 1, 256, 32, 7, 128, 4096, [4096], 1, cus=192) == 0  # invalid -> 0


def test_attn_plan_cuts_rows_into_nearly_equal_pieces():
    # rows of 17, 9 and 5 key blocks (prefixes 1024, 512, 256 with 16 nodes,
    # one KV head, one query tile each) = 31 block units.  4 compute units give
    # a piece target of 8 blocks: 3 + 2 + 1 pieces (6, 6, 5 / 5, 4 / 5), 6
    # work items, more than one wave; the dispatch model then prefers pieces
    # of at most 9 blocks (9, 8 / 9 / 5): 4 items in one wave, span 9 + 4
    # against 18 for the 6 items (each item costs its blocks plus 4)
    L = jf.lib()
    assert _ws(L, 3, 16, 4, 1, 128, 16, [1024, 512, 256], 1, cus=4) == _attn_ws_bytes(4)
    # 2 compute units: a target of 16 blocks gives the same pieces (9, 8 / 9 /
    # 5), 4 items in two waves
    assert _ws(L, 3, 16, 4, 1, 128, 16, [1024, 512, 256], 1, cus=2) == _attn_ws_bytes(4)
    # one compute unit: every row in one piece, nothing to merge
    assert _ws(L, 3, 16, 4, 1, 128, 16, [1024, 512, 256], 1, cus=1) == 0


def test_attn_plan_models_dispatch_per_xcd():
    # rows of 17, 17, 3, 3 and 3 key blocks (prefixes 1024, 1024, 128 x 3 with
    # 16 nodes, one KV head, one query tile) = 43 units; 8 compute units, one
    # in each of the 8 XCDs.  The target of 6 blocks gives pieces 6, 6, 5 of
    # the long rows: 9 items costing 10 10 9 10 10 9 7 7 7.  Workgroup ids go
    # round-robin over the XCDs, so the ninth item (cost 7) queues behind the
    # first (cost 10) in the first XCD: span 17 (one pool of 8 units would
    # start it on a unit that frees at 7: span 14).  Pieces of at most 9-11 blocks (9, 8)
    # give 7 items in one wave, span 13 <= 0.9 x 17, and win (the largest of
    # the tied sizes); against the pool's 14 they would not.
    L = jf.lib()
    assert _ws(L, 5, 16, 4, 1, 128, 16, [1024, 1024, 128, 128, 128], 1, cus=8) == _attn_ws_bytes(7)


def test_attn_plan_refuses_item_counts_beyond_32_bits():
    # 256 sequences x 1024 nodes at 32/8 heads (128 rows each) with prefix
    # bounds near 2^31 in 16-token pages: pieces of at most 2046 pages (511
    # blocks) give ~2e9 work items, past the 32-bit item indices -> refused,
    # before any device access (the pointers here are not real)
    L = jf.lib()
    pl = np.full(256, 2 ** 31 - 64, np.int32)
    assert _attn(L, B=256, N=1024, Hq=32, Hkv=8, pl=pl, num_pages=1, page_size=16,
                 max_pages=2 ** 27) == jf.JF_ERR_UNSUPPORTED
    assert _ws(L, 256, 1024, 32, 8, 128, 16, pl, 1) == 0
    # bounds of 2^28 tokens (~3e8 items) plan, and stop at the missing workspace
    pl = np.full(256, 2 ** 28, np.int32)
    assert _attn(L, B=256, N=1024, Hq=32, Hkv=8, pl=pl, num_pages=1, page_size=16,
                 max_pages=2 ** 27) == jf.JF_ERR_WORKSPACE


def test_attn_plan_of_packed_trees():
    # packed trees of 256 and 16 nodes (4 and 1 query tiles of 256 rows per KV
    # head) are planned together: 68 and 65 key blocks, 8 KV heads -> 2696
    # block units over 256 compute units; the workspace is whole work items
    L = jf.lib()
    packed = _ws(L, 2, 256, 32, 8, 128, 4096, [4096, 4096], 1, no=[0, 256, 272])
    assert packed > 0 and packed % _attn_ws_bytes(1) == 0
    # one compute unit's worth of splits: every (sequence, head, tile) unsplit
    assert _ws(L, 2, 256, 32, 8, 128, 4096, [4096, 4096], 1, no=[0, 256, 272], cus=1) == 0
    # invalid offsets -> 0
    assert _ws(L, 2, 256, 32, 8, 128, 4096, [4096, 4096], 1, no=[0, 256, 256]) == 0


def test_fuse_plan_for_fewer_compute_units():
    # 256 rows x 4096 outputs from 3 x 4096 inputs: 32 output tiles; 256 units
    # take 8 K slices of fp32 partials, 192 units 6
    L = jf.lib()
    full = L.jf_fuse_proj_workspace_size(256, 4096, 3, 4096, 1)
    assert full == 8 * 256 * 4096 * 4
    assert L.jf_fuse_proj_workspace_size_cus(256, 4096, 3, 4096, 1, 0) == full
    assert L.jf_fuse_proj_workspace_size_cus(256, 4096, 3, 4096, 1, 192) == 6 * 256 * 4096 * 4
    assert L.jf_fuse_proj_workspace_size_cus(256, 4096, 3, 4096, 1, 32) == 0      # one slice: no partials
    assert L.jf_fuse_proj_workspace_size_cus(256, 100, 3, 4096, 1, 192) == 0      # invalid -> 0
    # the MLP's gate/up projection, 256 x 4096 -> 24576: 192 tiles, more than
    # half a wave of 256 units, so no K split (two slices would only make two
    # half-length waves plus the partials); 96 tiles still split in two
    assert L.jf_fuse_proj_workspace_size_cus(256, 4096, 1, 24576, 1, 256) == 0
    assert L.jf_fuse_proj_workspace_size_cus(256, 4096, 1, 12288, 1, 256) == 3 * 256 * 12288 * 4


def test_fuse_and_topk_argument_errors():
    L = jf.lib()
    xs = (ctypes.c_void_p * 3)(0x10000, 0x20000, 0x30000)
    assert L.jf_fuse_proj(None, 3, 16, 256, 256, FAKE, 256, 1, FAKE, 0, None, 0, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_fuse_proj(xs, 0, 16, 256, 256, FAKE, 256, 1, FAKE, 0, None, 0, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_fuse_proj(xs, 3, 16, 100, 128, FAKE, 256, 1, FAKE, 0, None, 0, None) == jf.JF_ERR_UNSUPPORTED
    assert L.jf_fuse_proj(xs, 3, 16, 256, 200, FAKE, 256, 1, FAKE, 0, None, 0, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_fuse_proj(xs, 3, 16, 256, 260, FAKE, 256, 1, FAKE, 0, None, 0, None) == jf.JF_ERR_ALIGN
    assert L.jf_fuse_proj(xs, 3, 16, 256, 256, FAKE, 256, 0, FAKE, 1, None, 0, None) == jf.JF_ERR_UNSUPPORTED
    assert L.jf_node_topk(None, 4, 100, 100, 1, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_node_topk(FAKE, 4, 100, 99, 1, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_node_topk(FAKE, 4, 100, 100, 1, 65, FAKE, FAKE, None, FAKE, 1 << 20, None) == jf.JF_ERR_UNSUPPORTED
    assert L.jf_node_topk(FAKE, 4, 100, 100, 1, 101, FAKE, FAKE, None, FAKE, 1 << 20, None) == jf.JF_ERR_UNSUPPORTED
    assert L.jf_node_topk(FAKE, 4, 100, 100, 1, 4, FAKE, FAKE, None, FAKE, 1 << 20, None) == jf.JF_ERR_ALIGN
    assert L.jf_node_topk(FAKE, 4, 104, 104, 1, 4, FAKE, FAKE, None, None, 0, None) == jf.JF_ERR_WORKSPACE


def test_noalloc_topk_argument_errors():
    L = jf.lib()
    ok = [FAKE, 4, 104, 104, 1, 4, FAKE, FAKE, None, None]
    assert L.jf_node_topk_noalloc(*ok[:0], None, *ok[1:]) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[1] = 0
    assert L.jf_node_topk_noalloc(*bad) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[5] = 65
    assert L.jf_node_topk_noalloc(*bad) == jf.JF_ERR_UNSUPPORTED
    bad = list(ok); bad[0] = FAKE_ODD
    assert L.jf_node_topk_noalloc(*bad) == jf.JF_ERR_ALIGN
    # a size whose workspace exceeds the static scratch is refused before any HIP call
    big = [FAKE, 1024, 622592, 622592, 1, 64, FAKE, FAKE, None, None]
    assert jf.jf_node_topk_workspace_size(1024, 622592, 64) > jf.NODE_TOPK_SCRATCH_BYTES
    assert L.jf_node_topk_noalloc(*big) == jf.JF_ERR_WORKSPACE


def test_noalloc_scratch_limit_matches_the_header():
    src = open(os.path.join(ROOT, "include", "jf.h")).read()
    m = re.search(r"#define JF_NODE_TOPK_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == jf.NODE_TOPK_SCRATCH_BYTES


def test_path_and_expand_argument_errors():
    L = jf.lib()
    assert L.jf_path_scores(None, FAKE, 1, 4, FAKE, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_path_scores(FAKE, FAKE, 0, 4, FAKE, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_path_scores(FAKE, FAKE, 1, 4097, FAKE, None, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_path_scores(FAKE, FAKE_ODD, 1, 4, FAKE, None, None) == jf.JF_ERR_ALIGN

    def exp(**kw):
        a = dict(score=FAKE, depth=FAKE, idx=FAKE, val=FAKE, lse=FAKE, parent=FAKE, token=FAKE,
                 B=1, N=256, k=8, M=256, max_depth=16, np_=FAKE, nt=FAKE, ns=FAKE, nd=FAKE)
        a.update(kw)
        return L.jf_tree_expand(a["score"], a["depth"], a["idx"], a["val"], a["lse"], a["parent"],
                                a["token"], a["B"], a["N"], a["k"], a["M"], a["max_depth"],
                                a["np_"], a["nt"], a["ns"], a["nd"], None)

    assert exp(lse=None) == jf.JF_ERR_INVALID_ARG
    assert exp(parent=None) == jf.JF_ERR_INVALID_ARG
    assert exp(token=None) == jf.JF_ERR_INVALID_ARG
    assert exp(token=FAKE_ODD) == jf.JF_ERR_ALIGN
    assert exp(nd=None) == jf.JF_ERR_INVALID_ARG
    assert exp(B=0) == jf.JF_ERR_INVALID_ARG
    assert exp(k=0) == jf.JF_ERR_INVALID_ARG
    assert exp(M=0) == jf.JF_ERR_INVALID_ARG
    assert exp(N=2049) == jf.JF_ERR_UNSUPPORTED          # 2049 * 8 candidates > 16384
    assert exp(N=16384, k=2) == jf.JF_ERR_UNSUPPORTED
    assert exp(val=FAKE_ODD) == jf.JF_ERR_ALIGN


def test_accept_argument_errors():
    L = jf.lib()
    ok = [FAKE, FAKE, FAKE, FAKE, 2, 64, FAKE, FAKE, FAKE, None, None, None]
    assert L.jf_tree_accept(*ok[:0], None, *ok[1:]) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[3] = None
    assert L.jf_tree_accept(*bad) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[4] = 0
    assert L.jf_tree_accept(*bad) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[5] = 4097
    assert L.jf_tree_accept(*bad) == jf.JF_ERR_INVALID_ARG
    bad = list(ok); bad[9] = FAKE_ODD                      # path misaligned
    assert L.jf_tree_accept(*bad) == jf.JF_ERR_ALIGN


def test_rope_argument_errors():
    L = jf.lib()

    def rope(**kw):
        a = dict(q=FAKE, k=FAKE, depth=FAKE, pl=FAKE, B=1, N=16, Hq=32, Hkv=8, D=128, theta=0.0,
                 dtype=jf.JF_BF16)
        a.update(kw)
        return L.jf_tree_rope(a["q"], a["k"], a["depth"], a["pl"], a["B"], a["N"], a["Hq"],
                              a["Hkv"], a["D"], a["theta"], a["dtype"], None)

    assert rope(q=None) == jf.JF_ERR_INVALID_ARG
    assert rope(pl=None) == jf.JF_ERR_INVALID_ARG
    assert rope(D=127) == jf.JF_ERR_INVALID_ARG
    assert rope(D=0) == jf.JF_ERR_INVALID_ARG
    assert rope(Hkv=0) == jf.JF_ERR_INVALID_ARG
    assert rope(D=512) == jf.JF_ERR_UNSUPPORTED
    assert rope(dtype=5) == jf.JF_ERR_INVALID_ARG
    assert rope(q=FAKE_ODD) == jf.JF_ERR_ALIGN


def test_rmsnorm_argument_errors():
    L = jf.lib()
    assert L.jf_rmsnorm(None, 4, 64, 64, None, 1e-6, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_rmsnorm(FAKE, 0, 64, 64, None, 1e-6, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_rmsnorm(FAKE, 4, 64, 63, None, 1e-6, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_rmsnorm(FAKE, 4, 64, 64, None, -1.0, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_rmsnorm(FAKE, 4, 64, 80, None, 1e-6, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG  # in place, strided
    assert L.jf_rmsnorm(FAKE_ODD, 4, 64, 64, None, 1e-6, 1, FAKE, None) == jf.JF_ERR_ALIGN
    assert L.jf_rmsnorm(FAKE, 4, 64, 64, None, 1e-6, 9, FAKE, None) == jf.JF_ERR_INVALID_ARG


def test_swiglu_argument_errors():
    L = jf.lib()
    assert L.jf_swiglu(None, 4, 64, 128, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_swiglu(FAKE, 0, 64, 128, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_swiglu(FAKE, 4, 64, 127, 1, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_swiglu(FAKE, 4, 64, 128, 7, FAKE, None) == jf.JF_ERR_INVALID_ARG
    assert L.jf_swiglu(FAKE_ODD, 4, 64, 128, 1, FAKE, None) == jf.JF_ERR_ALIGN


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "tree_causal_draft_parent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "liboracle" not in src, f


def test_attn_plans_hold_whole_items_on_random_shapes():
    # host-side planner properties over seeded random batches: the workspace is
    # empty or whole work items (256 fp32 rows of 128 + an lse each), no more
    # items than the block units allow, at least one item a (sequence, KV
    # head, query tile) row; one compute unit never splits; repeated plans agree
    L = jf.lib()
    rng = np.random.default_rng(2024)
    per_item = _attn_ws_bytes(1)
    for _ in range(300):
        B = int(rng.integers(1, 65))
        N = int(rng.integers(1, 513))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        paged = bool(rng.integers(0, 2))
        pl = rng.integers(0, 20001, size=B).astype(np.int32)
        page = 16 if paged else max(int(pl.max()), 1)
        cus = int(rng.choice([0, 1, 8, 96, 112, 192, 256]))
        ws = _ws(L, B, N, Hq, Hkv, 128, page, pl, 1, cus=cus)
        assert ws == _ws(L, B, N, Hq, Hkv, 128, page, pl, 1, cus=cus)
        assert ws % per_item == 0
        rows = B * Hkv * -(-(N * (Hq // Hkv)) // 256)
        blocks = [-(-int(p) // 64) + -(-N // 64) for p in pl]
        units = Hkv * -(-(N * (Hq // Hkv)) // 256) * sum(blocks)
        items = ws // per_item
        if items:
            assert rows < items <= units
        if cus == 1:
            assert ws == 0


def test_fuse_plans_on_random_shapes():
    # the projection's split: no workspace, or split_k >= 2 slices of whole
    # 256/128/32-row x 128-column fp32 tiles; one compute unit never splits
    L = jf.lib()
    rng = np.random.default_rng(2025)
    for _ in range(300):
        M = int(rng.integers(1, 5000))
        H_in = 64 * int(rng.integers(1, 65))
        k = int(rng.integers(1, 5))
        H_out = int(rng.integers(1, 20000))
        cus = int(rng.choice([0, 1, 8, 96, 144, 192, 256]))
        ws = L.jf_fuse_proj_workspace_size_cus(M, H_in, k, H_out, 1, cus)
        bm = 256 if M >= 192 else (128 if M > 32 else 32)
        tile = bm * 128 * 4
        tiles = -(-M // bm) * -(-H_out // 128)
        assert ws % (tiles * tile) == 0
        s = ws // (tiles * tile)
        assert s == 0 or 2 <= s <= (k * H_in // 64) // 8
        if cus == 1:
            assert ws == 0
