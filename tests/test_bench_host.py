"""bench.py's host-side arithmetic on a machine without a GPU: algorithmic
bytes and flops of the tree attention on a hand-counted case, the roofline
bound from arithmetic intensity, and the freshness rule of the recorded HBM
traffic (a record counts only while the call's kernel sources are unchanged)."""
import json

import numpy as np
import pytest

import bench
from tree_causal_draft_parent_amd import profsum


def _tiny(node_off=None):
    # one sequence of 2 nodes (node 1 under node 0: depths 1 and 2) over a
    # 3-token prefix
    a = {"prefix_len": np.array([3], np.int32), "parent": np.array([[-1, 0]], np.int32)}
    if node_off is not None:
        a["parent"] = np.array([-1, 0], np.int32)
        a["node_off"] = np.array(node_off, np.int32)
    return a


def test_attention_algorithmic_counts_by_hand():
    # Hq = 2, Hkv = 1, D = 4, bf16 (2 bytes):
    #   visible (node, key) pairs = 2 nodes x 3 prefix keys + depths 1 + 2 = 9
    #   flops = 4 * Hq * D * 9 = 288 (two products of D per head and pair)
    #   bytes = q 2*2*4*2 + tree K/V 2*2*1*4*2 + prefix K/V 2*3*1*4*2
    #         + mask 2 rows * 1 word * 8 + out 2*2*4*2 + lse 2*2*4
    #         = 32 + 32 + 48 + 16 + 32 + 16 = 176
    alg = bench.attn_algorithmic(_tiny(), Hq=2, Hkv=1, D=4)
    assert alg == {"bytes": 176, "flops": 288, "prefix_kv_bytes": 48}
    # the same tree given as a packed batch of one
    assert bench.attn_algorithmic(_tiny([0, 2]), Hq=2, Hkv=1, D=4) == alg
    # an FP8 prefix cache halves only the prefix bytes
    fp8 = bench.attn_algorithmic(_tiny(), Hq=2, Hkv=1, D=4, kv_e=1)
    assert fp8 == {"bytes": 176 - 24, "flops": 288, "prefix_kv_bytes": 24}


def test_bound_follows_the_ridge():
    assert bench.RIDGE == pytest.approx(312.5)
    assert bench.bound_of(313.0 * 1000, 1000) == "mfma"
    assert bench.bound_of(312.0 * 1000, 1000) == "hbm"
    assert bench.bound_of(0, 1000) == "hbm"
    # 8 GB in 1 ms is the HBM peak; 2.5 PFLOP over 1 GB in 1 s is the MFMA peak
    gbs, tfs, b, frac = bench.roof_numbers({"bytes": 8e9, "flops": 0}, 1.0)
    assert (b, frac) == ("hbm", pytest.approx(1.0)) and gbs == pytest.approx(8000.0)
    gbs, tfs, b, frac = bench.roof_numbers({"bytes": 1e9, "flops": 2.5e15}, 1000.0)
    assert (b, frac) == ("mfma", pytest.approx(1.0)) and tfs == pytest.approx(2500.0)


def test_recorded_traffic_counts_only_for_unchanged_sources(tmp_path, monkeypatch):
    cur = profsum.file_hashes()
    rec = {"workload": "w", "file_sha256": dict(cur),
           "kernels": {"k_fuse_gemm_bf16<256>": {"fetch_bytes": 100, "write_bytes": 20},
                       "k_fuse_reduce<256>": {"fetch_bytes": 30, "write_bytes": 4},
                       "k_topk_stage1<unsigned short, true, 16, true>": {"fetch_bytes": 7, "write_bytes": 1}}}
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    path.write_text(json.dumps(rec))
    total, src = bench.measured_traffic("fuse", "w")
    assert total == 154 and "k_fuse.hip sha256" in src      # the call's kernels only
    assert bench.measured_traffic("fuse", "other")[0] is None
    assert bench.measured_traffic("attn", "w")[0] is None   # no counters for its kernels
    # a changed kernel source of the call, or of the shared header, voids it
    for fn in ("k_fuse.hip", "jf_internal.h"):
        stale = dict(rec, file_sha256=dict(cur, **{fn: "0" * 64}))
        path.write_text(json.dumps(stale))
        total, why = bench.measured_traffic("fuse", "w")
        assert total is None and "changed" in why
    # another call's source changing leaves it valid
    path.write_text(json.dumps(dict(rec, file_sha256=dict(cur, **{"k_attn.hip": "0" * 64}))))
    assert bench.measured_traffic("fuse", "w")[0] == 154
