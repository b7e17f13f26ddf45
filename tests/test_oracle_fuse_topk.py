"""Pins of the oracle's fused projection and top-k (CPU only)."""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from tree_causal_draft_parent_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("k,M,H_in,H_out", [(3, 5, 16, 7), (1, 1, 3, 2), (3, 33, 64, 40)])
def test_fuse_is_matmul_of_concatenation(k, M, H_in, H_out):
    inp = synth.make_fuse_inputs(M=M, H_in=H_in, H_out=H_out, n_fused=k, dtype="bf16", seed=k + M)
    x = synth.to_f64(inp["x"], "bf16")
    w = synth.to_f64(inp["w"], "bf16")
    y = oracle.fuse_proj(x, w)
    cat = np.concatenate(list(x), axis=1)   # [M, k*H_in], layer l at columns l*H_in..
    ref = np.matmul(cat, w.T)
    assert np.max(np.abs(y - ref)) < 1e-12
    rows = np.array([M - 1, 0])
    assert np.max(np.abs(oracle.fuse_proj(x, w, rows=rows) - ref[rows])) < 1e-12


def test_fuse_identity_selects_each_layer():
    M, H = 4, 6
    x = synth.to_f64(synth.make_fuse_inputs(M=M, H_in=H, H_out=H, n_fused=3, dtype="f32")["x"], "f32")
    for l in range(3):
        w = np.zeros((H, 3 * H))
        w[:, l * H:(l + 1) * H] = np.eye(H)
        assert np.array_equal(oracle.fuse_proj(x, w), x[l])


def _lexsort_topk(x, k):
    xc = np.where(x == 0, 0.0, x)   # -0 and +0 compare equal
    order = np.lexsort((np.arange(x.shape[0]), -xc))
    return order[:k]


def test_golden_row():
    lines = [l for l in open(os.path.join(GOLD, "topk_row.txt")) if not l.startswith("#")]
    x = np.array([float(t) for t in lines[0].split()[1:]])
    exp_idx = [int(t) for t in lines[1].split()[1:]]
    for k in range(1, 9):
        idx, val, lse = oracle.topk(x[None], k)
        assert list(idx[0]) == exp_idx[:k]
        assert np.array_equal(val[0], x[exp_idx[:k]])
    ref = math.log(math.exp(7) + 2 * math.exp(5) + 2 * math.exp(3) + 2)
    assert abs(lse[0] - ref) < 1e-13


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k", [1, 4, 8, 64])
def test_topk_matches_lexsort(dtype, k):
    R, V = 6, 3000
    bits = synth.make_logits(R=R, V=V, dtype=dtype, seed=k)
    if k == 8:
        bits = synth.tie_forcing_logits(bits, dtype)
    x = synth.to_f64(bits, dtype)
    idx, val, lse = oracle.topk(x, k)
    for r in range(R):
        ref = _lexsort_topk(x[r], k)
        assert np.array_equal(idx[r], ref)
        assert np.array_equal(val[r], x[r, ref])
    assert np.max(np.abs(lse - scipy.special.logsumexp(x, axis=1))) < 1e-12


def test_topk_degenerate_rows():
    x = np.full((2, 50), 1.5)
    x[1] = -np.inf
    idx, val, lse = oracle.topk(x, 10)
    assert np.array_equal(idx[0], np.arange(10)) and np.array_equal(idx[1], np.arange(10))
    assert lse[1] == -np.inf
    assert abs(lse[0] - (1.5 + math.log(50))) < 1e-13
    # k == V returns the full order
    y = np.array([[0.0, -0.0, 2.0, -1.0]])
    idx, val, _ = oracle.topk(y, 4)
    assert list(idx[0]) == [2, 0, 1, 3]
