"""Pins of the oracle's ancestor-mask builder (CPU only)."""
import os

import numpy as np
import pytest

import oracle
from tree_causal_draft_parent_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_mask_golden(name):
    rows = []
    parent = None
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("parent:"):
            parent = np.array([int(t) for t in line.split()[1:]], dtype=np.int32)
            continue
        node, par, depth, bits = line.split()
        rows.append((int(node), int(par), int(depth), bits))
    return parent, rows


def _bits(mask_row, N):
    return "".join("1" if (int(mask_row[j // 64]) >> (j % 64)) & 1 else "0" for j in range(N))


@pytest.mark.parametrize("name", ["mask_tree7.txt", "mask_unordered3.txt"])
def test_golden_trees(name):
    parent, rows = _read_mask_golden(name)
    N = parent.shape[0]
    mask, depth, st, bad = oracle.tree_mask(parent[None])
    assert st == oracle.OK and bad == -1
    for node, par, d, bits in rows:
        assert parent[node] == par
        assert depth[0, node] == d
        assert _bits(mask[0, node], N) == bits


@pytest.mark.parametrize("N", [1, 5, 64, 65, 200])
def test_chain_is_lower_triangular(N):
    mask, depth, st, _ = oracle.tree_mask(synth.chain_tree(N)[None])
    assert st == oracle.OK
    dense = np.array([[int(_bits(mask[0, i], N)[j]) for j in range(N)] for i in range(N)])
    assert np.array_equal(dense, np.tril(np.ones((N, N), dtype=int)))
    assert np.array_equal(depth[0], np.arange(1, N + 1))


@pytest.mark.parametrize("N", [1, 63, 64, 130])
def test_star_is_identity(N):
    mask, depth, st, _ = oracle.tree_mask(synth.star_tree(N)[None])
    assert st == oracle.OK
    dense = np.array([[int(_bits(mask[0, i], N)[j]) for j in range(N)] for i in range(N)])
    assert np.array_equal(dense, np.eye(N, dtype=int))
    assert np.all(depth == 1)


@pytest.mark.parametrize("seed", range(6))
def test_recursion_and_popcount(seed):
    rng = np.random.default_rng(seed)
    B, N = 3, int(rng.integers(1, 300))
    par = np.stack([synth.best_first_tree(rng, N, 16, (1, 8)) for _ in range(B)])
    mask, depth, st, _ = oracle.tree_mask(par)
    assert st == oracle.OK
    W = (N + 63) // 64
    for b in range(B):
        for i in range(N):
            row = mask[b, i]
            pc = sum(bin(int(w)).count("1") for w in row)
            assert pc == depth[b, i]
            assert (int(row[i // 64]) >> (i % 64)) & 1
            p = par[b, i]
            expect = np.zeros(W, dtype=np.uint64) if p < 0 else mask[b, p].copy()
            expect[i // 64] |= np.uint64(1) << np.uint64(i % 64)
            assert np.array_equal(row, expect)
    # padding bits beyond N stay clear
    if N % 64:
        assert np.all((mask[:, :, -1] >> np.uint64(N % 64)) == 0)


def test_bad_trees():
    # self-parent
    _, _, st, bad = oracle.tree_mask(np.array([[-1, 1, 0]], np.int32))
    assert st == oracle.BAD_TREE and bad == 1
    # two-cycle reachable from a later node; the smallest bad row is reported
    _, _, st, bad = oracle.tree_mask(np.array([[-1, 3, 1, 2, 0]], np.int32))
    assert st == oracle.BAD_TREE and bad == 1
    # out of range parent, in the second sequence
    par = np.array([[-1, 0, 1], [-1, 7, 0]], np.int32)
    _, _, st, bad = oracle.tree_mask(par)
    assert st == oracle.BAD_TREE and bad == 3 + 1
    # below -1
    _, _, st, bad = oracle.tree_mask(np.array([[-1, -2]], np.int32))
    assert st == oracle.BAD_TREE and bad == 1
    # a node whose ancestor is bad is bad too
    _, _, st, bad = oracle.tree_mask(np.array([[5, 0, -1]], np.int32))
    assert st == oracle.BAD_TREE and bad == 0
