"""Pins of the oracle's rotary embedding at tree positions (CPU only).

A hand-derived rotation (tests/golden/rope_d4.txt); position 0 is the
identity; each pair keeps its norm; rotations compose by adding positions;
the score between a rotated query and key depends only on the difference of
their positions; a chain of nodes sits at the prefix length, +1, +2, ..."""
import os

import numpy as np
import pytest

import oracle
from tree_causal_draft_parent_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    d = {}
    for line in open(os.path.join(GOLD, name)):
        if line.startswith("#") or ":" not in line:
            continue
        key, vals = line.split(":", 1)
        d[key.strip()] = vals.split()
    return d


def test_rope_golden():
    g = _read("rope_d4.txt")
    x = np.array([float(t) for t in g["x"]]).reshape(1, 1, 1, 4)
    out = oracle.tree_rope(x, np.array([[int(g["depth"][0])]]), [int(g["prefix_len"][0])],
                           theta=float(g["theta"][0]))
    assert np.max(np.abs(out.ravel() - np.array([float(t) for t in g["out"]]))) < 1e-10


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rope_position_zero_is_identity_and_depth_zero_untouched():
    x = _rand((2, 3, 4, 64), 1)
    out = oracle.tree_rope(x, np.array([[1, 1, 0], [1, 0, 1]]), [0, 0])
    assert np.array_equal(out, x)


def test_rope_keeps_pair_norms():
    x = _rand((1, 5, 3, 128), 2)
    out = oracle.tree_rope(x, np.array([[1, 2, 3, 4, 5]]), [4093])
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = out[..., :64] ** 2 + out[..., 64:] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12


def test_rope_composes_by_adding_positions():
    x = _rand((1, 1, 2, 128), 3)
    once = oracle.tree_rope(x, np.array([[1]]), [700])                 # position 700
    twice = oracle.tree_rope(oracle.tree_rope(x, np.array([[1]]), [300]), np.array([[1]]), [400])
    assert np.max(np.abs(once - twice)) < 1e-9


@pytest.mark.parametrize("shift", [1, 37, 4096])
def test_rope_scores_depend_on_position_difference(shift):
    q = _rand((1, 1, 1, 128), 4)
    k = _rand((1, 1, 1, 128), 5)
    d = np.array([[1]])
    s0 = np.sum(oracle.tree_rope(q, d, [120]) * oracle.tree_rope(k, d, [100]))
    s1 = np.sum(oracle.tree_rope(q, d, [120 + shift]) * oracle.tree_rope(k, d, [100 + shift]))
    assert abs(s0 - s1) < 1e-9


def test_rope_chain_positions_follow_the_prefix():
    # node i of a chain has depth i + 1, so it sits at P + i: the same as a
    # single node of depth 1 under a prefix of P + i tokens
    N, P = 6, 50
    x = _rand((1, N, 2, 64), 6)
    par = synth.chain_tree(N)[None]
    _, depth, _, _ = oracle.tree_mask(par)
    out = oracle.tree_rope(x, depth, [P])
    for i in range(N):
        one = oracle.tree_rope(x[:, i:i + 1], np.array([[1]]), [P + i])
        assert np.max(np.abs(out[:, i:i + 1] - one)) < 1e-12
