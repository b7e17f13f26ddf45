"""Pins of the oracle's RMS normalisation (CPU only): hand-derived golden rows
(tests/golden/rmsnorm_small.txt), constant rows, unit RMS at eps = 0, scale
invariance, and the weight as a per-column factor."""
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    d = {}
    for line in open(os.path.join(GOLD, name)):
        if line.startswith("#") or ":" not in line:
            continue
        key, vals = line.split(":", 1)
        d[key.strip()] = [float(t) for t in vals.split()]
    return d


def test_rmsnorm_golden():
    g = _read("rmsnorm_small.txt")
    ya = oracle.rmsnorm(np.array([g["a_x"]]), eps=0.0)
    assert np.max(np.abs(ya[0] - g["a_y"])) < 1e-11
    yb = oracle.rmsnorm(np.array([g["b_x"]]), w=np.array(g["b_w"]), eps=g["b_eps"][0])
    assert np.array_equal(yb[0], np.array(g["b_y"]))


def test_rmsnorm_constant_rows():
    c = np.array([[2.0] * 10, [-0.5] * 10])
    y = oracle.rmsnorm(c, eps=1e-6)
    assert np.max(np.abs(y - np.sign(c) * np.abs(c) / np.sqrt(c ** 2 + 1e-6))) < 1e-15


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = np.random.default_rng(1).standard_normal((7, 300))
    y = oracle.rmsnorm(x, eps=0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y ** 2, axis=1)) - 1.0)) < 1e-13
    assert np.max(np.abs(oracle.rmsnorm(37.5 * x, eps=0.0) - y)) < 1e-13


def test_rmsnorm_weight_scales_columns():
    x = np.random.default_rng(2).standard_normal((5, 64))
    w = np.random.default_rng(3).standard_normal(64)
    assert np.max(np.abs(oracle.rmsnorm(x, w=w) - oracle.rmsnorm(x) * w)) < 1e-14


# ---------------------------------------------------------------------------
# Gated MLP activation

def test_swiglu_golden():
    g = _read("swiglu_small.txt")
    y = oracle.swiglu(np.array([g["gu"]]))
    assert np.max(np.abs(y[0] - np.array(g["y"]))) < 1e-11


def test_swiglu_odd_part_and_limits():
    rng = np.random.default_rng(4)
    g = rng.standard_normal((6, 50)) * 3
    ones = np.ones_like(g)
    sp = oracle.swiglu(np.concatenate([g, ones], axis=1))
    sm = oracle.swiglu(np.concatenate([-g, ones], axis=1))
    assert np.max(np.abs(sp - sm - g)) < 1e-13                # silu(g) - silu(-g) = g
    big = oracle.swiglu(np.array([[40.0, -40.0, 0.0, 3.0, 5.0, 9.0]]))
    assert abs(big[0, 0] - 120.0) < 1e-12 and abs(big[0, 1]) < 1e-14 and big[0, 2] == 0.0


def test_swiglu_matches_tanh_form():
    # logistic(g) = (1 + tanh(g / 2)) / 2, an independent formulation
    rng = np.random.default_rng(5)
    g, u = rng.standard_normal((4, 30)) * 4, rng.standard_normal((4, 30))
    ref = g * (1.0 + np.tanh(g / 2.0)) / 2.0 * u
    assert np.max(np.abs(oracle.swiglu(np.concatenate([g, u], axis=1)) - ref)) < 1e-13
