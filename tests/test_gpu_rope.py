"""jf_tree_rope vs the oracle (fp32: max-abs <= 1e-5; bf16 storage: each
element within max(2e-2, one bf16 ulp of the reference) and rel-RMS <= 1e-2,
the bf16 bar of the other calls).  Positions come from depths that each side
computes itself (jf_tree_mask_build on the GPU, the oracle's mask on the host)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, host_f64, say
from helpers import rel_rms
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _draw(shape, dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _run(parent, prefix, Hq, Hkv, D, dtype, seed, with_k=True, theta=0.0):
    B, N = parent.shape
    say(f"rope: B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} {dtype} k={with_k} P={list(prefix)[:4]}")
    q = _draw((B, N, Hq, D), dtype, seed)
    k = _draw((B, N, Hkv, D), dtype, seed + 1)
    _, dg, _ = jf.jf_tree_mask_build(dev_tensor(parent.astype(np.int32)))
    qd, kd = dev_tensor(q, dtype), dev_tensor(k, dtype) if with_k else None
    jf.jf_tree_rope(qd, kd, dg, dev_tensor(np.asarray(prefix, np.int32)), theta=theta)
    torch.cuda.synchronize()
    _, depth, _, _ = oracle.tree_mask(parent)
    th = 1e6 if theta <= 0 else theta
    pairs = [(qd, q)] + ([(kd, k)] if with_k else [])
    for got_t, x in pairs:
        got = host_f64(got_t)
        ref = oracle.tree_rope(synth.to_f64(x, dtype), depth, prefix, theta=th)
        err = np.abs(got - ref)
        if dtype == "f32":
            assert err.max() <= 1e-5, err.max()
        else:
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            assert np.all(err <= np.maximum(2e-2, ulp))
            assert rel_rms(got, ref) <= 1e-2
    if not with_k:
        assert kd is None


def _trees(B, N, max_depth, branching, seed):
    rng = np.random.default_rng(seed)
    return np.stack([synth.best_first_tree(rng, N, max_depth, branching) for _ in range(B)])


def test_tiny_fp32():
    _run(_trees(1, 16, 5, (1, 3), 1), [64], 4, 2, 64, "f32", 1)


def test_fp32_long_positions():
    # positions up to 32768 + 15: the angles must be formed in fp64
    _run(_trees(2, 256, 16, (1, 8), 2), [32768, 1], 4, 2, 128, "f32", 2)


def test_qwen3_8b_high_budget_bf16():
    _run(_trees(1, 256, 16, (1, 8), 3), [4096], 32, 8, 128, "bf16", 3)


def test_serving_batch_ragged_bf16():
    rng = np.random.default_rng(4)
    _run(_trees(32, 64, 16, (1, 8), 4), list(rng.integers(512, 8193, size=32)), 32, 8, 128, "bf16", 4)


def test_qwen3_30b_shape_bf16_queries_only():
    _run(_trees(4, 256, 16, (1, 8), 5), [32768] * 4, 32, 4, 128, "bf16", 5, with_k=False)


@pytest.mark.parametrize("D", [2, 256])
def test_head_dim_edges_and_theta(D):
    _run(_trees(1, 40, 16, (1, 8), 6), [1000], 3, 1, D, "f32", 6, theta=10000.0)


def test_bad_rows_are_unchanged():
    par = np.array([[-1, 2, 1, 0]], np.int32)          # nodes 1 and 2 form a cycle
    _run(par, [10], 2, 1, 64, "f32", 7)


def test_unaligned_rows_take_the_scalar_path():
    # q starting 4 bytes into an allocation: the 16-byte path is not taken
    B, N, Hq, D = 1, 24, 3, 64
    par = _trees(B, N, 16, (1, 8), 8)
    q = _draw((B, N, Hq, D), "f32", 8)
    buf = torch.zeros(B * N * Hq * D + 1, dtype=torch.float32, device="cuda")
    qd = buf[1:].view(B, N, Hq, D)
    qd.copy_(torch.from_numpy(q).cuda())
    _, dg, _ = jf.jf_tree_mask_build(dev_tensor(par.astype(np.int32)))
    say("rope: unaligned q")
    jf.jf_tree_rope(qd, None, dg, dev_tensor(np.array([300], np.int32)))
    torch.cuda.synchronize()
    _, depth, _, _ = oracle.tree_mask(par)
    ref = oracle.tree_rope(q.astype(np.float64), depth, [300])
    assert np.max(np.abs(host_f64(qd) - ref)) <= 1e-5
