"""jf_node_topk vs the oracle: bit-exact indices and values, lse within the
fp32 / bf16 tolerances."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, say
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _check(bits, dtype, k, ld=None, rows=None):
    R, V = bits.shape
    x = synth.to_f64(bits, dtype)
    say(f"topk: R={R} V={V} k={k} dtype={dtype} ld={ld}")
    if ld is not None and ld != V:
        pad = np.zeros((R, ld), dtype=bits.dtype)
        pad[:, :V] = bits
        t = dev_tensor(pad, dtype)[:, :V]
    else:
        t = dev_tensor(bits, dtype)
    idx, val, lse = jf.jf_node_topk(t, k)
    torch.cuda.synchronize()
    idx, val, lse = idx.cpu().numpy(), val.cpu().numpy(), lse.cpu().numpy()
    sel = np.arange(R) if rows is None else rows
    oi, ov, ol = oracle.topk(x[sel], k)
    assert np.array_equal(idx[sel], oi)
    assert np.array_equal(val[sel].astype(np.float64), ov)
    fin = np.isfinite(ol)
    assert np.array_equal(np.isfinite(lse[sel]), fin)
    # lse is fp32 arithmetic over exactly widened inputs for both dtypes; the
    # stated bounds are 1e-5 (fp32 path) and 2e-2 (bf16 path) max-abs.
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert np.max(np.abs(lse[sel][fin] - ol[fin]), initial=0.0) <= tol


def test_tiny_fp32_workload():
    w = synth.workload(0)
    _check(synth.make_logits(R=w.B * w.N, V=w.V, dtype="f32", seed=1013), "f32", w.topk)


@pytest.mark.parametrize("k", [1, 8, 64])
def test_bf16_vocab_rows(k):
    _check(synth.make_logits(R=16, V=151936, dtype="bf16", seed=k), "bf16", k)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tie_forcing_rows(dtype):
    bits = synth.tie_forcing_logits(synth.make_logits(R=8, V=20000, dtype=dtype, seed=5), dtype)
    _check(bits, dtype, 8)
    _check(bits, dtype, 64)


@pytest.mark.parametrize("V,ld", [(1, 8), (7, 8), (1001, 1008), (4099, 4104), (513, 520)])
def test_ragged_vocab_and_stride(V, ld):
    bits = synth.make_logits(R=5, V=V, dtype="bf16", seed=V)
    _check(bits, "bf16", min(8, V), ld=ld)


def test_special_values():
    x = np.full((4, 3000), -np.inf, dtype=np.float32)
    x[1] = 2.5                             # all equal
    x[2, ::7] = 0.0
    x[2, 3::7] = -0.0                      # signed zeros, equal
    x[3, 100] = 1.0                        # one finite value among -inf
    _check(x, "f32", 8)
    _check(synth.f32_to_bf16_bits(x), "bf16", 8)


def test_qwen3_8b_high_budget_rows_full_size():
    w = synth.workload(2)
    bits = synth.make_logits(R=w.B * w.N, V=w.V, dtype="bf16", seed=1015)
    _check(bits, "bf16", w.topk)


def test_qwen3_30b_rows_full_size():
    # 4 x 256 nodes = 1024 rows of 151936 logits, every row
    w = synth.workload(4)
    _check(synth.make_logits(R=w.B * w.N, V=w.V, dtype="bf16", seed=1017), "bf16", w.topk)


def test_serving_batch_rows_full_size():
    # 32 sequences x 64 nodes = 2048 rows of 151936 logits, every row
    w = synth.workload(3)
    _check(synth.make_logits(R=w.B * w.N, V=w.V, dtype="bf16", seed=1016), "bf16", w.topk)


# 128 rows or more with at most 16 slices a row take the one-block-a-row path
# (slices merged in LDS); these cases cover it for both dtypes, k = 1 and 64,
# forced ties and a ragged vocabulary with a padded row stride.
@pytest.mark.parametrize("dtype,R,V,k", [("bf16", 128, 151936, 1), ("bf16", 128, 151936, 64),
                                         ("f32", 128, 50000, 8), ("bf16", 130, 4099, 8)])
def test_one_block_per_row_path(dtype, R, V, k):
    ld = V if V % 8 == 0 else (V + 7) // 8 * 8 + 8       # padded row stride for the ragged case
    bits = synth.make_logits(R=R, V=V, dtype=dtype, seed=R + V + k)
    _check(bits, dtype, k, ld=ld)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_block_per_row_ties(dtype):
    bits = synth.tie_forcing_logits(synth.make_logits(R=128, V=20000, dtype=dtype, seed=9), dtype)
    _check(bits, dtype, 8)


@pytest.mark.parametrize("dtype,V", [("bf16", 64 * 9728), ("f32", 64 * 4864)])
def test_largest_vocabulary_at_k64(dtype, V):
    # the call's limit ceil(V / S) * k <= 4096 with S = 9728 (bf16) / 4864
    # (fp32), reached exactly at k = 64; both merge paths (3 rows: per-slice
    # waves and a second pass)
    bits = synth.make_logits(R=3, V=V, dtype=dtype, seed=V)
    _check(bits, dtype, 64)


def test_beyond_largest_vocabulary_is_refused():
    t = torch.zeros((1, 64 * 9728 + 1), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(jf.JfError):
        jf.jf_node_topk(t, 64)


# k above 16: every lane is "hot", the k-th largest lane maximum leaves
# hundreds of survivors a slice, and the kernel raises the threshold from a
# histogram of the survivors' keys (bins 2^sh keys wide) before ranking them.
# These cases reach that step with one-key bins (bf16, normal logits), wider
# bins (fp32 keys; bf16 logits spread over several binades, values up to a
# few hundred), and k between the powers of two; the next test covers a row
# where no bin helps (all equal: the selection reads the slice again).
@pytest.mark.parametrize("dtype,R,k,wide", [("bf16", 128, 17, False), ("bf16", 128, 33, False),
                                            ("f32", 128, 64, False), ("bf16", 128, 64, True),
                                            ("bf16", 16, 40, True), ("f32", 16, 64, False)])
def test_large_k_threshold_refinement(dtype, R, k, wide):
    V = 151936 if dtype == "bf16" else 50000
    bits = synth.make_logits(R=R, V=V, dtype=dtype, seed=R * 100 + k)
    if wide:
        x = synth.bf16_bits_to_f32(bits)
        x = (np.sign(x) * np.exp2(np.abs(x) / 2)).astype(np.float32)
        bits = synth.f32_to_bf16_bits(x)
    _check(bits, dtype, k)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_k_all_equal_and_ties(dtype):
    x = np.random.default_rng(4).standard_normal((128, 30000)).astype(np.float32)
    x[0] = 1.5                                  # one value everywhere
    x[1, :] = -np.inf
    x[1, ::50] = 2.0                            # 600 equal finite values among -inf
    x[2] = np.rint(x[2] * 2)                    # a handful of distinct values
    bits = synth.f32_to_bf16_bits(x) if dtype == "bf16" else x
    _check(bits, dtype, 64)
