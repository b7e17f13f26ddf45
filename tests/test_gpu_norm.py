"""jf_rmsnorm vs the oracle (fp32: max-abs <= 1e-5; bf16 storage: each element
within max(2e-2, one bf16 ulp of the reference) and rel-RMS <= 1e-2)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, host_f64, say
from helpers import rel_rms
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _draw(shape, dtype, seed, std=1.0):
    x = (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _check(got, ref, dtype):
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-5, err.max()
    else:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(err <= np.maximum(2e-2, ulp))
        assert rel_rms(got, ref) <= 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,H,weight", [(256, 4096, True), (7, 4096, False),
                                           (256 * 40, 128, True), (33, 100, True)])
def test_rows(dtype, rows, H, weight):
    say(f"rmsnorm: rows={rows} H={H} {dtype} weight={weight}")
    x = _draw((rows, H), dtype, rows + H, std=3.0)
    w = _draw((H,), dtype, H + 1) if weight else None
    y = jf.jf_rmsnorm(dev_tensor(x, dtype), None if w is None else dev_tensor(w, dtype), eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(synth.to_f64(x, dtype), None if w is None else synth.to_f64(w, dtype), 1e-6)
    _check(host_f64(y), ref, dtype)


def test_strided_rows_and_in_place():
    say("rmsnorm: strided rows, then in place")
    x = _draw((40, 264), "bf16", 9)
    xt = dev_tensor(x, "bf16")
    y = jf.jf_rmsnorm(xt[:, :256], eps=1e-5)                 # row stride 264
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(synth.to_f64(x[:, :256], "bf16"), None, 1e-5)
    _check(host_f64(y), ref, "bf16")
    xd = dev_tensor(np.ascontiguousarray(x[:, :256]), "bf16")
    jf.jf_rmsnorm(xd, eps=1e-5, y=xd)                        # in place
    torch.cuda.synchronize()
    _check(host_f64(xd), ref, "bf16")


def test_zero_rows_with_eps():
    x = np.zeros((4, 128), np.float32)
    y = jf.jf_rmsnorm(dev_tensor(x, "f32"), eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), x)


# ---------------------------------------------------------------------------
# Gated MLP activation

@pytest.mark.parametrize("dtype,M,I,ld", [("f32", 33, 100, None), ("f32", 5, 37, None),
                                          ("bf16", 256, 12288, None), ("bf16", 9, 64, 136),
                                          ("bf16", 3, 30, None)])
def test_swiglu(dtype, M, I, ld):
    say(f"swiglu: M={M} I={I} ld={ld} {dtype}")
    gu = _draw((M, 2 * I), dtype, M * I, std=3.0)
    if ld is not None:
        pad = np.zeros((M, ld), dtype=gu.dtype)
        pad[:, :2 * I] = gu
        t = dev_tensor(pad, dtype)[:, :2 * I]
    else:
        t = dev_tensor(gu, dtype)
    y = jf.jf_swiglu(t)
    torch.cuda.synchronize()
    _check(host_f64(y), oracle.swiglu(synth.to_f64(gu, dtype)), dtype)


def test_swiglu_extremes():
    g = np.array([[100.0, -100.0, 0.0, -0.0, 1e-30, 88.0, -88.0, 20.0]], np.float32)
    u = np.array([[1.0, 1.0, 5.0, 5.0, 1.0, 0.5, 2.0, -1.0]], np.float32)
    gu = np.concatenate([g, u], axis=1)
    y = jf.jf_swiglu(dev_tensor(gu, "f32"))
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref = oracle.swiglu(gu.astype(np.float64))
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) <= 1e-5
