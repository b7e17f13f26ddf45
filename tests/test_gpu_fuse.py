"""jf_fuse_proj vs the oracle (fp32 inputs: max-abs <= 1e-5; bf16 inputs with
fp32 accumulation: max-abs <= 2e-2 and rel-RMS <= 1e-2; bf16 outputs may also
differ from the exact value by the output's own rounding, one bf16 ulp)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, host_f64, say
from helpers import rel_rms
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _run(inp, out_dtype=torch.float32, ldx=None, rows=None, cus=0):
    dt = inp["dtype"]
    k, M, H_in = inp["x"].shape
    say(f"fuse: k={k} M={M} H_in={H_in} H_out={inp['w'].shape[0]} dtype={dt} out={out_dtype} ldx={ldx} cus={cus}")
    if ldx is not None:
        pad = np.zeros((k, M, ldx), dtype=inp["x"].dtype)
        pad[:, :, :H_in] = inp["x"]
        xt = dev_tensor(pad, dt)
        xs = [xt[l, :, :H_in] for l in range(k)]
    else:
        xt = dev_tensor(inp["x"], dt)
        xs = [xt[l] for l in range(k)]
    y = jf.jf_fuse_proj(xs, dev_tensor(inp["w"], dt), out_dtype=out_dtype, cus=cus)
    torch.cuda.synchronize()
    got = host_f64(y)
    ref = oracle.fuse_proj(synth.to_f64(inp["x"], dt), synth.to_f64(inp["w"], dt), rows=rows)
    if rows is not None:
        got = got[rows]
    if dt == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-5
    else:
        err = np.abs(got - ref)
        if out_dtype == torch.bfloat16:
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            assert np.all(err <= np.maximum(2e-2, ulp))
        else:
            assert err.max() <= 2e-2, err.max()
        assert rel_rms(got, ref) <= 1e-2


def test_tiny_fp32_workload():
    _run(synth.make_workload(0, parts=("fuse",))["fuse"])


@pytest.mark.parametrize("M,H_in,H_out", [(1, 64, 1), (200, 192, 130), (129, 128, 257)])
def test_bf16_ragged_tiles(M, H_in, H_out):
    _run(synth.make_fuse_inputs(M=M, H_in=H_in, H_out=H_out, n_fused=3, dtype="bf16", seed=M))


@pytest.mark.parametrize("M,H_in,H_out", [(200, 1024, 300), (100, 512, 257), (20, 1024, 130), (256, 2048, 4100)])
def test_split_k_ragged_tiles(M, H_in, H_out):
    # K split into slices over few tiles whose rows or columns run past M or
    # H_out (256-, 128- and 32-row tiles): the slices' partials cover whole
    # tiles, and the sum drops what lies outside the output; bf16 and fp32
    # outputs
    inp = synth.make_fuse_inputs(M=M, H_in=H_in, H_out=H_out, n_fused=3, dtype="bf16", seed=M + H_out)
    _run(inp)
    _run(inp, out_dtype=torch.bfloat16)


def test_bf16_out_and_strided_rows():
    inp = synth.make_fuse_inputs(M=70, H_in=256, H_out=300, n_fused=3, dtype="bf16", seed=2)
    _run(inp, out_dtype=torch.bfloat16)
    _run(inp, ldx=264)


def test_fp32_ragged():
    _run(synth.make_fuse_inputs(M=33, H_in=50, H_out=17, n_fused=2, dtype="f32", seed=4))


def test_qwen3_8b_low_budget_full():
    _run(synth.make_workload(1, parts=("fuse",))["fuse"])


def test_qwen3_8b_high_budget_full():
    # every row and column of the 256-node step's projection (8 K slices)
    _run(synth.make_workload(2, parts=("fuse",))["fuse"])


def test_serving_batch_shape_full():
    # 32 sequences x 64 nodes = 2048 rows, 3 x 4096 -> 4096 (8 x 32 tiles of
    # 256 x 128, no K split): every row and column
    _run(synth.make_workload(3, parts=("fuse",))["fuse"])


@pytest.mark.parametrize("cus", [192, 32, 5])
def test_split_planned_for_fewer_compute_units(cus):
    # jf_fuse_proj_cus: fewer K slices (192 units: 6, 32: 1, 5: 1), same
    # results to the parity bar, every row
    _run(synth.make_workload(2, parts=("fuse",))["fuse"], cus=cus)


@pytest.mark.parametrize("cus", [0, 144, 96])
def test_qwen3_30b_shape_full(cus):
    # 4 x 256 nodes = 1024 rows, 3 x 2048 -> 2048 (64 tiles): every row and
    # column, with the K split planned for all units (4 slices), for 144 (3)
    # and for 96 (none: the tiles fill more than half of them)
    _run(synth.make_workload(4, parts=("fuse",))["fuse"], cus=cus)


def test_context_rows_full():
    # one row per prefix token of a 4096-token prefix (plus a ragged 4-row tail):
    # the MFMA-bound shape, 17 x 32 tiles of 256 x 128 with no K split; every
    # row and column
    _run(synth.make_fuse_inputs(M=4100, H_in=4096, H_out=4096, n_fused=3, dtype="bf16", seed=1019))


def test_lm_head_shape_full():
    # the draft layer's LM head as the same call with one layer: 256 tree-node
    # rows x 4096 hidden -> 151936 vocabulary logits (1187 output tiles, no K
    # split, the last one ragged); every row and column (the oracle holds the
    # weights in float64, about 5 GB of host memory)
    inp = synth.make_fuse_inputs(M=256, H_in=4096, H_out=151936, n_fused=1, dtype="bf16", seed=2027)
    say("fuse: LM head 256 x 4096 -> 151936")
    xt = dev_tensor(inp["x"], "bf16")
    y = jf.jf_fuse_proj([xt[0]], dev_tensor(inp["w"], "bf16"), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = host_f64(y)
    del y, xt
    ref = oracle.fuse_proj(synth.to_f64(inp["x"], "bf16"), synth.to_f64(inp["w"], "bf16"))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(got - ref) <= np.maximum(2e-2, ulp))
    assert rel_rms(got, ref) <= 1e-2
