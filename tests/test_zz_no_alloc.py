"""jf_node_topk_noalloc (no workspace, static per-GPU scratch) against
jf_node_topk on the same logits: two calls in a row, the second smaller,
with indices, values and normalisers identical bit for bit.  Both calls take
the per-slice path (fewer than 128 rows), whose kernels keep their partial
results in the scratch.  Called through the C ABI (the binding only
marshals arguments)."""
import numpy as np
import pytest
import torch

from gpu_util import dev_tensor, say
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _both(logits, k, with_lse):
    R = logits.shape[0]
    ref = jf.jf_node_topk(logits, k, with_lse=with_lse)
    idx = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((R, k), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    got = jf.jf_node_topk_noalloc(logits, k, idx, val, lse)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_topk_matches_topk_twice(dtype):
    cases = [(96, 151936, 8, True), (16, 50000, 4, False)] if dtype == "bf16" else \
        [(64, 100000, 16, True), (8, 3000, 3, True)]
    for seed, (R, V, k, with_lse) in enumerate(cases):
        need = jf.jf_node_topk_workspace_size(R, V, k)
        say(f"noalloc top-k: {dtype} R={R} V={V} k={k} lse={with_lse} workspace={need}")
        assert 0 < need <= jf.NODE_TOPK_SCRATCH_BYTES
        logits = dev_tensor(synth.make_logits(R=R, V=V, dtype=dtype, seed=300 + seed), dtype)
        ref, got = _both(logits, k, with_lse)
        assert torch.equal(got[0], ref[0])
        assert np.array_equal(got[1].cpu().numpy().view(np.uint32), ref[1].cpu().numpy().view(np.uint32))
        if with_lse:
            assert np.array_equal(got[2].cpu().numpy().view(np.uint32),
                                  ref[2].cpu().numpy().view(np.uint32))


def test_noalloc_topk_refuses_sizes_beyond_the_scratch():
    # 1024 rows x k = 64 over 622,592 entries needs more than the scratch holds
    R, V, k = 1024, 622592, 64
    assert jf.jf_node_topk_workspace_size(R, V, k) > jf.NODE_TOPK_SCRATCH_BYTES
    logits = torch.zeros((R, V), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    val = torch.empty((R, k), dtype=torch.float32, device="cuda")
    with pytest.raises(jf.JfError) as e:
        jf.jf_node_topk_noalloc(logits, k, idx, val)
    assert e.value.status == jf.JF_ERR_WORKSPACE
