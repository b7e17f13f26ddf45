"""The seeded generators: determinism, shapes, bf16 rounding, tree statistics."""
import numpy as np
import pytest
import torch

from tree_causal_draft_parent_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                  np.inf, -np.inf, 3.4e38], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("N,depth,br", [(16, 5, (1, 3)), (16, 8, (1, 4)), (256, 16, (1, 8)), (64, 16, (1, 8))])
def test_best_first_tree_shape(N, depth, br):
    rng = np.random.default_rng(N)
    for _ in range(5):
        par = synth.best_first_tree(rng, N, depth, br)
        assert par.shape == (N,)
        assert np.all(par < np.arange(N))
        d = np.zeros(N, int)
        for i in range(N):
            d[i] = 1 if par[i] < 0 else d[par[i]] + 1
        assert d.max() <= depth
        kids = np.bincount(par[par >= 0], minlength=N)
        assert kids.max() <= br[1]


def test_workloads_deterministic_and_shaped():
    a = synth.make_workload(0)
    b = synth.make_workload(0)
    for key in ("q", "k_cache", "parent", "block_table"):
        assert np.array_equal(a["attn"][key], b["attn"][key])
    assert a["attn"]["q"].shape == (1, 16, 4, 64)
    assert a["fuse"]["x"].shape == (3, 16, 256) and a["fuse"]["w"].shape == (256, 768)
    assert a["logits"].shape == (16, 1000)
    p3 = synth.prefix_lengths(3)
    assert p3.shape == (32,) and p3.min() >= 512 and p3.max() <= 8192


def test_paged_layout_is_a_permutation():
    inp = synth.make_attn_inputs(B=5, N=4, Hq=2, Hkv=1, D=8, dtype="bf16",
                                 prefix_lens=[1, 16, 17, 0, 40], page_size=16,
                                 shuffled_pages=True, seed=1)
    bt = inp["block_table"]
    used = bt[bt >= 0]
    assert sorted(used.tolist()) == list(range(inp["num_pages"]))
    assert list((bt >= 0).sum(axis=1)) == [1, 1, 2, 0, 3]
