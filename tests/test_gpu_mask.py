"""jf_tree_mask_build vs the oracle: bit-exact masks, depths and tree status."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, say
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _run(parent: np.ndarray):
    say(f"mask: B={parent.shape[0]} N={parent.shape[1]}")
    m, d, s = jf.jf_tree_mask_build(dev_tensor(parent))
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint64), d.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("N", [1, 16, 63, 64, 65, 256, 1000, 4096])
def test_random_forests(N):
    rng = np.random.default_rng(N)
    B = 3
    par = np.stack([synth.best_first_tree(rng, N, 16, (1, 8)) for _ in range(B)]).astype(np.int32)
    mask, depth, st = _run(par)
    om, od, ost, _ = oracle.tree_mask(par)
    assert ost == oracle.OK
    assert np.array_equal(mask, om)
    assert np.array_equal(depth, od)
    assert np.all(st == -1)


@pytest.mark.parametrize("kind", ["chain", "star", "unordered"])
def test_shapes(kind):
    N = 200
    if kind == "chain":
        par = synth.chain_tree(N)[None]
    elif kind == "star":
        par = synth.star_tree(N)[None]
    else:
        rng = np.random.default_rng(3)
        base = synth.best_first_tree(rng, N, 16, (1, 8))
        perm = rng.permutation(N)           # new id of old node j is perm[j]
        inv = np.argsort(perm)
        par = np.array([[perm[base[inv[n]]] if base[inv[n]] >= 0 else -1 for n in range(N)]], np.int32)
    mask, depth, st = _run(par.astype(np.int32))
    om, od, _, _ = oracle.tree_mask(par)
    assert np.array_equal(mask, om) and np.array_equal(depth, od) and st[0] == -1


def test_bad_trees_are_reported_per_sequence():
    par = np.array([[-1, 0, 1, 2],      # fine
                    [-1, 2, 1, 0],      # 1 <-> 2 cycle
                    [-1, 0, 9, 1],      # out of range at node 2
                    [3, -1, 1, 3]],     # self-parent at node 3 (node 0 hangs below it)
                   np.int32)
    mask, depth, st = _run(par)
    assert list(st) == [-1, 1, 2, 0]
    for b in range(4):
        om, od, ost, bad = oracle.tree_mask(par[b:b + 1])
        assert (bad == -1) == (st[b] == -1)
        if bad >= 0:
            assert bad == st[b]
        ok_rows = od[0] > 0
        assert np.array_equal(depth[b], od[0])
        assert np.array_equal(mask[b][ok_rows], om[0][ok_rows])
        assert np.all(mask[b][~ok_rows] == 0)


@pytest.mark.parametrize("counts", [[16, 64, 256, 1, 100], [4096, 3], [65] * 40])
def test_packed_trees_of_different_sizes(counts):
    rng = np.random.default_rng(len(counts))
    par = np.concatenate([synth.best_first_tree(rng, n, 16, (1, 8)) for n in counts]).astype(np.int32)
    no = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    say(f"mask packed: counts={counts[:6]} T={no[-1]}")
    m, d, s = jf.jf_tree_mask_build(dev_tensor(par), node_off=no)
    torch.cuda.synchronize()
    om, od, ost, _ = oracle.tree_mask(par, node_off=no)
    assert ost == oracle.OK
    assert np.array_equal(m.cpu().numpy().view(np.uint64), om)
    assert np.array_equal(d.cpu().numpy(), od)
    assert np.all(s.cpu().numpy() == -1)


def test_packed_bad_tree_reports_local_index():
    # sequence 1 (rows 2..4): node 1's parent 5 is out of its range [-1, 3)
    par = np.array([-1, 0, -1, 5, 0], np.int32)
    m, d, s = jf.jf_tree_mask_build(dev_tensor(par), node_off=np.array([0, 2, 5]))
    torch.cuda.synchronize()
    assert list(s.cpu().numpy()) == [-1, 1]
    om, od, ost, bad = oracle.tree_mask(par, node_off=np.array([0, 2, 5]))
    assert ost == oracle.BAD_TREE and bad == 3
    ok = od > 0
    assert np.array_equal(m.cpu().numpy().view(np.uint64)[ok], om[ok])
    assert np.array_equal(d.cpu().numpy(), od)
