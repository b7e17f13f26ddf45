"""jf_path_scores and jf_tree_expand vs the oracle, bit for bit.

Path scores: the kernel sums in fp64 in the oracle's order (node, then each
parent up to the prefix) and rounds once, so it must equal the oracle's fp64
score rounded to fp32 exactly.  Expansion: the candidate scores are the same
two fp32 roundings on both sides and the selection is a total order, so the
new parents, tokens, scores (as bit patterns) and depths must all be equal.
Inputs come from the seeded generators only; none from the GPU path."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev_tensor, say
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def _path(parent: np.ndarray, logp: np.ndarray):
    say(f"path_scores: B={parent.shape[0]} N={parent.shape[1]}")
    s, st = jf.jf_path_scores(dev_tensor(parent.astype(np.int32)), dev_tensor(logp.astype(np.float32)))
    torch.cuda.synchronize()
    return s.cpu().numpy(), st.cpu().numpy()


def _expect_path(parent, logp):
    score, st, bad = oracle.path_scores(parent, logp.astype(np.float32).astype(np.float64))
    return score.astype(np.float32), st, bad


@pytest.mark.parametrize("N", [1, 16, 64, 65, 256, 1000, 4096])
def test_path_random_forests(N):
    inp = synth.make_path_inputs(B=3, N=N, seed=N)
    got, st = _path(inp["parent"], inp["logp"])
    want, ost, _ = _expect_path(inp["parent"], inp["logp"])
    assert ost == oracle.OK and np.all(st == -1)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("kind", ["chain", "star", "unordered"])
def test_path_shapes(kind):
    N = 300
    rng = np.random.default_rng(11)
    if kind == "chain":
        par = synth.chain_tree(N)
    elif kind == "star":
        par = synth.star_tree(N)
    else:
        base = synth.best_first_tree(rng, N, 16, (1, 8))
        perm = rng.permutation(N)
        inv = np.argsort(perm)
        par = np.array([perm[base[inv[n]]] if base[inv[n]] >= 0 else -1 for n in range(N)])
    par = par.astype(np.int32)[None]
    lp = (-np.abs(rng.standard_normal((1, N)) * 2.0)).astype(np.float32)
    lp[0, ::7] = -0.0                       # signed zeros sum like the oracle's
    got, st = _path(par, lp)
    want, _, _ = _expect_path(par, lp)
    assert st[0] == -1
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_path_bad_trees_are_reported_per_sequence():
    par = np.array([[-1, 0, 1, 2],
                    [-1, 2, 1, 0],      # 1 <-> 2 cycle
                    [-1, 0, 9, 1],      # out of range at node 2
                    [3, -1, 1, 3]],     # self-parent at node 3
                   np.int32)
    lp = -np.arange(1, 17, dtype=np.float32).reshape(4, 4) / 8
    got, st = _path(par, lp)
    assert list(st) == [-1, 1, 2, 0]
    for b in range(4):
        want, ost, bad = _expect_path(par[b:b + 1], lp[b:b + 1])
        assert np.array_equal(got[b:b + 1].view(np.uint32), want.view(np.uint32))
        assert (ost == oracle.OK) == (st[b] == -1)
        if st[b] >= 0:
            assert bad == st[b]


# ---------------------------------------------------------------------------
def _expand(inp, M):
    B, N, k = inp["idx"].shape
    say(f"tree_expand: B={B} N={N} k={k} M={M} max_depth={inp['max_depth']}")
    outs = jf.jf_tree_expand(dev_tensor(inp["score"]), dev_tensor(inp["depth"]),
                             dev_tensor(inp["idx"]), dev_tensor(inp["val"]), dev_tensor(inp["lse"]),
                             dev_tensor(inp["parent"]), dev_tensor(inp["token"]), M,
                             inp["max_depth"])
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _check_expand(inp, M, full=False):
    gp, gt, gs, gd = _expand(inp, M)
    op, ot, os_, od = oracle.tree_expand(inp["score"], inp["depth"], inp["idx"], inp["val"],
                                         inp["lse"], M, inp["max_depth"], inp["parent"],
                                         inp["token"])
    assert np.array_equal(gp, op)
    assert np.array_equal(gt, ot)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gd, od)
    return (gp, gt, gs, gd) if full else gp


@pytest.mark.parametrize("B,N,k,M,max_depth", [
    (1, 16, 4, 16, 5),            # tiny workload shape
    (1, 16, 8, 16, 8),            # 16-node budget, top-8
    (1, 256, 8, 256, 16),         # 256-node budget, one sequence
    (32, 64, 8, 64, 16),          # serving batch, 64 nodes each
    (4, 256, 8, 256, 16),         # four sequences of 256 nodes
    (1, 100, 7, 37, 16),          # ragged candidate count
    (3, 2048, 8, 300, 16),        # 16384 candidates: the largest sort
    (1, 256, 64, 16384, 16),      # k = 64, every candidate kept
    (2, 50, 3, 1, 16),            # budget of one
])
@pytest.mark.parametrize("ties", [False, True])
def test_expand_matches_oracle(B, N, k, M, max_depth, ties):
    inp = synth.make_expand_inputs(B=B, N=N, k=k, max_depth=max_depth, seed=B * 1000 + N + k,
                                   ties=ties)
    _check_expand(inp, M)


def test_expand_budget_above_eligible_and_depth_cap():
    inp = synth.make_expand_inputs(B=2, N=10, k=3, max_depth=16, seed=5)
    inp["max_depth"] = 4                      # most nodes are at the cap
    gp = _check_expand(inp, 50)
    assert (gp == -2).any()


def test_expand_nothing_eligible():
    inp = synth.make_expand_inputs(B=2, N=40, k=4, max_depth=16, seed=6)
    inp["max_depth"] = 1
    gp = _check_expand(inp, 8)
    assert np.all(gp == -2)


def test_expand_signed_zero_and_infinite_scores():
    inp = synth.make_expand_inputs(B=1, N=64, k=4, max_depth=16, seed=7, ties=True)
    inp["score"][0, ::3] = -0.0
    inp["val"][0, ::5, :] = inp["lse"][0, ::5, None]          # t = +0
    inp["score"][0, 1::9] = -np.inf
    _check_expand(inp, 200)


@pytest.mark.parametrize("N,k", [(10, 8), (256, 8)])
def test_expand_all_scores_equal(N, k):
    # one selection bin holds every candidate: up to 96 of them are ranked
    # inside the bin, more take the full sort
    inp = synth.make_expand_inputs(B=2, N=N, k=k, max_depth=16, seed=8)
    inp["score"][:] = 0.0
    inp["val"][:] = inp["lse"][..., None]
    _check_expand(inp, min(N * k, 300))


@pytest.mark.parametrize("child_frac", [0.0, 1.0])
def test_expand_existing_children(child_frac):
    # no listed token taken / as many taken as the lists allow
    inp = synth.make_expand_inputs(B=4, N=256, k=8, max_depth=16, seed=11, child_frac=child_frac)
    _check_expand(inp, 256)


def test_expand_two_growth_steps():
    # the second step sees the first step's children and proposes none again
    inp = synth.make_expand_inputs(B=2, N=64, k=8, max_depth=64, seed=12)
    p1, t1, s1, d1 = _check_expand(inp, 64, full=True)
    extra = synth.make_expand_inputs(B=2, N=64, k=8, max_depth=64, seed=13)
    grown = {key: np.concatenate([inp[key], extra[key]], axis=1) for key in ("idx", "val", "lse")}
    grown.update(score=np.concatenate([inp["score"], s1], axis=1),
                 depth=np.concatenate([inp["depth"], d1], axis=1),
                 parent=np.concatenate([inp["parent"], p1], axis=1),
                 token=np.concatenate([inp["token"], t1], axis=1), max_depth=64)
    p2, t2, _, _ = _check_expand(grown, 64, full=True)
    for b in range(2):
        pairs = list(zip(grown["parent"][b].tolist(), grown["token"][b].tolist())) + \
            list(zip(p2[b].tolist(), t2[b].tolist()))
        assert len(pairs) == len(set(pairs))


def test_expand_crowded_bin_near_the_cut():
    # a wide score range with a dense cluster at the budget boundary
    inp = synth.make_expand_inputs(B=1, N=512, k=8, max_depth=16, seed=9)
    inp["score"][0, 100:300] = 1.0
    inp["val"][0, 100:300, :] = inp["lse"][0, 100:300, None]
    inp["score"][0, :5] = 50.0
    _check_expand(inp, 256)


# ---------------------------------------------------------------------------
def _accept(par, v, with_path=True):
    B, N = par.shape
    say(f"tree_accept: B={B} N={N} path={with_path}")
    outs = jf.jf_tree_accept(dev_tensor(par.astype(np.int32)), dev_tensor(v["token"]),
                             dev_tensor(v["target_next"]), dev_tensor(v["root_next"]),
                             with_path=with_path)
    torch.cuda.synchronize()
    return [None if o is None else o.cpu().numpy() for o in outs]


def _check_accept(par, v):
    alen, anode, ntok, path, st = _accept(par, v)
    olen, onode, otok, opath, obad = oracle.tree_accept(par, v["token"], v["target_next"],
                                                        v["root_next"])
    assert np.array_equal(alen, olen) and np.array_equal(anode, onode)
    assert np.array_equal(ntok, otok) and np.array_equal(path, opath)
    assert np.array_equal(st, obad)
    return alen


@pytest.mark.parametrize("N,q", [(1, 0.9), (16, 0.8), (64, 0.9), (256, 0.95), (1000, 0.97),
                                 (4096, 0.99)])
def test_accept_random_trees(N, q):
    rng = np.random.default_rng(N + 5)
    par = np.stack([synth.best_first_tree(rng, N, 16, (1, 8)) for _ in range(4)]).astype(np.int32)
    v = synth.make_verify_inputs(par, q=q, seed=N)
    _check_accept(par, v)


def test_accept_serving_batch():
    rng = np.random.default_rng(32)
    par = np.stack([synth.best_first_tree(rng, 64, 16, (1, 8)) for _ in range(32)]).astype(np.int32)
    v = synth.make_verify_inputs(par, q=0.9, seed=32)
    alen = _check_accept(par, v)
    assert alen.max() > 1


def test_accept_long_chain_and_none():
    N = 4096
    par = synth.chain_tree(N)[None].astype(np.int32)
    v = dict(token=np.arange(N, dtype=np.int32)[None], target_next=np.arange(1, N + 1, dtype=np.int32)[None],
             root_next=np.array([0], np.int32))
    assert _check_accept(par, v)[0] == N
    v["root_next"][:] = 77777
    assert _check_accept(par, v)[0] == 0


def test_accept_duplicates_star_and_bad_trees():
    par = np.array([[-1, -1, 1, 2, 0]], np.int32)
    v = dict(token=np.array([[4, 4, 6, 8, 9]], np.int32),
             target_next=np.array([[1, 6, 8, 2, 3]], np.int32), root_next=np.array([4], np.int32))
    _check_accept(par, v)
    star = synth.star_tree(12)[None].astype(np.int32)
    v = dict(token=np.array([[5, 9, 9, 5, 9, 3, 9, 9, 9, 9, 9, 9]], np.int32),
             target_next=np.arange(12, dtype=np.int32)[None], root_next=np.array([9], np.int32))
    _check_accept(star, v)
    par = np.array([[-1, 0, 1, 2], [-1, 2, 1, 0], [-1, 0, 9, 1], [3, -1, 1, 3]], np.int32)
    v = dict(token=np.zeros((4, 4), np.int32), target_next=np.zeros((4, 4), np.int32),
             root_next=np.zeros(4, np.int32))
    _check_accept(par, v)


def test_accept_without_path():
    rng = np.random.default_rng(3)
    par = np.stack([synth.best_first_tree(rng, 256, 16, (1, 8)) for _ in range(2)]).astype(np.int32)
    v = synth.make_verify_inputs(par, q=0.95, seed=3)
    alen, anode, ntok, path, st = _accept(par, v, with_path=False)
    olen, onode, otok, _, _ = oracle.tree_accept(par, v["token"], v["target_next"], v["root_next"])
    assert path is None
    assert np.array_equal(alen, olen) and np.array_equal(anode, onode) and np.array_equal(ntok, otok)
