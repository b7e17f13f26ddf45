"""Pins of the oracle's path scores and one-level best-first expansion (CPU only).

Path scores: a hand-derived golden forest (tests/golden/path_tree7.txt); a
chain equals numpy's cumulative sum; a star equals the inputs; the recursion
score(i) = score(parent(i)) + logp(i) on random forests; relabelling the nodes
permutes the scores; bad trees are reported like the mask's.
Expansion: hand-derived golden steps (tests/golden/expand_small.txt, and
expand_grown.txt where two candidates are already children); a brute force
with numpy's lexsort over float32 scores that drops the (parent, token) pairs
already in the tree; two successive steps never give a node two children with
the same token; the output order, the depth cap, the budget and ties on
integer-valued inputs."""
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


def test_path_golden_forest():
    g = _read("path_tree7.txt")
    par = np.array([[int(t) for t in g["parent"]]], np.int32)
    lp = np.array([[float(t) for t in g["logp"]]])
    score, st, bad = oracle.path_scores(par, lp)
    assert st == oracle.OK and bad == -1
    assert np.array_equal(score[0], np.array([float(t) for t in g["score"]]))


def test_path_chain_is_cumulative_sum():
    N = 50
    lp = synth.make_path_inputs(B=1, N=N, seed=3)["logp"].astype(np.float64)
    score, st, _ = oracle.path_scores(synth.chain_tree(N)[None], lp)
    assert st == oracle.OK
    assert np.max(np.abs(score[0] - np.cumsum(lp[0]))) < 1e-12


def test_path_star_is_identity():
    N = 40
    lp = synth.make_path_inputs(B=1, N=N, seed=4)["logp"].astype(np.float64)
    score, st, _ = oracle.path_scores(synth.star_tree(N)[None], lp)
    assert st == oracle.OK and np.array_equal(score, lp)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_path_recursion_and_relabelling(seed):
    inp = synth.make_path_inputs(B=3, N=120, seed=seed)
    par, lp = inp["parent"], inp["logp"].astype(np.float64)
    score, st, _ = oracle.path_scores(par, lp)
    assert st == oracle.OK
    for b in range(3):
        p = par[b]
        up = np.where(p >= 0, score[b][np.maximum(p, 0)], 0.0)
        assert np.max(np.abs(score[b] - up - lp[b])) < 1e-12
    # relabel the nodes of sequence 0 by a permutation: scores follow the nodes
    rng = np.random.default_rng(seed)
    perm = rng.permutation(120)                  # new id of old node i is perm[i]
    inv = np.argsort(perm)
    p0 = par[0]
    newpar = np.where(p0[inv] >= 0, perm[np.maximum(p0[inv], 0)], -1).astype(np.int32)
    s2, st2, _ = oracle.path_scores(newpar[None], lp[0][inv][None])
    assert st2 == oracle.OK
    assert np.max(np.abs(s2[0] - score[0][inv])) < 1e-12


def test_path_bad_trees_match_the_mask():
    par = np.array([[-1, 0, 3, 2, 1], [-1, 0, 1, 9, 2]], np.int32)   # a cycle; an out-of-range parent
    lp = -np.ones((2, 5))
    score, st, bad = oracle.path_scores(par, lp)
    _, _, mst, mbad = oracle.tree_mask(par)
    assert st == oracle.BAD_TREE and st == mst and bad == mbad == 2
    assert score[0, 2] == 0.0 and score[0, 3] == 0.0 and score[1, 3] == 0.0 and score[1, 0] == -1.0


def _golden_expand(name="expand_small.txt"):
    g = _read(name)
    f = lambda k: np.array([float(t) for t in g[k]], np.float32)
    i = lambda k: np.array([int(t) for t in g[k]], np.int32)
    return dict(score=f("score")[None], depth=i("depth")[None], lse=f("lse")[None],
                val=f("val").reshape(1, 4, 2), idx=i("idx").reshape(1, 4, 2),
                max_depth=int(g["max_depth"][0]), parent=i("parent")[None],
                token=i("token")[None]), g


def _expand(inp, M, **kw):
    a = {**inp, **kw}
    return oracle.tree_expand(a["score"], a["depth"], a["idx"], a["val"], a["lse"], M,
                              a["max_depth"], a["parent"], a["token"])


@pytest.mark.parametrize("name,M", [("expand_small.txt", 5), ("expand_small.txt", 8),
                                    ("expand_grown.txt", 3), ("expand_grown.txt", 5)])
def test_expand_golden(name, M):
    inp, g = _golden_expand(name)
    p, t, s, d = _expand(inp, M)
    assert list(p[0]) == [int(x) for x in g[f"m{M}_parent"]]
    assert list(t[0]) == [int(x) for x in g[f"m{M}_token"]]
    assert list(d[0]) == [int(x) for x in g[f"m{M}_depth"]]
    assert np.array_equal(s[0], np.array([float(x) for x in g[f"m{M}_score"]], np.float32))


def _brute(inp, M):
    """Brute force: every eligible candidate's float32 score, ordered with
    lexsort; a candidate whose (parent, token) pair is already a child in the
    tree is dropped (a set of the tree's pairs)."""
    B, N, k = inp["idx"].shape
    out = []
    for b in range(B):
        t = (inp["val"][b] - inp["lse"][b][:, None]).astype(np.float32)   # float32 arithmetic
        s = (inp["score"][b][:, None] + t).astype(np.float32)
        p = np.repeat(np.arange(N), k).reshape(N, k)
        r = np.tile(np.arange(k), (N, 1))
        kids = set(zip(inp["parent"][b].tolist(), inp["token"][b].tolist()))
        new = np.array([[(i, int(inp["idx"][b, i, j])) not in kids for j in range(k)]
                        for i in range(N)])
        ok = ((inp["depth"][b] >= 1) & (inp["depth"][b] + 1 <= inp["max_depth"]))[:, None] & new
        s, p, r = s[ok].ravel(), p[ok].ravel(), r[ok].ravel()
        order = np.lexsort((r, p, -s.astype(np.float64)))[:M]
        out.append((p[order], r[order], s[order]))
    return out


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("N,k,M", [(16, 4, 10), (64, 8, 64), (256, 8, 256), (40, 3, 200)])
def test_expand_matches_lexsort(ties, N, k, M):
    inp = synth.make_expand_inputs(B=2, N=N, k=k, seed=N + k + M, ties=ties, max_depth=12)
    p, t, s, d = _expand(inp, M)
    for b, (bp, br, bs) in enumerate(_brute(inp, M)):
        n = len(bp)
        assert np.array_equal(p[b, :n], bp)
        assert np.array_equal(t[b, :n], inp["idx"][b][bp, br])
        assert np.array_equal(s[b, :n], bs)
        assert np.array_equal(d[b, :n], inp["depth"][b][bp] + 1)
        assert np.all(p[b, n:] == -2) and np.all(t[b, n:] == -1) and np.all(d[b, n:] == 0)
        assert np.all(np.isneginf(s[b, n:]))
        assert np.all(np.diff(s[b, :n].astype(np.float64)) <= 0)         # best first
        assert np.all(d[b, :n] <= inp["max_depth"])


def test_expand_takes_all_when_budget_allows():
    # no child carries a listed token: every candidate is new
    inp = synth.make_expand_inputs(B=1, N=10, k=2, seed=9, max_depth=100, child_frac=0.0)
    p, t, s, d = _expand(inp, 25)
    assert sorted(zip(p[0, :20], t[0, :20])) == sorted(
        (i, inp["idx"][0, i, r]) for i in range(10) for r in range(2))
    assert np.all(p[0, 20:] == -2)


def test_expand_skips_existing_children():
    # every listed token of every node is already a child: nothing is new
    inp = synth.make_expand_inputs(B=1, N=6, k=2, seed=10, max_depth=100, child_frac=0.0)
    kids_p, kids_t = [-1] * 6, list(range(1000, 1006))
    for i in range(6):
        kids_p += [i, i]
        kids_t += [int(inp["idx"][0, i, 0]), int(inp["idx"][0, i, 1])]
    n = len(kids_p)
    pad = lambda a, fill: np.concatenate([a, np.full((1, n - 6) + a.shape[2:], fill, a.dtype)], axis=1)
    grown = dict(score=pad(inp["score"], -1.0), depth=pad(inp["depth"], 100), idx=pad(inp["idx"], 7),
                 val=pad(inp["val"], 0.0), lse=pad(inp["lse"], 1.0), max_depth=100,
                 parent=np.array([kids_p], np.int32), token=np.array([kids_t], np.int32))
    # the padded nodes (depth 100 = max_depth) have no eligible children
    p, t, s, d = _expand(grown, 8)
    assert np.all(p == -2) and np.all(t == -1) and np.all(np.isneginf(s))


@pytest.mark.parametrize("N,k,M", [(16, 4, 16), (64, 8, 64)])
def test_two_growth_steps_never_duplicate_siblings(N, k, M):
    # grow the tree twice: the second step sees the first step's children and
    # proposes none of them again, so no node ends with two children carrying
    # the same token (the first step's lists are unchanged: a node's
    # conditional distribution does not depend on its children)
    inp = synth.make_expand_inputs(B=2, N=N, k=k, seed=N + k, max_depth=64)
    p1, t1, s1, d1 = _expand(inp, M)
    extra = synth.make_expand_inputs(B=2, N=M, k=k, seed=N + k + 1, max_depth=64)
    grown = {}
    for key in ("idx", "val", "lse"):
        grown[key] = np.concatenate([inp[key], extra[key]], axis=1)
    grown["score"] = np.concatenate([inp["score"], s1], axis=1)
    grown["depth"] = np.concatenate([inp["depth"], d1], axis=1)
    grown["parent"] = np.concatenate([inp["parent"], p1], axis=1)
    grown["token"] = np.concatenate([inp["token"], t1], axis=1)
    grown["max_depth"] = inp["max_depth"]
    assert np.all(p1 >= 0)                     # the budget was filled both times
    p2, t2, s2, d2 = _expand(grown, M)
    assert np.all(p2 >= 0)
    for b in range(2):
        pairs = list(zip(grown["parent"][b].tolist(), grown["token"][b].tolist())) + \
            list(zip(p2[b].tolist(), t2[b].tolist()))
        assert len(pairs) == len(set(pairs)), "a node got two children with the same token"


def test_expand_signed_zero_is_plus_zero():
    # -0 ties +0 (candidate order decides) and is written as +0
    inp = synth.make_expand_inputs(B=1, N=2, k=1, seed=14, max_depth=100, child_frac=0.0)
    inp["score"][:] = np.array([-0.0, 0.0], np.float32)
    inp["val"][:] = np.array([[[-0.0], [0.0]]], np.float32)
    inp["lse"][:] = 0.0
    p, t, s, d = _expand(inp, 2, max_depth=100)
    assert list(p[0]) == [0, 1]
    assert list(s[0].view(np.uint32)) == [0, 0]


# ---------------------------------------------------------------------------
# Greedy verification (longest accepted path)

def test_accept_golden():
    g = _read("accept_tree7.txt")
    arr = {k: np.array([[int(t) for t in g[k]]], np.int32)
           for k in ("parent", "token", "target_next")}
    root = np.array([int(g["root_next"][0])], np.int32)
    alen, anode, ntok, path, bad = oracle.tree_accept(arr["parent"], arr["token"],
                                                      arr["target_next"], root)
    assert alen[0] == int(g["accept_len"][0]) and anode[0] == int(g["accept_node"][0])
    assert ntok[0] == int(g["next_token"][0]) and bad[0] == -1
    assert list(path[0]) == [int(t) for t in g["path"]]


def _greedy_decode(par, tok, nxt, root):
    """Top-down: from the prefix, repeatedly step to the child whose token is
    the target's next token (trees with distinct sibling tokens have at most
    one), as greedy decoding of the target would."""
    node, path = -1, []
    while True:
        want = root if node == -1 else nxt[node]
        kids = [c for c in range(len(par)) if par[c] == node and tok[c] == want]
        assert len(kids) <= 1
        if not kids:
            return len(path), node, want, path
        node = kids[0]
        path.append(node)


def _verify_inputs(rng, N, q):
    """A best-first tree with distinct sibling tokens; the target's next token
    after a node is one of its children's tokens with probability q."""
    par = synth.best_first_tree(rng, N, 16, (1, 8)).astype(np.int32)
    tok = np.zeros(N, np.int32)
    for p in range(-1, N):
        kids = np.flatnonzero(par == p)
        tok[kids] = rng.choice(1000, size=len(kids), replace=False)
    nxt = rng.integers(1000, 2000, size=N).astype(np.int32)      # never a draft token
    for j in range(N):
        kids = np.flatnonzero(par == j)
        if len(kids) and rng.random() < q:
            nxt[j] = tok[rng.choice(kids)]
    roots = np.flatnonzero(par == -1)
    root = tok[rng.choice(roots)] if rng.random() < 0.9 else 5000
    return par, tok, nxt, np.int32(root)


@pytest.mark.parametrize("N,q", [(16, 0.8), (64, 0.9), (256, 0.95)])
def test_accept_equals_greedy_decoding_synth(N, q):
    # the shared input generator's trees and tokens, checked the same way
    rng = np.random.default_rng(N)
    par = np.stack([synth.best_first_tree(rng, N, 16, (1, 8)) for _ in range(4)]).astype(np.int32)
    v = synth.make_verify_inputs(par, q=q, seed=N)
    alen, anode, ntok, path, bad = oracle.tree_accept(par, v["token"], v["target_next"],
                                                      v["root_next"])
    for b in range(4):
        L, node, want, p = _greedy_decode(par[b], v["token"][b], v["target_next"][b],
                                          v["root_next"][b])
        assert (alen[b], anode[b], ntok[b]) == (L, node, want) and list(path[b, :L]) == p


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N,q", [(16, 0.8), (64, 0.9), (256, 0.95)])
def test_accept_equals_greedy_decoding(seed, N, q):
    rng = np.random.default_rng(seed * 100 + N)
    B = 3
    ins = [_verify_inputs(rng, N, q) for _ in range(B)]
    par = np.stack([i[0] for i in ins])
    tok = np.stack([i[1] for i in ins])
    nxt = np.stack([i[2] for i in ins])
    root = np.array([i[3] for i in ins], np.int32)
    alen, anode, ntok, path, bad = oracle.tree_accept(par, tok, nxt, root)
    for b in range(B):
        L, node, want, p = _greedy_decode(par[b], tok[b], nxt[b], root[b])
        assert (alen[b], anode[b], ntok[b]) == (L, node, want)
        assert list(path[b, :L]) == p and np.all(path[b, L:] == -1) and bad[b] == -1


def test_accept_closed_cases():
    N = 12
    chain = synth.chain_tree(N)[None].astype(np.int32)
    tok = np.arange(100, 100 + N, dtype=np.int32)[None]
    nxt = np.arange(101, 101 + N, dtype=np.int32)[None]       # each node predicts the next
    alen, anode, ntok, path, _ = oracle.tree_accept(chain, tok, nxt, np.array([100], np.int32))
    assert alen[0] == N and anode[0] == N - 1 and ntok[0] == 100 + N
    assert list(path[0]) == list(range(N))
    # nothing accepted: the next token is the target's token after the prefix
    alen, anode, ntok, path, _ = oracle.tree_accept(chain, tok, nxt, np.array([7], np.int32))
    assert (alen[0], anode[0], ntok[0]) == (0, -1, 7) and np.all(path == -1)
    # star: several accepted roots of depth 1 -> the lowest index
    star = synth.star_tree(N)[None].astype(np.int32)
    tok = np.array([[5, 9, 9, 5, 9, 3, 9, 9, 9, 9, 9, 9]], np.int32)
    alen, anode, ntok, path, _ = oracle.tree_accept(star, tok, nxt, np.array([9], np.int32))
    assert (alen[0], anode[0], ntok[0]) == (1, 1, nxt[0, 1]) and path[0, 0] == 1


def test_accept_duplicate_siblings_take_the_deeper_branch():
    # nodes 0 and 1 both carry the target's first token; only node 1's branch
    # continues, so the deepest accepted node is under node 1
    par = np.array([[-1, -1, 1, 2, 0]], np.int32)
    tok = np.array([[4, 4, 6, 8, 9]], np.int32)
    nxt = np.array([[1, 6, 8, 2, 3]], np.int32)
    alen, anode, ntok, path, _ = oracle.tree_accept(par, tok, nxt, np.array([4], np.int32))
    assert (alen[0], anode[0], ntok[0]) == (3, 3, 2) and list(path[0, :3]) == [1, 2, 3]


def test_accept_bad_trees_accept_nothing():
    par = np.array([[-1, 0, 1, 2], [-1, 2, 1, 0], [-1, 0, 9, 1]], np.int32)
    tok = np.zeros((3, 4), np.int32)
    nxt = np.zeros((3, 4), np.int32)
    alen, anode, ntok, path, bad = oracle.tree_accept(par, tok, nxt, np.zeros(3, np.int32))
    assert list(bad) == [-1, 1, 2]
    assert alen[0] == 4 and list(alen[1:]) == [0, 0] and list(anode[1:]) == [-1, -1]
    _, _, mst, mbad = oracle.tree_mask(par[1:2])
    assert mst == oracle.BAD_TREE and mbad == 1
