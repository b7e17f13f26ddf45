"""Pins of the oracle's tree attention (CPU only).

What pins it, none of which reuses the oracle's code:
  * a hand-computed golden example (tests/golden/attn_tiny.txt);
  * chain trees == textbook causal attention over [prefix ; tree] (torch SDPA);
  * star trees  == each node attending to prefix + itself (torch SDPA);
  * any tree    == causal attention over [prefix ; root-to-node path], last row
                   (numpy brute force, tests/brute.py);
  * grouped heads follow h // (Hq/Hkv) (torch SDPA with grouped KV heads);
  * closed forms: q = 0 -> mean of the visible values; empty prefix with a lone
    root -> that root's value;
  * changing K/V of a non-ancestor leaves a node's output unchanged; relabelling
    the nodes permutes the outputs.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from brute import path_attention
from helpers import attn_f64, oracle_attn
from tree_causal_draft_parent_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _oracle_all(f, inp, scale=None):
    return oracle.tree_attn(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"], parent=inp["parent"],
                            k_cache=f["k_cache"], v_cache=f["v_cache"],
                            block_table=inp["block_table"], prefix_len=inp["prefix_len"],
                            page_size=inp["page_size"], scale=scale)


def test_golden_tiny():
    ln = math.log
    q = np.zeros((1, 3, 2, 1))
    q[0, :, 0, 0] = 1.0
    k_tree = np.array([ln(2), ln(3), ln(4)]).reshape(1, 3, 1, 1)
    v_tree = np.array([2.0, 4.0, 8.0]).reshape(1, 3, 1, 1)
    k_cache = np.zeros((1, 1, 1, 1))
    v_cache = np.ones((1, 1, 1, 1))
    out, lse = oracle.tree_attn(q=q, k_tree=k_tree, v_tree=v_tree,
                                parent=np.array([[-1, 0, 0]], np.int32), k_cache=k_cache,
                                v_cache=v_cache, block_table=np.zeros((1, 1), np.int32),
                                prefix_len=np.array([1], np.int32), page_size=1, scale=1.0)
    n = 0
    for line in open(os.path.join(GOLD, "attn_tiny.txt")):
        if line.startswith("#") or not line.strip():
            continue
        node, head, num, den, arg = [int(t) for t in line.split()]
        assert abs(out[0, node, head, 0] - num / den) < 1e-13
        assert abs(lse[0, node, head] - math.log(arg)) < 1e-13
        n += 1
    assert n == 6


def _sdpa(q, k, v, allowed, scale=None):
    """torch SDPA (CPU, float64) with a boolean mask; q [H, Lq, D], k/v [H, Lk, D]."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(allowed), scale=scale)
    return o.numpy()


def _contig(inp):
    """Prefix K/V of a contiguous-layout input as [B, P, Hkv, D] float64."""
    f = attn_f64(inp)
    return f, f["k_cache"], f["v_cache"]


@pytest.mark.parametrize("P,N,G", [(0, 5, 1), (7, 9, 2), (33, 70, 4)])
def test_chain_equals_causal(P, N, G):
    Hkv, D = 2, 16
    inp = synth.make_attn_inputs(B=1, N=N, Hq=Hkv * G, Hkv=Hkv, D=D, dtype="f32",
                                 prefix_lens=[P], parents=synth.chain_tree(N)[None], seed=11 + P)
    f, kc, vc = _contig(inp)
    out, _ = _oracle_all(f, inp)
    for h in range(Hkv * G):
        g = h // G
        k = np.concatenate([kc[0, :P, g], f["k_tree"][0, :, g]])[None]
        v = np.concatenate([vc[0, :P, g], f["v_tree"][0, :, g]])[None]
        q = f["q"][0, :, h][None]
        allowed = np.arange(P + N)[None, :] <= (P + np.arange(N))[:, None]
        ref = _sdpa(q, k, v, allowed)[0]
        assert np.max(np.abs(out[0, :, h] - ref)) < 1e-12


@pytest.mark.parametrize("P,N", [(0, 4), (5, 17), (64, 33)])
def test_star_equals_prefix_plus_self(P, N):
    Hkv, G, D = 1, 3, 8
    inp = synth.make_attn_inputs(B=1, N=N, Hq=Hkv * G, Hkv=Hkv, D=D, dtype="f32",
                                 prefix_lens=[P], parents=synth.star_tree(N)[None], seed=5 + N)
    f, kc, vc = _contig(inp)
    out, _ = _oracle_all(f, inp)
    for h in range(G):
        k = np.concatenate([kc[0, :P, 0], f["k_tree"][0, :, 0]])[None]
        v = np.concatenate([vc[0, :P, 0], f["v_tree"][0, :, 0]])[None]
        q = f["q"][0, :, h][None]
        cols = np.arange(P + N)[None, :]
        allowed = (cols < P) | (cols == (P + np.arange(N))[:, None])
        ref = _sdpa(q, k, v, allowed)[0]
        assert np.max(np.abs(out[0, :, h] - ref)) < 1e-12


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("paged", [False, True])
def test_brute_force_paths(seed, paged):
    rng = np.random.default_rng(seed)
    B = 2
    N = int(rng.integers(1, 14))
    P = rng.integers(0, 40, size=B).astype(np.int32)
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.choice([1, 2]))
    inp = synth.make_attn_inputs(B=B, N=N, Hq=Hkv * G, Hkv=Hkv, D=8, dtype="bf16",
                                 prefix_lens=P, page_size=4 if paged else 0,
                                 shuffled_pages=paged, max_depth=5, branching=(1, 3),
                                 seed=100 + seed)
    f = attn_f64(inp)
    out, lse = _oracle_all(f, inp)
    bo, bl = path_attention(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"], parent=inp["parent"],
                            k_cache=f["k_cache"], v_cache=f["v_cache"],
                            block_table=inp["block_table"], prefix_len=inp["prefix_len"],
                            page_size=inp["page_size"])
    assert np.max(np.abs(out - bo)) < 1e-12
    assert np.max(np.abs(lse - bl)) < 1e-12


def test_gqa_head_map_matches_sdpa_grouping():
    # A chain of 6 nodes under an 8-token prefix with 8 query heads on 2 KV heads;
    # torch's grouped-query SDPA shares KV head g with query heads g*G .. g*G+G-1.
    P, N, Hq, Hkv, D = 8, 6, 8, 2, 4
    inp = synth.make_attn_inputs(B=1, N=N, Hq=Hq, Hkv=Hkv, D=D, dtype="f32", prefix_lens=[P],
                                 parents=synth.chain_tree(N)[None], seed=3)
    f, kc, vc = _contig(inp)
    out, _ = _oracle_all(f, inp)
    k = np.concatenate([kc[0, :P], f["k_tree"][0]]).transpose(1, 0, 2)  # [Hkv, L, D]
    v = np.concatenate([vc[0, :P], f["v_tree"][0]]).transpose(1, 0, 2)
    q = f["q"][0].transpose(1, 0, 2)  # [Hq, N, D]
    allowed = np.arange(P + N)[None, :] <= (P + np.arange(N))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(allowed), enable_gqa=True)[0].numpy()
    assert np.max(np.abs(out[0].transpose(1, 0, 2) - ref)) < 1e-12


def test_zero_query_is_mean_of_visible_values():
    inp = synth.make_attn_inputs(B=1, N=12, Hq=2, Hkv=1, D=4, dtype="f32", prefix_lens=[9],
                                 max_depth=4, branching=(1, 3), seed=9)
    f = attn_f64(inp)
    f["q"][:] = 0.0
    out, lse = _oracle_all(f, inp)
    par = inp["parent"][0]
    for i in range(12):
        vis = [f["v_cache"][0, p, 0] for p in range(9)]
        j = i
        n_anc = 0
        while j != -1:
            vis.append(f["v_tree"][0, j, 0])
            j = par[j]
            n_anc += 1
        ref = np.mean(vis, axis=0)
        assert np.max(np.abs(out[0, i, 0] - ref)) < 1e-13
        assert abs(lse[0, i, 0] - math.log(9 + n_anc)) < 1e-13


def test_empty_prefix_lone_root_returns_its_value():
    inp = synth.make_attn_inputs(B=1, N=1, Hq=4, Hkv=2, D=8, dtype="f32", prefix_lens=[0],
                                 parents=np.array([[-1]], np.int32), seed=2)
    f = attn_f64(inp)
    out, _ = _oracle_all(f, inp)
    for h in range(4):
        assert np.array_equal(out[0, 0, h], f["v_tree"][0, 0, h // 2])


def test_non_ancestor_perturbation_and_relabelling():
    N = 20
    inp = synth.make_attn_inputs(B=1, N=N, Hq=2, Hkv=1, D=8, dtype="f32", prefix_lens=[10],
                                 max_depth=6, branching=(1, 4), seed=21)
    f = attn_f64(inp)
    out, _ = _oracle_all(f, inp)
    par = inp["parent"][0]
    anc_of_last = set()
    j = N - 1
    while j != -1:
        anc_of_last.add(j)
        j = par[j]
    f2 = {k: v.copy() for k, v in f.items()}
    for j in range(N):
        if j not in anc_of_last:
            f2["k_tree"][0, j] += 3.0
            f2["v_tree"][0, j] -= 5.0
    out2, _ = _oracle_all(f2, inp)
    assert np.array_equal(out[0, N - 1], out2[0, N - 1])
    # relabel nodes by a permutation: outputs permute the same way
    perm = np.random.default_rng(0).permutation(N)   # new id of old node j is perm[j]
    inv = np.argsort(perm)
    par_new = np.array([perm[par[inv[n]]] if par[inv[n]] >= 0 else -1 for n in range(N)], np.int32)
    f3 = dict(f)
    for key in ("q", "k_tree", "v_tree"):
        f3[key] = f[key][:, inv]
    inp3 = dict(inp, parent=par_new[None])
    out3, _ = _oracle_all(f3, inp3)
    assert np.max(np.abs(out3[0] - out[0, inv])) < 1e-12


def test_rows_subset_matches_full():
    inp = synth.make_attn_inputs(B=3, N=9, Hq=4, Hkv=2, D=16, dtype="bf16", prefix_lens=[5, 0, 17],
                                 page_size=4, shuffled_pages=True, seed=4)
    out, lse = oracle_attn(inp)
    rows = np.array([0, 7, 50, 3 * 9 * 4 - 1])
    o2, l2 = oracle_attn(inp, rows=rows)
    assert np.array_equal(o2, out.reshape(-1, 16)[rows])
    assert np.array_equal(l2, lse.reshape(-1)[rows])


# ---------------------------------------------------------------------------
# Packed trees of different sizes, bad page ids, FP8 prefix caches

def _packed_inputs(seed, counts, P, paged=True, kv_dtype=None, D=8, G=2, Hkv=2):
    return synth.make_attn_inputs(B=len(counts), N=0, Hq=Hkv * G, Hkv=Hkv, D=D, dtype="bf16",
                                  prefix_lens=P, page_size=4 if paged else 0,
                                  shuffled_pages=paged, max_depth=5, branching=(1, 3),
                                  seed=seed, node_counts=counts, kv_dtype=kv_dtype)


@pytest.mark.parametrize("seed", range(3))
def test_packed_trees_match_path_brute_force(seed):
    # each sequence of a ragged packed batch, through the brute force of its own
    # root-to-node paths (the brute force knows nothing of the packing)
    counts = [3, 11, 1, 7][: 2 + seed]
    P = np.array([5, 0, 9, 13][: len(counts)], np.int32)
    inp = _packed_inputs(200 + seed, counts, P)
    f = attn_f64(inp)
    out, lse = oracle.tree_attn(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"],
                                parent=inp["parent"], k_cache=f["k_cache"], v_cache=f["v_cache"],
                                block_table=inp["block_table"], prefix_len=P,
                                page_size=inp["page_size"], node_off=inp["node_off"])
    off = inp["node_off"]
    for b, n in enumerate(counts):
        sl = slice(off[b], off[b + 1])
        bo, bl = path_attention(q=f["q"][None, sl], k_tree=f["k_tree"][None, sl],
                                v_tree=f["v_tree"][None, sl], parent=inp["parent"][None, sl],
                                k_cache=f["k_cache"], v_cache=f["v_cache"],
                                block_table=inp["block_table"][b:b + 1], prefix_len=P[b:b + 1],
                                page_size=inp["page_size"])
        assert np.max(np.abs(out[sl] - bo[0])) < 1e-12
        assert np.max(np.abs(lse[sl] - bl[0])) < 1e-12


def test_packed_mask_rows_match_each_tree_alone():
    counts = [5, 70, 1, 64]
    inp = _packed_inputs(210, counts, np.array([1, 2, 3, 4], np.int32))
    mask, depth, st, bad = oracle.tree_mask(inp["parent"], node_off=inp["node_off"])
    assert st == oracle.OK and mask.shape == (sum(counts), 2)
    off = inp["node_off"]
    for b, n in enumerate(counts):
        m1, d1, _, _ = oracle.tree_mask(inp["parent"][None, off[b]:off[b + 1]])
        assert np.array_equal(mask[off[b]:off[b + 1], :m1.shape[2]], m1[0])
        assert np.all(mask[off[b]:off[b + 1], m1.shape[2]:] == 0)
        assert np.array_equal(depth[off[b]:off[b + 1]], d1[0])


def test_packed_bad_tree_reports_its_row():
    par = np.array([-1, 0, -1, 5, 0], np.int32)        # sequence 1 = rows 2..4; row 3's parent 5 >= 3
    _, _, st, bad = oracle.tree_mask(par, node_off=np.array([0, 2, 5]))
    assert st == oracle.BAD_TREE and bad == 3


def test_bad_page_reads_as_zero_key_and_zero_value():
    # a block-table entry out of range equals a valid page holding zeros there
    inp = synth.make_attn_inputs(B=2, N=6, Hq=4, Hkv=2, D=8, dtype="bf16",
                                 prefix_lens=np.array([10, 7], np.int32), page_size=4,
                                 shuffled_pages=True, max_depth=4, branching=(1, 2), seed=220,
                                 extra_pages=1)
    f = attn_f64(inp)
    zero_page = inp["num_pages"] - 1                  # the spare page, never in the table
    f["k_cache"][zero_page] = 0.0
    f["v_cache"][zero_page] = 0.0
    bt_bad, bt_zero = inp["block_table"].copy(), inp["block_table"].copy()
    bt_bad[0, 1] = 999
    bt_zero[0, 1] = zero_page
    kw = dict(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"], parent=inp["parent"],
              k_cache=f["k_cache"], v_cache=f["v_cache"], prefix_len=inp["prefix_len"],
              page_size=4)
    o1, l1, flag = oracle.tree_attn(block_table=bt_bad, bad_page_ok=True, **kw)
    o2, l2 = oracle.tree_attn(block_table=bt_zero, **kw)
    assert flag
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    with pytest.raises(ValueError):
        oracle.tree_attn(block_table=bt_bad, **kw)


def test_fp8_decode_matches_the_library_and_known_values():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(got[nan])) and np.all(np.isnan(ref[nan]))
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6
    assert got[0x01] == 2.0 ** -9 and got[0xB8] == -1.0 and got[0x3C] == 1.5
    assert np.signbit(got[0x80]) and got[0x80] == 0.0
    assert np.array_equal(oracle.fp8_e4m3_to_f64(codes[:0x7F], 0.25), got[:0x7F] * 0.25)


def test_fp8_cache_attention_equals_decoded_values():
    # the generator's codes decode within half an E4M3 step of the drawn values,
    # and attention over an FP8 cache is attention over its decoded values
    inp = _packed_inputs(230, [6, 9], np.array([12, 5], np.int32), kv_dtype="fp8")
    assert inp["k_cache"].dtype == np.uint8 and inp["k_scale"] > 0
    f = attn_f64(inp)
    v = f["k_cache"] / inp["k_scale"]
    assert np.max(np.abs(v)) <= 448.0
    out, lse = oracle_attn(inp)
    o2, l2 = oracle.tree_attn(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"],
                              parent=inp["parent"], k_cache=f["k_cache"], v_cache=f["v_cache"],
                              block_table=inp["block_table"], prefix_len=inp["prefix_len"],
                              page_size=inp["page_size"], node_off=inp["node_off"])
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
