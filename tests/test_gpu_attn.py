"""jf_tree_attn_fwd vs the oracle.

fp32 path: max-abs <= 1e-5.  bf16 path (fp32 accumulation): max-abs <= 2e-2
and relative RMS <= 1e-2 over the compared outputs; lse compared the same way.
Small cases compare every output; full-size workloads compare every output
where the oracle is quick enough, else a seeded sample of rows.
"""
import numpy as np
import pytest
import torch

from gpu_util import dev_tensor, host_f64, say, upload_attn
from helpers import oracle_attn, rel_rms
from tree_causal_draft_parent_amd import jf, synth

pytestmark = pytest.mark.gpu


def run_gpu(inp, page_status=None, cus=0):
    d = upload_attn(inp)
    mask, _, st = jf.jf_tree_mask_build(d["parent"])
    out, lse = jf.jf_tree_attn_fwd(d["q"], d["k_tree"], d["v_tree"], mask, d["k_cache"],
                                   d["v_cache"], d["block_table"], inp["prefix_len"],
                                   page_status=page_status, cus=cus)
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy() == -1)
    return host_f64(out), host_f64(lse)


def compare(inp, rows=None, label="", cus=0):
    B, N, Hq, D = inp["q"].shape
    say(f"attn {label}: B={B} N={N} Hq={Hq} Hkv={inp['k_tree'].shape[2]} D={D} "
        f"P={list(inp['prefix_len'][:4])} page={inp['page_size']} dtype={inp['dtype']} "
        f"rows={'all' if rows is None else len(rows)} cus={cus}")
    out, lse = run_gpu(inp, cus=cus)
    ro, rl = oracle_attn(inp, rows=rows)
    go = out.reshape(-1, D) if rows is None else out.reshape(-1, D)[rows]
    gl = lse.reshape(-1) if rows is None else lse.reshape(-1)[rows]
    ro = ro.reshape(-1, D)
    rl = rl.reshape(-1)
    err = np.max(np.abs(go - ro))
    lerr = np.max(np.abs(gl - rl))
    if inp["dtype"] == "f32":
        assert err <= 1e-5, err
        assert lerr <= 1e-5, lerr
    else:
        assert err <= 2e-2, err
        assert rel_rms(go, ro) <= 1e-2, rel_rms(go, ro)
        assert lerr <= 2e-2, lerr
        assert rel_rms(gl, rl) <= 1e-2
    return out, lse


def test_tiny_fp32_workload():
    compare(synth.make_workload(0, parts=("attn",))["attn"], label="tiny fp32")


@pytest.mark.parametrize("paged", [False, True])
def test_bf16_multi_tile_ragged(paged):
    # 100 nodes -> two tree blocks (64 + 36); G = 4 -> 400 query rows -> 4 tiles,
    # the last one partial; prefixes of 0, 1, 63, 64, 65 and 700 tokens.
    inp = synth.make_attn_inputs(B=6, N=100, Hq=8, Hkv=2, D=128, dtype="bf16",
                                 prefix_lens=[0, 1, 63, 64, 65, 700], page_size=16 if paged else 0,
                                 shuffled_pages=paged, seed=77)
    compare(inp, label="ragged")


@pytest.mark.parametrize("kind", ["chain", "star"])
def test_bf16_chain_and_star(kind):
    N = 130
    par = synth.chain_tree(N) if kind == "chain" else synth.star_tree(N)
    inp = synth.make_attn_inputs(B=1, N=N, Hq=4, Hkv=1, D=128, dtype="bf16", prefix_lens=[300],
                                 parents=par[None], seed=5)
    compare(inp, label=kind)


def test_fp32_paged_ragged():
    inp = synth.make_attn_inputs(B=3, N=20, Hq=6, Hkv=3, D=64, dtype="f32",
                                 prefix_lens=[0, 17, 150], page_size=16, shuffled_pages=True, seed=8)
    compare(inp, label="fp32 paged")


def test_paged_equals_contiguous_bitwise():
    kw = dict(B=3, N=64, Hq=8, Hkv=2, D=128, dtype="bf16", prefix_lens=[1000, 37, 4096], seed=3)
    a = synth.make_attn_inputs(page_size=0, **kw)
    b = synth.make_attn_inputs(page_size=16, shuffled_pages=True, **kw)
    # copy the contiguous prefix into b's shuffled pages
    for bb in range(3):
        P = int(kw["prefix_lens"][bb])
        for pos in range(P):
            pg = b["block_table"][bb, pos // 16]
            b["k_cache"][pg, pos % 16] = a["k_cache"][bb, pos]
            b["v_cache"][pg, pos % 16] = a["v_cache"][bb, pos]
    for key in ("q", "k_tree", "v_tree", "parent"):
        b[key] = a[key]
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_bad_page_is_flagged_without_fault():
    inp = synth.make_attn_inputs(B=2, N=8, Hq=4, Hkv=1, D=128, dtype="bf16", prefix_lens=[40, 20],
                                 page_size=16, seed=1)
    inp["block_table"][1, 0] = inp["num_pages"] + 5   # out of range, caught by the kernel
    ps = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    run_gpu(inp, page_status=ps)
    assert int(ps.item()) == jf.JF_ERR_BAD_PAGE


def test_qwen3_8b_low_budget_full():
    compare(synth.make_workload(1, parts=("attn",))["attn"], label="qwen3-8b n16")


def test_qwen3_8b_high_budget_full():
    compare(synth.make_workload(2, parts=("attn",))["attn"], label="qwen3-8b n256")


@pytest.mark.parametrize("cus", [192, 64, 7])
def test_splits_planned_for_fewer_compute_units(cus):
    # jf_tree_attn_fwd_cus: fewer, longer key splits; same results to the
    # parity bar (all rows at 4096 prefix tokens and 256 nodes)
    compare(synth.make_workload(2, parts=("attn",))["attn"], label="qwen3-8b n256", cus=cus)


def test_serving_batch_fewer_compute_units_sampled():
    inp = synth.make_workload(3, parts=("attn",))["attn"]
    compare(inp, rows=_sample_rows(inp, 256, 5), label="serving b32", cus=192)


def _sample_rows(inp, n, seed):
    B, N, Hq, _ = inp["q"].shape
    return np.sort(np.random.default_rng(seed).choice(B * N * Hq, size=n, replace=False))


def test_serving_batch_full_size_sampled():
    inp = synth.make_workload(3, parts=("attn",))["attn"]
    compare(inp, rows=_sample_rows(inp, 512, 3), label="serving b32")


def test_qwen3_30b_shape_full_size_sampled():
    inp = synth.make_workload(4, parts=("attn",))["attn"]
    compare(inp, rows=_sample_rows(inp, 256, 4), label="qwen3-30b")


def test_score_jump_past_reference_maximum():
    # Keys after the first 64-key block are made to score far above it (a key
    # equal to 4 q gives a raw score of about 4 |q|^2 = 512 with D = 128, over
    # 2^32 in exp2 units above the first block's maximum of about 40), which
    # sends the first split of each (KV head, query tile) through its second
    # pass with the true maxima.  The oracle's softmax is exact, so the
    # output must still match it.
    inp = synth.make_attn_inputs(B=1, N=24, Hq=8, Hkv=2, D=128, dtype="bf16", prefix_lens=[640],
                                 seed=11)
    q = synth.bf16_bits_to_f32(inp["q"])              # [B, N, Hq, D]
    kc = synth.bf16_bits_to_f32(inp["k_cache"])       # [pages, page_size, Hkv, D]
    G = 8 // 2
    for p in range(64 + 5, 640, 64):                  # one key per block, never in block 0
        node = (p // 64) % 24
        for g in range(2):
            kc[0, p, g] = 4.0 * q[0, node, g * G]
    inp["k_cache"] = synth.f32_to_bf16_bits(kc)
    compare(inp, label="score jump")


def test_maximum_tree_size():
    # N = 1024 nodes, the call's limit: 16 tree blocks, 1024 * 4 query rows
    inp = synth.make_attn_inputs(B=1, N=1024, Hq=8, Hkv=2, D=128, dtype="bf16", prefix_lens=[512],
                                 seed=1024)
    rows = np.sort(np.random.default_rng(5).choice(1024 * 8, 1024, replace=False))
    compare(inp, rows=rows, label="N=1024")


def test_maximum_batch():
    # B = 256 sequences, the call's limit, ragged prefixes including empty ones
    pl = list(np.random.default_rng(256).integers(0, 200, size=256))
    pl[0] = 0
    inp = synth.make_attn_inputs(B=256, N=8, Hq=4, Hkv=1, D=128, dtype="bf16", prefix_lens=pl,
                                 page_size=16, shuffled_pages=True, seed=256)
    compare(inp, label="B=256")
