"""Shared test plumbing: widen generated inputs and call the oracle."""
import numpy as np

import oracle
from tree_causal_draft_parent_amd import synth


def attn_f64(inp):
    dt = inp["dtype"]
    f = {k: synth.to_f64(inp[k], dt) for k in ("q", "k_tree", "v_tree")}
    if inp.get("kv_dtype") == "fp8":
        f["k_cache"] = oracle.fp8_e4m3_to_f64(inp["k_cache"], inp["k_scale"])
        f["v_cache"] = oracle.fp8_e4m3_to_f64(inp["v_cache"], inp["v_scale"])
    else:
        f["k_cache"] = synth.to_f64(inp["k_cache"], dt)
        f["v_cache"] = synth.to_f64(inp["v_cache"], dt)
    return f


def oracle_attn(inp, rows=None, scale=None, prefix_len=None, bad_page_ok=False):
    f = attn_f64(inp)
    return oracle.tree_attn(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"],
                            parent=inp["parent"], k_cache=f["k_cache"], v_cache=f["v_cache"],
                            block_table=inp["block_table"],
                            prefix_len=inp["prefix_len"] if prefix_len is None else prefix_len,
                            page_size=inp["page_size"], scale=scale, rows=rows,
                            node_off=inp.get("node_off"), bad_page_ok=bad_page_ok)


def rel_rms(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((a - ref) ** 2)) / max(den, 1e-300))
