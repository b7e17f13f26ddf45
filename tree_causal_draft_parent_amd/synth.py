"""Seeded synthetic inputs for the tree-causal draft-head hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no masks, attention, projection or selection).  Both the
HIP path and the fp64 oracle take their inputs from here.

Workload shapes follow the draft budgets the pages discuss (16- and 256-token
trees, "Empirical Results" on the JetFlow blog page; low/high budget in the
arXiv page's section 1) and the Qwen3-8B / Qwen3-30B-A3B target shapes the
pages evaluate on.  Value distributions: queries, keys and values ~ N(0, 1);
projection weights ~ N(0, 0.02); fused hidden inputs ~ N(0, 1); draft logits
~ N(0, 4), the second argument always being the standard deviation.

bf16 tensors are produced by drawing float32 and rounding to nearest-even, and
are returned as ``uint16`` bit patterns; ``bf16_bits_to_f32`` widens them
exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# workload table
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    prefix: Sequence[int] | None  # fixed prefix length per sequence (None: ragged)
    prefix_range: tuple | None    # (lo, hi) inclusive, for ragged prefixes
    N: int
    max_depth: int
    branching: tuple              # (lo, hi) inclusive children per expansion
    Hq: int
    Hkv: int
    D: int
    dtype: str                    # "f32" or "bf16"
    H: int                        # hidden size of the fused projection (3H -> H)
    n_fused: int
    V: int                        # vocab of the per-node draft logits
    topk: int
    page_size: int                # 0: one contiguous region per sequence
    shuffled_pages: bool


WORKLOADS: Dict[int, Workload] = {
    # tiny fp32 tree, oracle-sized
    0: Workload("tiny-fp32-p64-n16", 1, (64,), None, 16, 5, (1, 3), 4, 2, 64,
                "f32", 256, 3, 1000, 4, 0, False),
    # Qwen3-8B-shaped draft layer, low budget (16 nodes)
    1: Workload("qwen3-8b-p1024-n16", 1, (1024,), None, 16, 8, (1, 4), 32, 8, 128,
                "bf16", 4096, 3, 151936, 8, 0, False),
    # Qwen3-8B-shaped draft layer, high budget (256 nodes)
    2: Workload("qwen3-8b-p4096-n256", 1, (4096,), None, 256, 16, (1, 8), 32, 8, 128,
                "bf16", 4096, 3, 151936, 8, 0, False),
    # serving batch: 32 sequences, ragged prefixes, paged KV in shuffled pages
    3: Workload("serving-b32-ragged-paged-n64", 32, None, (512, 8192), 64, 16, (1, 8),
                32, 8, 128, "bf16", 4096, 3, 151936, 8, 16, True),
    # Qwen3-30B-A3B-shaped draft layer, long prefix
    4: Workload("qwen3-30b-a3b-b4-p32768-n256", 4, (32768,) * 4, None, 256, 16, (1, 8),
                32, 4, 128, "bf16", 2048, 3, 151936, 8, 0, False),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# ----------------------------------------------------------------------------
# bf16 bit handling (round to nearest even; the data never holds NaN)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


# ----------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------


def best_first_tree(rng: np.random.Generator, N: int, max_depth: int,
                    branching: tuple) -> np.ndarray:
    """A parent array of N nodes grown best-first, as a drafter would grow it.

    The prefix end is a virtual root (id -1, path log-probability 0, depth 0).
    Repeatedly take the frontier entry with the highest path log-probability
    (ties: lower id, the virtual root ranking lowest-id) and give it c children,
    c uniform in ``branching``.  The children's conditional probabilities are a
    seeded softmax sorted in descending order; a child's path log-probability is
    its parent's plus the log of its own conditional.  Children shallower than
    ``max_depth`` join the frontier.  If the frontier runs dry, the virtual root
    is offered again (the result is then a forest of prefix children).  Node ids
    are creation order, so every parent id is smaller than its child's.
    """
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    score = np.zeros(N, dtype=np.float64)
    frontier: List[int] = [-1]  # node ids; -1 is the virtual root
    count = 0
    lo, hi = branching
    while count < N:
        if not frontier:
            frontier.append(-1)

        def key(nid: int):
            s = 0.0 if nid < 0 else score[nid]
            return (-s, nid)

        frontier.sort(key=key)
        p = frontier.pop(0)
        c = int(rng.integers(lo, hi + 1))
        c = min(c, N - count)
        logits = rng.standard_normal(c) * 2.0
        prob = np.exp(logits - logits.max())
        prob = np.sort(prob / prob.sum())[::-1]
        pd = 0 if p < 0 else depth[p]
        ps = 0.0 if p < 0 else score[p]
        for r in range(c):
            nid = count
            parent[nid] = p
            depth[nid] = pd + 1
            score[nid] = ps + float(np.log(prob[r]))
            count += 1
            if depth[nid] < max_depth:
                frontier.append(nid)
    return parent


def chain_tree(N: int) -> np.ndarray:
    p = np.arange(-1, N - 1, dtype=np.int32)
    return p


def star_tree(N: int) -> np.ndarray:
    return np.full(N, -1, dtype=np.int32)


# ----------------------------------------------------------------------------
# full input sets
# ----------------------------------------------------------------------------


def _seeds(seed: int, names: Sequence[str]) -> Dict[str, np.random.Generator]:
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(names, children)}


_STREAMS = ("tree", "prefix_len", "pages", "q", "k_tree", "v_tree", "k_cache",
            "v_cache", "x", "w", "logits")


def f32_to_fp8_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities, max 448) codes of float32 values,
    rounded to nearest even and clamped to +-448; the data never holds NaN.
    Code layout: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
    exponent 0 holds the subnormals m * 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), 448.0)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)         # 0..8 (8: the least normal)
    f, E = np.frexp(a[~sub])                                           # a = f * 2^E, f in [0.5, 1)
    e = E - 1                                                          # a in [2^e, 2^(e+1))
    m = np.rint(a[~sub] / np.ldexp(1.0, e - 3)).astype(np.int64)       # 8..16, ties to even
    up = m == 16
    e, m = np.where(up, e + 1, e), np.where(up, 8, m)
    code[~sub] = ((e + 7) << 3) | (m - 8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def _draw_fp8(rng: np.random.Generator, shape) -> tuple:
    """N(0, 1) values as E4M3 codes with one per-tensor scale (max |x| / 448):
    value = decoded code * scale."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    scale = float(np.float32(max(float(np.max(np.abs(x))), 1e-30) / 448.0))
    return f32_to_fp8_e4m3_codes(x.astype(np.float64) / scale), scale


def make_attn_inputs(*, B: int, N: int, Hq: int, Hkv: int, D: int, dtype: str,
                     prefix_lens: Sequence[int], page_size: int = 0,
                     shuffled_pages: bool = False, parents: Optional[np.ndarray] = None,
                     max_depth: int = 16, branching: tuple = (1, 8),
                     seed: int = 1234, extra_pages: int = 0,
                     node_counts: Optional[Sequence[int]] = None,
                     kv_dtype: Optional[str] = None) -> dict:
    """Inputs of one tree-attention call.

    Prefix K/V live in a page pool ``[num_pages, page_size, Hkv, D]`` addressed
    through ``block_table[B, max_pages]`` (padding -1).  ``page_size == 0`` asks
    for the contiguous form: one page per sequence, ``page_size = max(P)``, page
    id = sequence id.

    ``node_counts`` (one tree size per sequence) asks for packed trees:
    sequence b owns rows ``node_off[b] .. node_off[b+1]-1`` of q ``[T, Hq, D]``,
    k_tree / v_tree ``[T, Hkv, D]`` and parent ``[T]`` (parents local to the
    sequence), and ``N`` becomes the largest count.  ``kv_dtype="fp8"`` draws
    the prefix cache as E4M3 codes (uint8) with per-tensor scales ``k_scale``
    and ``v_scale`` (value = decoded code * scale).
    """
    rng = _seeds(seed, _STREAMS)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32)
    assert prefix_lens.shape == (B,)
    packed = node_counts is not None
    if packed:
        counts = np.asarray(node_counts, dtype=np.int64)
        assert counts.shape == (B,) and np.all(counts >= 1)
        node_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        N = int(counts.max())
        if parents is None:
            parents = np.concatenate([best_first_tree(rng["tree"], int(n), max_depth, branching)
                                      for n in counts]).astype(np.int32)
        parents = np.asarray(parents, dtype=np.int32).reshape(int(node_off[-1]))
        rows = (int(node_off[-1]),)
    else:
        node_off = None
        if parents is None:
            parents = np.stack([best_first_tree(rng["tree"], N, max_depth, branching)
                                for _ in range(B)]).astype(np.int32)
        parents = np.asarray(parents, dtype=np.int32).reshape(B, N)
        rows = (B, N)
    Pmax = int(prefix_lens.max()) if B > 0 else 0
    if page_size == 0:
        ps = max(Pmax, 1)
        max_pages = 1
        num_pages = B + extra_pages
        block_table = np.arange(B, dtype=np.int32).reshape(B, 1)
    else:
        ps = page_size
        npg = [(int(p) + ps - 1) // ps for p in prefix_lens]
        max_pages = max(max(npg) if npg else 0, 1)
        num_pages = int(sum(npg)) + extra_pages
        ids = np.arange(num_pages, dtype=np.int32)
        if shuffled_pages:
            ids = rng["pages"].permutation(ids).astype(np.int32)
        block_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            block_table[b, :npg[b]] = ids[off:off + npg[b]]
            off += npg[b]
    q = _draw(rng["q"], rows + (Hq, D), 1.0, dtype)
    k_tree = _draw(rng["k_tree"], rows + (Hkv, D), 1.0, dtype)
    v_tree = _draw(rng["v_tree"], rows + (Hkv, D), 1.0, dtype)
    out = dict(B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, page_size=ps,
               max_pages=max_pages, num_pages=num_pages, prefix_len=prefix_lens,
               parent=parents, block_table=block_table, q=q, k_tree=k_tree,
               v_tree=v_tree, node_off=node_off, kv_dtype=kv_dtype or dtype)
    if kv_dtype == "fp8":
        out["k_cache"], out["k_scale"] = _draw_fp8(rng["k_cache"], (num_pages, ps, Hkv, D))
        out["v_cache"], out["v_scale"] = _draw_fp8(rng["v_cache"], (num_pages, ps, Hkv, D))
    else:
        assert kv_dtype in (None, dtype)
        out["k_cache"] = _draw(rng["k_cache"], (num_pages, ps, Hkv, D), 1.0, dtype)
        out["v_cache"] = _draw(rng["v_cache"], (num_pages, ps, Hkv, D), 1.0, dtype)
    return out


def make_fuse_inputs(*, M: int, H_in: int, H_out: int, n_fused: int, dtype: str,
                     seed: int = 1234, w_std: float = 0.02) -> dict:
    rng = _seeds(seed, _STREAMS)
    x = _draw(rng["x"], (n_fused, M, H_in), 1.0, dtype)
    w = _draw(rng["w"], (H_out, n_fused * H_in), w_std, dtype)
    return dict(M=M, H_in=H_in, H_out=H_out, n_fused=n_fused, dtype=dtype, x=x, w=w)


def make_logits(*, R: int, V: int, dtype: str, seed: int = 1234, std: float = 4.0) -> np.ndarray:
    rng = _seeds(seed, _STREAMS)
    return _draw(rng["logits"], (R, V), std, dtype)


def tie_forcing_logits(logits_bits: np.ndarray, dtype: str) -> np.ndarray:
    """Round draft logits to integers so that many values repeat (tie stress)."""
    x = bf16_bits_to_f32(logits_bits) if dtype == "bf16" else np.asarray(logits_bits, np.float32)
    x = np.rint(x).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_path_inputs(*, B: int, N: int, max_depth: int = 16, branching=(1, 8),
                     seed: int = 1234) -> dict:
    """Best-first parent arrays and each node's conditional log-probability of
    its own token (float32, -|N(0, 2)|)."""
    rng = _seeds(seed, ("tree", "logp"))
    parents = np.stack([best_first_tree(rng["tree"], N, max_depth, branching) for _ in range(B)])
    logp = (-np.abs(rng["logp"].standard_normal((B, N)) * 2.0)).astype(np.float32)
    return dict(parent=parents.astype(np.int32), logp=logp)


def make_expand_inputs(*, B: int, N: int, k: int, V: int = 151936, max_depth: int = 16,
                       seed: int = 1234, ties: bool = False, child_frac: float = 0.5) -> dict:
    """Inputs of one expansion step: the current nodes' path scores (float32,
    N(-5, 3)), depths U{1..max_depth}, and per-node top-k lists as the top-k
    call returns them (distinct token ids U[0, V), values N(8, 3) in
    descending order) with a row log-normaliser above the row's largest value.
    ties=True rounds scores, values and normalisers to integers so that many
    candidates tie.  The tree the step grows: a forest in creation order
    (parent -1 with probability 1/4, else a uniform earlier node); a child
    carries one of its parent's listed tokens not taken by a sibling with
    probability child_frac, else a token its parent does not list; siblings'
    tokens are distinct."""
    rng = _seeds(seed, ("score", "depth", "idx", "val", "lse", "parent", "token"))
    score = rng["score"].standard_normal((B, N)) * 3.0 - 5.0
    depth = rng["depth"].integers(1, max_depth + 1, size=(B, N)).astype(np.int32)
    idx = np.empty((B, N, k), np.int32)
    for b in range(B):
        for i in range(N):
            idx[b, i] = rng["idx"].choice(V, size=k, replace=False)
    val = np.sort(rng["val"].standard_normal((B, N, k)) * 3.0 + 8.0, axis=-1)[..., ::-1]
    lse = val[..., 0] + rng["lse"].uniform(0.0, 3.0, size=(B, N))
    if ties:
        score, val, lse = np.round(score), np.round(val), np.ceil(lse)
    parent = np.full((B, N), -1, np.int32)
    token = np.empty((B, N), np.int32)
    rp, rt = rng["parent"], rng["token"]
    for b in range(B):
        used = {}                                   # parent -> tokens its children carry
        for i in range(N):
            p = -1 if i == 0 or rp.random() < 0.25 else int(rp.integers(0, i))
            parent[b, i] = p
            taken = used.setdefault(p, set())
            listed = set(int(t) for t in idx[b, p]) if p >= 0 else set()
            free = [t for t in idx[b, p] if int(t) not in taken] if p >= 0 else []
            if free and rt.random() < child_frac:
                t = int(free[int(rt.integers(len(free)))])
            else:
                t = int(rt.integers(0, V))
                while t in listed or t in taken:
                    t = int(rt.integers(0, V))
            token[b, i] = t
            taken.add(t)
    return dict(score=score.astype(np.float32), depth=depth, idx=idx,
                val=np.ascontiguousarray(val, dtype=np.float32), lse=lse.astype(np.float32),
                max_depth=max_depth, parent=parent, token=token)


def make_verify_inputs(parent: np.ndarray, *, q: float = 0.9, seed: int = 1234) -> dict:
    """Draft tokens and target tokens for greedy verification of the trees
    `parent` [B, N]: sibling tokens are distinct draws from [0, 1000); the
    target's next token after a node is one of its children's tokens with
    probability q, else a token in [1000, 2000) that no node carries; after
    the prefix it is one root's token with probability 0.9, else 5000."""
    rng = _seeds(seed, ("tok", "nxt", "root"))
    B, N = parent.shape
    tok = np.zeros((B, N), np.int32)
    nxt = rng["nxt"].integers(1000, 2000, size=(B, N)).astype(np.int32)
    root = np.full(B, 5000, np.int32)
    for b in range(B):
        kids_of = {}
        for i, p in enumerate(parent[b]):
            kids_of.setdefault(int(p), []).append(i)
        for p, kids in kids_of.items():
            tok[b, kids] = rng["tok"].choice(1000, size=len(kids), replace=False)
        for j in range(N):
            kids = kids_of.get(j)
            if kids and rng["nxt"].random() < q:
                nxt[b, j] = tok[b, kids[rng["nxt"].integers(len(kids))]]
        roots = kids_of.get(-1, [])
        if roots and rng["root"].random() < 0.9:
            root[b] = tok[b, roots[rng["root"].integers(len(roots))]]
    return dict(token=tok, target_next=nxt, root_next=root)


def config_seed(i: int) -> int:
    return 1000 + i


def prefix_lengths(i: int, seed: Optional[int] = None) -> np.ndarray:
    w = WORKLOADS[i]
    if w.prefix is not None:
        return np.asarray(w.prefix, dtype=np.int32)
    rng = _seeds(config_seed(i) if seed is None else seed, _STREAMS)["prefix_len"]
    lo, hi = w.prefix_range
    return rng.integers(lo, hi + 1, size=w.B).astype(np.int32)


def make_workload(i: int, parts=("attn", "fuse", "topk"), seed: Optional[int] = None) -> dict:
    """All inputs of one draft step for workload ``i``.

    The fused projection runs over one row per tree node (M = B*N); the logits
    hold one row per tree node as well.
    """
    w = WORKLOADS[i]
    s = config_seed(i) if seed is None else seed
    out = {"workload": w, "seed": s}
    if "attn" in parts:
        out["attn"] = make_attn_inputs(
            B=w.B, N=w.N, Hq=w.Hq, Hkv=w.Hkv, D=w.D, dtype=w.dtype,
            prefix_lens=prefix_lengths(i, seed), page_size=w.page_size,
            shuffled_pages=w.shuffled_pages, max_depth=w.max_depth,
            branching=w.branching, seed=s)
    if "fuse" in parts:
        out["fuse"] = make_fuse_inputs(M=w.B * w.N, H_in=w.H, H_out=w.H,
                                       n_fused=w.n_fused, dtype=w.dtype, seed=s + 7)
    if "topk" in parts:
        out["logits"] = make_logits(R=w.B * w.N, V=w.V, dtype=w.dtype, seed=s + 13)
    return out
