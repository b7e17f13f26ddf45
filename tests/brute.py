"""Independent numpy checkers used to pin the oracle (never the HIP path).

Each one reaches the same quantity as the oracle by a different route, so that
a plausible mistake in the oracle (a dropped key set, a wrong sign, a swapped
index) shows up as a disagreement.
"""
import numpy as np


def root_path(parent, i):
    """Tree nodes from the first node below the prefix down to node i."""
    path = []
    j = int(i)
    while j != -1:
        path.append(j)
        j = int(parent[j])
    return path[::-1]


def causal_attention(q, k, v, scale):
    """Textbook causal softmax attention: row r sees columns 0..r.

    q, k, v: [L, D] float64.  Returns out [L, D] and lse [L].
    """
    L = q.shape[0]
    s = (q @ k.T) * scale
    s = np.where(np.tril(np.ones((L, L), dtype=bool)), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ v) / z, (m + np.log(z))[:, 0]


def gather_prefix(k_cache, block_table, b, P, page_size):
    """Prefix rows of sequence b, in position order: [P, Hkv, D]."""
    pos = np.arange(P)
    pages = block_table[b, pos // page_size]
    return k_cache[pages, pos % page_size]


def path_attention(*, q, k_tree, v_tree, parent, k_cache, v_cache, block_table,
                   prefix_len, page_size, scale=None):
    """For every node: causal attention over [prefix ; root-to-node path] taken at
    its last position (the node itself), i.e. what one sequential drafting pass
    along that branch would compute.  All float64."""
    B, N, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, N, Hq))
    for b in range(B):
        P = int(prefix_len[b])
        kp = gather_prefix(k_cache, block_table, b, P, page_size)
        vp = gather_prefix(v_cache, block_table, b, P, page_size)
        for i in range(N):
            path = root_path(parent[b], i)
            for h in range(Hq):
                g = h // G
                kk = np.concatenate([kp[:, g], k_tree[b, path, g]], axis=0)
                vv = np.concatenate([vp[:, g], v_tree[b, path, g]], axis=0)
                # queries of the sequence: prefix positions get zeros (unused rows);
                # path positions get their own node's query; we read the last row.
                qq = np.zeros((kk.shape[0], D))
                qq[P:] = q[b, path, h]
                o, l = causal_attention(qq, kk, vv, scale)
                out[b, i, h] = o[-1]
                lse[b, i, h] = l[-1]
    return out, lse
