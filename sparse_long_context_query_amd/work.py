"""Algorithmic work of one segmented HGA pass (for throughput reporting).

Counts only attended (query, key) pairs of the selected tokens, per query
head: a pair is "history" when the key comes from a selected history block
and "local" when it is a causal key of the active segment.
  forward   : 4*D FLOP per pair (q.k and p*v)
  backward  : 4*D per history pair (dO.v and dS*k for dq)
              8*D per local pair  (dO.v, dS*k, dS*q for dk, p*dO for dv)
The recomputation of q.k inside the backward is not counted (the
"with recompute" figure adds 2*D per pair).
"""

from __future__ import annotations


def pair_counts(shape, segments=None, groups=None):
    """(history pairs, local pairs) summed over segments and query heads.
    `groups` limits the count to a number of (sequence, KV head) groups."""
    L, Bh, k = shape.seg_len, shape.hist_block, shape.top_k
    G = shape.group
    ngroups = shape.batch * shape.n_kv_heads if groups is None else groups
    segs = range(shape.nseg) if segments is None else segments
    hist = loc = 0
    for s in segs:
        nb = s * L // Bh
        keff = min(k, nb)
        hist += ngroups * G * L * keff * Bh
        loc += ngroups * G * L * (L + 1) // 2
    return hist, loc


def flops(shape, segments=None, groups=None) -> dict:
    h, l_ = pair_counts(shape, segments, groups)
    D = shape.head_dim
    return {
        "hist_pairs": h,
        "local_pairs": l_,
        "fwd": 4 * D * (h + l_),
        "bwd": 4 * D * h + 8 * D * l_,
        "bwd_recompute": 6 * D * h + 10 * D * l_,
        "bwd_dq": 4 * D * (h + l_),     # dq kernel: dO.v and dS*k over every pair
        "bwd_dkdv": 4 * D * l_,         # dk/dv kernel: dS*q and p*dO over local pairs
    }


def dense_causal_flops(shape) -> dict:
    """Dense causal attention over the whole sequence at the same shape."""
    S, D = shape.seq_len, shape.head_dim
    pairs = shape.batch * shape.n_q_heads * S * (S + 1) // 2
    return {"fwd": 4 * D * pairs, "bwd": 8 * D * pairs}
