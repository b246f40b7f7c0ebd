"""HGA oracle, loop form: one (sequence, head, token) at a time in plain
Python floats (IEEE double).  For tiny shapes only.

TEST INFRASTRUCTURE ONLY (same rules as ``hga_oracle``).  It restates the
same definitions as the vectorized form token by token, so that a mistake in
one (a transposed operand, a wrong head mapping, an off-by-one in the causal
range) shows up as a disagreement between the two.  The page citations and
readings are the ones listed in ``hga_oracle``'s header.
"""

from __future__ import annotations

import math
from typing import Optional


def _summary(k, b, g, blk, Bh):
    D = len(k[b][g][0])
    acc = [0.0] * D
    for t in range(blk * Bh, (blk + 1) * Bh):
        row = k[b][g][t]
        for d in range(D):
            acc[d] += float(row[d])
    return [a / Bh for a in acc]


def _qmean(q, b, g, G, first, Bq):
    D = len(q[b][0][0])
    acc = [0.0] * D
    for h in range(g * G, (g + 1) * G):
        for t in range(first, first + Bq):
            row = q[b][h][t]
            for d in range(D):
                acc[d] += float(row[d])
    n = G * Bq
    return [a / n for a in acc]


def _select(scores, top_k):
    nb = len(scores)
    if nb <= top_k:
        chosen = list(range(nb))
    else:
        ranked = sorted(range(nb), key=lambda i: (-scores[i], i))
        chosen = sorted(ranked[:top_k])
    return chosen + [-1] * (top_k - len(chosen))


def run_loop(q, k, v, do, shape, scale: Optional[float] = None, bwd: bool = True):
    """Nested lists (or arrays) in, nested lists out:
    sel[b][g][jglobal][slot], o[b][h][t][d], lse[b][h][t], and if bwd
    dq[b][h][t][d], dk/dv[b][g][t][d]."""
    B, Hq, S, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    L, Bh, Bq, top_k = shape.seg_len, shape.hist_block, shape.query_block, shape.top_k
    sc = 1.0 / math.sqrt(D) if scale is None or scale <= 0 else scale
    nqb = L // Bq
    sel = [[[None] * (S // Bq) for _ in range(Hkv)] for _ in range(B)]
    o = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    dq = [[[[0.0] * D for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    dk = [[[[0.0] * D for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]
    dv = [[[[0.0] * D for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]

    def dot(x, y):
        return sum(float(a) * float(c) for a, c in zip(x, y))

    for b in range(B):
        for s in range(S // L):
            t0 = s * L
            nb = t0 // Bh
            summaries = [_summary(k, b, g, i, Bh) for g in range(Hkv) for i in range(nb)]
            for g in range(Hkv):
                for j in range(nqb):
                    qbar = _qmean(q, b, g, G, t0 + j * Bq, Bq)
                    scores = [dot(qbar, summaries[g * nb + i]) for i in range(nb)]
                    chosen = _select(scores, top_k)
                    sel[b][g][s * nqb + j] = chosen
                    hist = [blk * Bh + r for blk in chosen if blk >= 0 for r in range(Bh)]
                    for h in range(g * G, (g + 1) * G):
                        for t in range(t0 + j * Bq, t0 + (j + 1) * Bq):
                            keys = hist + list(range(t0, t + 1))
                            z = [sc * dot(q[b][h][t], k[b][g][i]) for i in keys]
                            m = max(z)
                            ssum = sum(math.exp(x - m) for x in z)
                            l_ = m + math.log(ssum)
                            p = [math.exp(x - l_) for x in z]
                            orow = [0.0] * D
                            for pi, i in zip(p, keys):
                                vi = v[b][g][i]
                                for d in range(D):
                                    orow[d] += pi * float(vi[d])
                            o[b][h][t] = orow
                            lse[b][h][t] = l_
                            if not bwd:
                                continue
                            dorow = [float(x) for x in do[b][h][t]]
                            delta = sum(a * c for a, c in zip(dorow, orow))
                            for pi, i in zip(p, keys):
                                dp = dot(dorow, v[b][g][i])
                                ds = pi * (dp - delta)
                                ki = k[b][g][i]
                                for d in range(D):
                                    dq[b][h][t][d] += sc * ds * float(ki[d])
                                if i >= t0:  # local key: receives gradient
                                    qrow = q[b][h][t]
                                    for d in range(D):
                                        dk[b][g][i][d] += sc * ds * float(qrow[d])
                                        dv[b][g][i][d] += pi * dorow[d]
    out = {"sel": sel, "o": o, "lse": lse}
    if bwd:
        out.update(dq=dq, dk=dk, dv=dv)
    return out
