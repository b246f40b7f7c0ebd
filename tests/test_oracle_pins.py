"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form, a brute-force count, an
independent library routine (torch's CPU scaled_dot_product_attention and
autograd in float64), finite differences, or the generator's construction.
They are chosen so that a plausible mistake (a dropped term, a wrong sign,
a transposed operand, a wrong head mapping, an off-by-one in the causal
range, a wrong tie rule) fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import hga_loop, hga_oracle as orc
from synth import HGAShape, WORKLOADS, make_inputs


def small_shape(**kw):
    base = dict(name="t", batch=1, seq_len=64, n_q_heads=2, n_kv_heads=1,
                head_dim=8, seg_len=16, hist_block=8, query_block=8, top_k=2,
                dtype="f32")
    base.update(kw)
    return HGAShape(**base)


# ---------------------------------------------------------------- summaries
def test_summaries_closed_form():
    """K = 3 + 2*t - d (integers): the mean of block i is the midpoint
    3 + 2*(i*Bh + (Bh-1)/2) - d exactly."""
    B, H, S, D, Bh = 2, 3, 96, 5, 16
    t = np.arange(S)[None, None, :, None]
    d = np.arange(D)[None, None, None, :]
    k = np.broadcast_to(3.0 + 2.0 * t - d + 0 * np.arange(B)[:, None, None, None]
                        + 7.0 * np.arange(H)[None, :, None, None], (B, H, S, D))
    kbar = orc.block_summaries(k, Bh)
    i = np.arange(S // Bh)[None, None, :, None]
    expect = 3.0 + 2.0 * (i * Bh + (Bh - 1) / 2.0) - d + 7.0 * np.arange(H)[None, :, None, None]
    assert kbar.shape == (B, H, S // Bh, D)
    np.testing.assert_array_equal(kbar, np.broadcast_to(expect, kbar.shape))


def test_query_means_closed_form():
    """Q = h + 0.5*t + 10*d: the mean over the G heads of group g and the
    Bq tokens of block j is (g*G + (G-1)/2) + 0.5*(first + (Bq-1)/2) + 10*d."""
    B, Hq, Hkv, S, D = 1, 8, 2, 64, 4
    G = Hq // Hkv
    h = np.arange(Hq)[None, :, None, None]
    t = np.arange(S)[None, None, :, None]
    d = np.arange(D)[None, None, None, :]
    q = np.broadcast_to(h + 0.5 * t + 10.0 * d, (B, Hq, S, D)).astype(np.float64)
    t0, L, Bq = 32, 32, 8
    qbar = orc.query_means(q, Hkv, t0, L, Bq)
    for g in range(Hkv):
        for j in range(L // Bq):
            first = t0 + j * Bq
            exp = (g * G + (G - 1) / 2.0) + 0.5 * (first + (Bq - 1) / 2.0) + 10.0 * np.arange(D)
            np.testing.assert_allclose(qbar[0, g, j], exp, rtol=0, atol=1e-12)


# ----------------------------------------------------------------- top-k
def brute_topk(scores, k):
    """Rank of i = #{i' : s_i' > s_i or (s_i' == s_i and i' < i)};
    keep rank < k; emit ascending, -1 padded."""
    nb = len(scores)
    keep = [i for i in range(nb)
            if sum(1 for j in range(nb)
                   if scores[j] > scores[i] or (scores[j] == scores[i] and j < i)) < k]
    keep = sorted(keep)
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("nb,k", [(0, 3), (2, 3), (3, 3), (7, 3), (20, 1), (33, 8), (64, 32)])
def test_topk_matches_bruteforce_random(nb, k):
    rng = np.random.default_rng(nb * 100 + k)
    for _ in range(20):
        s = rng.standard_normal(nb)
        assert list(orc.topk_blocks(s, k)) == brute_topk(list(s), k)


@pytest.mark.parametrize("nb,k", [(10, 3), (16, 5), (40, 8), (9, 9), (12, 11)])
def test_topk_ties_go_to_lower_index(nb, k):
    """Heavy exact ties (integer scores drawn from 3 values)."""
    rng = np.random.default_rng(nb + 7 * k)
    for _ in range(30):
        s = rng.integers(-1, 2, size=nb).astype(np.float64)
        got = list(orc.topk_blocks(s, k))
        assert got == brute_topk(list(s), k)


def test_topk_all_equal_takes_first_k():
    assert list(orc.topk_blocks(np.zeros(10), 4)) == [0, 1, 2, 3]
    assert list(orc.topk_blocks(np.array([1.0, 2.0, 2.0, 1.0, 2.0]), 2)) == [1, 2]


def test_topk_exhaustive_tiny():
    """Every score vector over {0,1,2}^5 and every k: matches brute force."""
    for s in itertools.product([0.0, 1.0, 2.0], repeat=5):
        for k in range(1, 6):
            assert list(orc.topk_blocks(np.array(s), k)) == brute_topk(list(s), k)


# ------------------------------------------------------- planted selection
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_2k"])
def test_selection_recovers_planted_blocks(name):
    """The generator plants min(k, nb) blocks per segment along the
    segment's direction; the oracle's selection must be exactly that set
    for every query block and KV head."""
    shape = WORKLOADS[name]
    inp = make_inputs(shape, seed=0)
    for s in range(shape.nseg):
        sel = orc.select_segment(inp["q"], inp["k"], shape, s)
        planted = inp["planted"][0][s]
        want = list(planted) + [-1] * (shape.top_k - len(planted))
        for g in range(shape.n_kv_heads):
            for j in range(shape.n_qblocks):
                assert list(sel[0, g, j]) == want, (s, g, j)


# ------------------------------------------------------ selection gap
def _gap_inputs(score_rows, G=1, Bq=2, Bh=2, D=3):
    """q, k and a shape whose block scores are exactly score_rows[j][i]:
    block i's keys all equal (score_rows[0][i], score_rows[1][i], ...) in
    the first len(score_rows) coordinates, and the queries of query block j
    of the last segment are e_j (every head, every token).  Integer and
    dyadic values only, so every mean and dot product is exact."""
    rows = np.asarray(score_rows, dtype=np.float64)
    nqb, nb = rows.shape
    L = nqb * Bq
    assert L % Bh == 0 and nqb <= D
    nb_seg = L // Bh
    nseg = -(-nb // nb_seg) + 1
    S = nseg * L
    seg = nseg - 1
    shape = HGAShape("gap", 1, S, G, 1, D, L, Bh, Bq, 1, "f32")
    q = np.zeros((1, G, S, D))
    k = np.zeros((1, 1, S, D))
    t0 = seg * L
    for j in range(nqb):
        q[0, :, t0 + j * Bq:t0 + (j + 1) * Bq, j] = 1.0
    for i in range(nb):
        k[0, 0, i * Bh:(i + 1) * Bh, :nqb] = rows[:, i]
    # blocks between the given ones and the segment start score a large
    # negative value, below every given score
    for i in range(nb, t0 // Bh):
        k[0, 0, i * Bh:(i + 1) * Bh, :nqb] = -1000.0
    return q, k, shape, seg


@pytest.mark.parametrize("scores,top_k,expect", [
    # sorted: 5, 3, 3, 2.5, 1 -> k=3: 3 - 2.5; an off-by-one would read
    # 3 - 3 = 0 (k-1 / k) or 2.5 - 1 = 1.5 (k+1 / k+2)
    ([[3, 5, 1, 2.5, 3]], 3, 0.5),
    ([[3, 5, 1, 2.5, 3]], 2, 0.0),            # tie of 3, 3 across the boundary
    ([[3, 5, 1, 2.5, 3]], 1, 2.0),
    ([[3, 5, 1, 2.5, 3]], 4, 1.5),
    ([[4, 4, 4, 4]], 2, 0.0),                 # all tied
    ([[-1, -2, -0.5, -4]], 2, 1.0),           # negative scores: -0.5, -1 | -2
    ([[-1, -2, -0.5, -4]], 1, 0.5),           # -0.5 | -1
    # two query blocks: the smaller of their gaps (row 1: 7, 6.75 | 2)
    ([[3, 5, 1, 2.5, 3], [7, 2, 6.75, 0, 1]], 2, 0.0),
    ([[9, 5, 1, 2.5, 3], [7, 2, 6.75, 0, 1]], 2, 2.0),   # row 0: 9, 5 | 3; row 1: 4.75
    ([[9, 5, 1, 2.5, 3], [7, 2, 6.75, 0, 1]], 3, 0.5),   # row 0: 3 | 2.5; row 1: 2 | 1
])
def test_selection_gap_hand_built(scores, top_k, expect):
    """selection_gap on block scores fixed by construction (exact values):
    the gap between the k-th and (k+1)-th largest score, minimum over the
    segment's query blocks, 0 for a tie across the boundary."""
    q, k, shape, seg = _gap_inputs(scores, G=2)
    nb = len(scores[0])
    shape = shape.replace(top_k=top_k)
    # the padding blocks (score -1000) sit below every given score, so the
    # gap is decided by the given ones whenever k < nb
    assert top_k < nb
    assert orc.selection_gap(q, k, shape, seg) == expect


def test_selection_gap_inf_when_all_taken():
    """nb <= k: every history block is taken, there is no boundary."""
    q, k, shape, seg = _gap_inputs([[3, 5, 1, 2.5]])
    nb = shape.n_hist_blocks(seg)
    assert orc.selection_gap(q, k, shape.replace(top_k=nb), seg) == math.inf
    assert orc.selection_gap(q, k, shape.replace(top_k=nb + 5), seg) == math.inf
    assert orc.selection_gap(q, k, shape.replace(top_k=nb - 1), seg) < math.inf
    assert orc.selection_gap(q, k, shape.replace(top_k=1), 0) == math.inf


def _loop_gap(q, k, shape, seg):
    """The k-th boundary gap written with explicit loops: block means, the
    group-and-token mean query, every score, then a selection sort of the
    scores (largest first) and the difference of places k and k+1."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    L, Bh, Bq, kk = shape.seg_len, shape.hist_block, shape.query_block, shape.top_k
    t0 = seg * L
    nb = t0 // Bh
    if nb <= kk:
        return math.inf
    best = math.inf
    for b in range(B):
        for g in range(Hkv):
            kbar = []
            for i in range(nb):
                m = [0.0] * D
                for t in range(i * Bh, (i + 1) * Bh):
                    for d in range(D):
                        m[d] += float(k[b, g, t, d])
                kbar.append([x / Bh for x in m])
            for j in range(L // Bq):
                qb = [0.0] * D
                for h in range(g * G, (g + 1) * G):
                    for t in range(t0 + j * Bq, t0 + (j + 1) * Bq):
                        for d in range(D):
                            qb[d] += float(q[b, h, t, d])
                qb = [x / (G * Bq) for x in qb]
                sc = [sum(qb[d] * kbar[i][d] for d in range(D)) for i in range(nb)]
                for a in range(kk + 1):       # selection sort of the first k+1 places
                    m = max(range(a, nb), key=lambda i: sc[i])
                    sc[a], sc[m] = sc[m], sc[a]
                best = min(best, sc[kk - 1] - sc[kk])
    return best


@pytest.mark.parametrize("seed", range(4))
def test_selection_gap_loop_form(seed):
    """Random inputs (GQA, batch 2, several query blocks): selection_gap
    equals the loop-written gap to rounding."""
    shape = small_shape(batch=2, n_q_heads=4, n_kv_heads=2, seq_len=96, seg_len=32,
                        hist_block=4, query_block=8, top_k=3)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, 4, 96, 8))
    k = rng.standard_normal((2, 2, 96, 8))
    for seg in range(shape.nseg):
        a = orc.selection_gap(q, k, shape, seg)
        b = _loop_gap(q, k, shape, seg)
        if math.isinf(b):
            assert math.isinf(a)
        else:
            assert abs(a - b) <= 1e-12, (seg, a, b)
    # and with the summaries handed in
    kbar = orc.block_summaries(k, shape.hist_block)
    assert orc.selection_gap(q, k, shape, 2, kbar=kbar) == orc.selection_gap(q, k, shape, 2)


@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_2k", "train_16k", "infer_131k",
                                  "batch4_32k"])
def test_generator_gap_and_fp32_selection(name):
    """Every workload's planted inputs keep a gap of at least 1e-3 at the
    k-th boundary of every (sequence, KV head, query block) with more
    history blocks than k, and fp32 scoring picks the fp64 sets."""
    shape = WORKLOADS[name]
    inp = make_inputs(shape, seed=0, with_do=False)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    for s in range(shape.nseg):
        gap = orc.selection_gap(inp["q"], inp["k"], shape, s, kbar=kbar)
        assert gap >= 1e-3, (s, gap)
        a = orc.select_segment(inp["q"], inp["k"], shape, s, precision="f64", kbar=kbar)
        b = orc.select_segment(inp["q"], inp["k"], shape, s, precision="f32", kbar=kbar)
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- forward
def _torch_sdpa(q, k, v, mask=None, causal=False):
    """torch CPU float64 SDPA with GQA expanded by repeat_interleave."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    kt = torch.as_tensor(k, dtype=torch.float64).repeat_interleave(G, dim=1)
    vt = torch.as_tensor(v, dtype=torch.float64).repeat_interleave(G, dim=1)
    qt = torch.as_tensor(q, dtype=torch.float64)
    m = None if mask is None else torch.as_tensor(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, is_causal=causal).numpy()


@pytest.mark.parametrize("shape", [
    small_shape(top_k=8),                                       # k covers all
    small_shape(n_q_heads=4, n_kv_heads=2, top_k=100, seq_len=96, seg_len=32,
                hist_block=16, query_block=8),
    small_shape(seq_len=32, seg_len=32, top_k=1),               # one segment
])
def test_forward_equals_dense_causal_when_k_covers_history(shape):
    inp = make_inputs(shape, seed=3)
    out = orc.run(inp, bwd=False)
    ref = _torch_sdpa(inp["q"], inp["k"], inp["v"], causal=True)
    np.testing.assert_allclose(out["o"], ref, rtol=0, atol=1e-12)


def _hga_mask(sel, shape, seg):
    """Boolean [B,Hq,L,t0+L] visibility mask of segment `seg` built from
    the selection: history token visible iff its block is selected for the
    query's (KV head, query block); local token visible iff not after the
    query."""
    B, Hkv, nqb, k = sel.shape
    G = shape.group
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    t0 = seg * L
    m = np.zeros((B, shape.n_q_heads, L, t0 + L), dtype=bool)
    for b in range(B):
        for h in range(shape.n_q_heads):
            g = h // G
            for r in range(L):
                j = r // Bq
                for blk in sel[b, g, j]:
                    if blk >= 0:
                        m[b, h, r, blk * Bh:(blk + 1) * Bh] = True
                m[b, h, r, t0:t0 + r + 1] = True
    return m


@pytest.mark.parametrize("shape", [
    small_shape(),
    small_shape(n_q_heads=4, n_kv_heads=2, seq_len=96, seg_len=32, hist_block=16,
                query_block=8, top_k=3, head_dim=16),
    small_shape(batch=2, hist_block=4, query_block=16, top_k=5),
])
def test_forward_and_backward_match_torch_masked_sdpa_with_detached_history(shape):
    """For every segment: O equals torch SDPA with the selection mask, and
    dQ, dK, dV of the segment rows equal torch autograd of the same SDPA
    with the history keys/values detached (loss = sum(O * dO))."""
    inp = make_inputs(shape, seed=11)
    out = orc.run(inp)
    G = shape.group
    for s in range(shape.nseg):
        t0, L = s * shape.seg_len, shape.seg_len
        nqb = shape.n_qblocks
        sel = out["sel"][:, :, s * nqb:(s + 1) * nqb]
        mask = torch.as_tensor(_hga_mask(sel, shape, s))
        q = torch.tensor(inp["q"][:, :, t0:t0 + L], dtype=torch.float64, requires_grad=True)
        kl = torch.tensor(inp["k"][:, :, t0:t0 + L], dtype=torch.float64, requires_grad=True)
        vl = torch.tensor(inp["v"][:, :, t0:t0 + L], dtype=torch.float64, requires_grad=True)
        kh = torch.tensor(inp["k"][:, :, :t0], dtype=torch.float64)   # detached history
        vh = torch.tensor(inp["v"][:, :, :t0], dtype=torch.float64)
        kc = torch.cat([kh, kl], dim=2).repeat_interleave(G, dim=1)
        vc = torch.cat([vh, vl], dim=2).repeat_interleave(G, dim=1)
        o = torch.nn.functional.scaled_dot_product_attention(q, kc, vc, attn_mask=mask)
        do = torch.tensor(inp["do"][:, :, t0:t0 + L], dtype=torch.float64)
        (o * do).sum().backward()
        np.testing.assert_allclose(out["o"][:, :, t0:t0 + L], o.detach().numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(out["dq"][:, :, t0:t0 + L], q.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(out["dk"][:, :, t0:t0 + L], kl.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(out["dv"][:, :, t0:t0 + L], vl.grad.numpy(), atol=1e-11, rtol=0)


def test_uniform_attention_closed_form():
    """Q lives in the first half of the feature dims and K in the second, so
    every logit and every block score is exactly 0: selection takes the
    first min(k, nb) blocks (ties to the lower index), O is the plain mean
    of V over (selected tokens + local tokens up to the query) and LSE is
    ln(count)."""
    shape = small_shape(seq_len=96, seg_len=32, hist_block=8, query_block=8,
                        top_k=3, n_q_heads=4, n_kv_heads=2, head_dim=8)
    rng = np.random.default_rng(5)
    D = shape.head_dim
    q = rng.standard_normal((1, 4, 96, D))
    k = rng.standard_normal((1, 2, 96, D))
    q[..., D // 2:] = 0.0
    k[..., :D // 2] = 0.0
    v = rng.standard_normal((1, 2, 96, D))
    out = orc.run({"q": q, "k": k, "v": v, "do": None, "shape": shape}, bwd=False)
    L, Bh, kk = shape.seg_len, shape.hist_block, shape.top_k
    for s in range(shape.nseg):
        t0 = s * L
        nb = t0 // Bh
        first = list(range(min(kk, nb)))
        for j in range(shape.n_qblocks):
            assert list(out["sel"][0, 0, s * shape.n_qblocks + j]) == first + [-1] * (kk - len(first))
        hist = [b * Bh + r for b in first for r in range(Bh)]
        for h in range(4):
            g = h // 2
            for t in range(t0, t0 + L):
                keys = hist + list(range(t0, t + 1))
                np.testing.assert_allclose(out["o"][0, h, t], v[0, g, keys].mean(axis=0), atol=1e-13)
                assert abs(out["lse"][0, h, t] - math.log(len(keys))) < 1e-13


def test_softmax_rows_sum_to_one():
    shape = small_shape(n_q_heads=4, n_kv_heads=2, top_k=3)
    inp = make_inputs(shape, seed=2)
    out = orc.run(inp, bwd=False)
    D = shape.head_dim
    sc = 1.0 / math.sqrt(D)
    for s in range(shape.nseg):
        t0 = s * shape.seg_len
        for h in range(4):
            g = h // 2
            for t in range(t0, t0 + shape.seg_len):
                j = s * shape.n_qblocks + (t - t0) // shape.query_block
                keys, _ = orc.key_indices(out["sel"][0, g, j], shape.hist_block, t0, shape.seg_len)
                keys = keys[keys <= t]
                z = sc * inp["k"][0, g, keys].astype(np.float64) @ inp["q"][0, h, t].astype(np.float64)
                assert abs(np.exp(z - out["lse"][0, h, t]).sum() - 1.0) < 1e-13


# --------------------------------------------------------------- backward
def test_backward_matches_central_finite_differences():
    """loss_s = sum over segment s of O * dO, with the selection held fixed
    and history rows held constant.  Central differences (h = 1e-6) on 240
    random coordinates of the segment's Q, K and V rows."""
    shape = small_shape(n_q_heads=4, n_kv_heads=2, top_k=2)
    inp = make_inputs(shape, seed=9)
    q, k, v, do = (inp[x].astype(np.float64) for x in ("q", "k", "v", "do"))
    rng = np.random.default_rng(0)
    L = shape.seg_len
    for s in range(shape.nseg):
        t0 = s * L
        sel = orc.select_segment(q, k, shape, s)
        dq, dk, dv = orc.segment_backward(q, k, v, do, sel, shape, s)

        def loss(qq, kk2, vv):
            o, _ = orc.segment_forward(qq, kk2, vv, sel, shape, s)
            return float((o * do[:, :, t0:t0 + L]).sum())

        h = 1e-6
        for which, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            for _ in range(20):
                b = 0
                hh = rng.integers(arr.shape[1])
                t = t0 + rng.integers(L)
                d = rng.integers(arr.shape[3])
                xp = arr.copy(); xp[b, hh, t, d] += h
                xm = arr.copy(); xm[b, hh, t, d] -= h
                args_p = {"q": q, "k": k, "v": v}; args_p[which] = xp
                args_m = {"q": q, "k": k, "v": v}; args_m[which] = xm
                fd = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                      loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
                an = grad[b, hh, t - t0, d]
                assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, s, hh, t, d, fd, an)


def test_k_all_gradients_vs_dense():
    """k covering all history: dQ equals dense causal dQ (torch autograd on
    the whole sequence); with one segment (L = S) dK and dV equal dense too."""
    for shape, dkdv_dense in ((small_shape(top_k=16), False),
                              (small_shape(seq_len=32, seg_len=32, top_k=4), True)):
        inp = make_inputs(shape, seed=4)
        out = orc.run(inp)
        G = shape.group
        q = torch.tensor(inp["q"], dtype=torch.float64, requires_grad=True)
        k = torch.tensor(inp["k"], dtype=torch.float64, requires_grad=True)
        v = torch.tensor(inp["v"], dtype=torch.float64, requires_grad=True)
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), is_causal=True)
        (o * torch.tensor(inp["do"], dtype=torch.float64)).sum().backward()
        np.testing.assert_allclose(out["dq"], q.grad.numpy(), atol=1e-11, rtol=0)
        if dkdv_dense:
            np.testing.assert_allclose(out["dk"], k.grad.numpy(), atol=1e-11, rtol=0)
            np.testing.assert_allclose(out["dv"], v.grad.numpy(), atol=1e-11, rtol=0)
        else:
            assert np.abs(out["dk"] - k.grad.numpy()).max() > 1e-3  # truncation is real


# ------------------------------------------------------ two forms agree
@pytest.mark.parametrize("shape", [
    small_shape(),
    small_shape(n_q_heads=4, n_kv_heads=2, seq_len=48, seg_len=16, hist_block=4,
                query_block=8, top_k=3, head_dim=4),
    small_shape(batch=2, n_q_heads=3, n_kv_heads=3, seq_len=32, seg_len=16,
                hist_block=8, query_block=4, top_k=1, head_dim=4),
])
def test_loop_form_equals_vectorized_form(shape):
    inp = make_inputs(shape, seed=21)
    vec = orc.run(inp)
    lp = hga_loop.run_loop(inp["q"], inp["k"], inp["v"], inp["do"], shape)
    np.testing.assert_array_equal(vec["sel"], np.array(lp["sel"], dtype=np.int32))
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(vec[key], np.array(lp[key]), atol=1e-12, rtol=0, err_msg=key)


def test_gather_blocks_copies_chosen_slabs():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 64, 4)).astype(np.float32)
    sel = np.array([[[[3, 1, -1]] * 2] * 3] * 2, dtype=np.int32)
    g = orc.gather_blocks(x, sel, 8)
    assert g.shape == (2, 3, 2, 3, 8, 4)
    np.testing.assert_array_equal(g[1, 2, 0, 0], x[1, 2, 24:32])
    np.testing.assert_array_equal(g[0, 1, 1, 1], x[0, 1, 8:16])
    assert not g[:, :, :, 2].any()
