"""Pins of the oracle's decode step against things other than itself.

The decode step has no worked example on the pages; it is pinned by
(1) dense causal attention (torch CPU float64 SDPA) when k covers the whole
history, (2) a brute-force selection written with explicit loops plus torch
SDPA under the boolean mask that selection implies, (3) the closed form of
the very first token, and (4) the segment forward of the same oracle, which
has pins of its own, on a query block that the decode step reproduces.
"""

import math

import numpy as np
import pytest
import torch

from oracle import hga_oracle as orc
from synth import HGAShape, make_inputs


def shp(**kw):
    base = dict(name="d", batch=1, seq_len=96, n_q_heads=4, n_kv_heads=2,
                head_dim=8, seg_len=32, hist_block=8, query_block=8, top_k=2,
                dtype="f32")
    base.update(kw)
    return HGAShape(**base)


def _sdpa(q, k, v, mask):
    """torch CPU float64 SDPA, GQA expanded by repeat_interleave."""
    G = q.shape[1] // k.shape[1]
    kt = torch.as_tensor(k, dtype=torch.float64).repeat_interleave(G, dim=1)
    vt = torch.as_tensor(v, dtype=torch.float64).repeat_interleave(G, dim=1)
    qt = torch.as_tensor(q, dtype=torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.as_tensor(np.array(mask, dtype=bool))).numpy()


def _brute_selection(q_new, k, shape, pos):
    """Selection written out with loops: block means, group-and-token mean
    query, unscaled dot products, rank = number of (score, index) pairs
    that beat a block; keep rank < k, ascending, -1 padded."""
    B, Hq, n, D = q_new.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    Bh, kk = shape.hist_block, shape.top_k
    nb = (pos // shape.seg_len) * shape.seg_len // Bh
    sel = np.full((B, Hkv, kk), -1, dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            qbar = [0.0] * D
            for hh in range(G):
                for t in range(n):
                    for d in range(D):
                        qbar[d] += float(q_new[b, g * G + hh, t, d]) / (G * n)
            sc = []
            for i in range(nb):
                s = 0.0
                for d in range(D):
                    kb = sum(float(k[b, g, i * Bh + r, d]) for r in range(Bh)) / Bh
                    s += qbar[d] * kb
                sc.append(s)
            keep = [i for i in range(nb)
                    if sum(1 for j in range(nb) if (sc[j], -j) > (sc[i], -i)) < kk]
            sel[b, g, :len(keep)] = sorted(keep)
    return sel


def _mask(sel, shape, pos, n, Hq):
    B, Hkv, _ = sel.shape
    G = Hq // Hkv
    t0 = (pos // shape.seg_len) * shape.seg_len
    m = np.zeros((B, Hq, n, pos + n), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for blk in sel[b, h // G]:
                if blk >= 0:
                    m[b, h, :, blk * shape.hist_block:(blk + 1) * shape.hist_block] = True
            for i in range(n):
                m[b, h, i, t0:pos + i + 1] = True
    return m


CASES = [(0, 1), (5, 3), (32, 1), (40, 8), (63, 1), (64, 16), (80, 16), (95, 1)]


@pytest.mark.parametrize("pos,n", CASES)
def test_decode_equals_dense_causal_when_k_covers_history(pos, n):
    shape = shp(top_k=12)  # 12 >= the 8 blocks before the last segment
    inp = make_inputs(shape, seed=21, with_do=False)
    q_new = inp["q"][:, :, pos:pos + n]
    sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos)
    causal = np.arange(pos + n)[None, :] <= (pos + np.arange(n))[:, None]
    ref = _sdpa(q_new, inp["k"][:, :, :pos + n], inp["v"][:, :, :pos + n],
                np.broadcast_to(causal, (1, shape.n_q_heads, n, pos + n)))
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("pos,n", CASES)
@pytest.mark.parametrize("top_k", [1, 3])
def test_decode_matches_bruteforce_selection_and_masked_sdpa(pos, n, top_k):
    shape = shp(top_k=top_k)
    inp = make_inputs(shape, seed=5, with_do=False)
    # fresh unplanted queries so that the selection is not the generator's
    rng = np.random.default_rng(pos * 31 + n)
    q_new = rng.standard_normal((1, shape.n_q_heads, n, shape.head_dim))
    sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos)
    want = _brute_selection(q_new, inp["k"], shape, pos)
    np.testing.assert_array_equal(sel, want)
    m = _mask(sel, shape, pos, n, shape.n_q_heads)
    ref = _sdpa(q_new, inp["k"][:, :, :pos + n], inp["v"][:, :, :pos + n], m)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # LSE: log of the softmax denominator over the same visible keys
    G = shape.group
    for h in range(shape.n_q_heads):
        z = (q_new[0, h] @ inp["k"][0, h // G, :pos + n].T) / math.sqrt(shape.head_dim)
        z = np.where(m[0, h], z, -np.inf)
        np.testing.assert_allclose(LSE[0, h], np.log(np.exp(z).sum(axis=1)), rtol=0,
                                   atol=1e-12)


def test_decode_first_token_closed_form():
    """pos = 0: no history, the only key is the token itself, so o = v[0]
    and lse = scale * q . k[0]."""
    shape = shp()
    inp = make_inputs(shape, seed=2, with_do=False)
    q_new = inp["q"][:, :, :1]
    sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, 0)
    assert (sel == -1).all()
    G = shape.group
    for h in range(shape.n_q_heads):
        np.testing.assert_allclose(O[0, h, 0], inp["v"][0, h // G, 0], rtol=0, atol=1e-15)
        want = float(np.dot(q_new[0, h, 0].astype(np.float64),
                            inp["k"][0, h // G, 0].astype(np.float64))) / math.sqrt(8)
        assert abs(LSE[0, h, 0] - want) < 1e-14


@pytest.mark.parametrize("seg,j", [(1, 0), (2, 3), (2, 1)])
def test_decode_of_a_whole_query_block_equals_the_segment_forward(seg, j):
    shape = shp(top_k=3)
    inp = make_inputs(shape, seed=9, with_do=False)
    t0, Bq = seg * shape.seg_len, shape.query_block
    pos = t0 + j * Bq
    sel_s = orc.select_segment(inp["q"], inp["k"], shape, seg)
    O_s, L_s = orc.segment_forward(inp["q"], inp["k"], inp["v"], sel_s, shape, seg)
    sel, O, LSE = orc.decode_step(inp["q"][:, :, pos:pos + Bq], inp["k"], inp["v"], shape, pos)
    np.testing.assert_array_equal(sel, sel_s[:, :, j])
    np.testing.assert_allclose(O, O_s[:, :, j * Bq:(j + 1) * Bq], rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE, L_s[:, :, j * Bq:(j + 1) * Bq], rtol=0, atol=1e-13)


def test_decode_rejects_tokens_across_a_segment_boundary():
    shape = shp()
    inp = make_inputs(shape, seed=1, with_do=False)
    with pytest.raises(ValueError):
        orc.decode_step(inp["q"][:, :, 30:34], inp["k"], inp["v"], shape, 30)
