"""GPU parity of the decode step (hga_decode_step through the C ABI)
against the fp64 oracle's decode_step: selection bit for bit (cases whose
fp64 score gap at the k-th boundary is at least 1e-3), O and LSE by
max-abs-relative error at 1e-5 (fp32) and 2e-2 (bf16)."""

import numpy as np
import pytest

from oracle import hga_oracle as orc
from synth import HGAShape, WORKLOADS, make_inputs

from gpu_util import TOL, assert_close, to_np, upload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_long_context_query_amd as hga  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


def shp(**kw):
    base = dict(name="d", batch=1, seq_len=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                seg_len=128, hist_block=32, query_block=32, top_k=3, dtype="bf16")
    base.update(kw)
    return HGAShape(**base)


def decode_gap(q_new, kbar, shape, pos):
    """Smallest fp64 score gap at the k-th boundary of the step's selection
    (inf when every history block is taken)."""
    B, Hq, n, D = q_new.shape
    Hkv = shape.n_kv_heads
    nb = (pos // shape.seg_len) * shape.seg_len // shape.hist_block
    if nb <= shape.top_k:
        return np.inf
    qbar = np.asarray(q_new, np.float64).reshape(B, Hkv, Hq // Hkv, n, D).mean(axis=(2, 3))
    sc = np.einsum("bgd,bgid->bgi", qbar, np.asarray(kbar[:, :, :nb], np.float64))
    srt = -np.sort(-sc, axis=-1)
    return float(np.min(srt[..., shape.top_k - 1] - srt[..., shape.top_k]))


def run_decode(shape, dev, pos, n, kbar_all=None):
    """Summaries of the blocks before the step's segment (the step itself
    adds the previous segment's when pos is the segment's first token),
    then one hga_decode_step; returns (sel, o, lse) on the host."""
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    B, Hq, D = shape.batch, shape.n_q_heads, shape.head_dim
    L, Bh = shape.seg_len, shape.hist_block
    t0 = pos // L * L
    summ = torch.zeros(s.summ, dtype=torch.float32, device="cuda")
    pre = (t0 - L) // Bh if (pos == t0 and t0 > 0) else t0 // Bh
    if pre > 0:
        hga.summarize(cfg, dev["k"], 0, pre, summ)
    q_new = dev["q"][:, :, pos:pos + n].contiguous()
    sel = torch.full((B, shape.n_kv_heads, shape.top_k), -7, dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, n, D), float("nan"), dtype=s.dt, device="cuda")
    lse = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device="cuda")
    hga.decode_step(cfg, pos, q_new, dev["k"], dev["v"], summ, sel, o, lse)
    torch.cuda.synchronize()
    return to_np(sel), to_np(o), to_np(lse), to_np(summ)


CASES = [(0, 1), (1, 4), (128, 1), (200, 2), (255, 1), (256, 2), (300, 1), (511, 1), (384, 2)]


@pytest.mark.parametrize("shape,cases", [
    (shp(), CASES),                                                   # G = 4, D = 128
    (shp(hist_block=16, query_block=16, top_k=5), CASES),             # chunks span 4 blocks
    (shp(top_k=40), CASES),                                           # k covers all history
    (shp(n_q_heads=16, n_kv_heads=2, top_k=4), [(130, 8), (500, 8), (3, 8)]),  # G*n = 64
    (shp(n_q_heads=2, n_kv_heads=2), [(129, 1), (510, 2), (260, 64)]),  # G = 1, n = 64
    (shp(head_dim=64, hist_block=64, query_block=64, top_k=2), CASES),  # D = 64
    (shp(head_dim=64, hist_block=32, query_block=32, top_k=3), [(300, 16), (130, 12)]),  # D = 64, G*n > 32
    (shp(batch=2, seq_len=256), [(0, 1), (128, 3), (255, 1)]),        # batch 2
    (shp(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2), CASES),
    (shp(dtype="f32", hist_block=8, query_block=8, top_k=6, seq_len=256), [(64, 1), (200, 5)]),
])
def test_decode_parity(shape, cases):
    inp = make_inputs(shape, seed=13, with_do=False)
    dev = upload(inp, shape)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    tol = TOL[shape.dtype]
    for pos, n in cases:
        q_new = inp["q"][:, :, pos:pos + n]
        gap = decode_gap(q_new, kbar, shape, pos)
        assert gap >= 1e-3, f"pos {pos} n {n}: selection gap {gap:.2e}"
        sel, o, lse, summ = run_decode(shape, dev, pos, n)
        want_sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos, kbar=kbar)
        np.testing.assert_array_equal(sel, want_sel, err_msg=f"pos {pos} n {n}")
        assert_close(f"o pos {pos} n {n}", o, O, tol)
        assert_close(f"lse pos {pos} n {n}", lse, LSE, tol)
        t0 = pos // shape.seg_len * shape.seg_len
        nb = t0 // shape.hist_block
        if nb > 0:
            assert_close("summ", summ[:, :, :nb], kbar[:, :, :nb], 1e-6)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decode_full_size_131k():
    """Three steps at the 131,072-token inference shape: the first 8 tokens
    of the last segment (the step summarizes the previous segment), a
    16-token block inside it (G*n = 64) and the very last token.  (With a
    single new token the query mean is noisy; the generator's gap guarantee
    holds for whole query blocks only, so the cases are ones whose fp64 gap
    is at least 1e-3, which the test asserts.)"""
    shape = WORKLOADS["infer_131k"]
    print("[decode 131k] generating inputs", flush=True)
    inp = make_inputs(shape, seed=0, with_do=False)
    dev = upload(inp, shape)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    S, L = shape.seq_len, shape.seg_len
    for pos, n in [(S - L, 8), (S - L + 100, 16), (S - 1, 1)]:
        print(f"[decode 131k] pos {pos} n {n}", flush=True)
        q_new = inp["q"][:, :, pos:pos + n]
        assert decode_gap(q_new, kbar, shape, pos) >= 1e-3
        sel, o, lse, _ = run_decode(shape, dev, pos, n)
        want_sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos, kbar=kbar)
        np.testing.assert_array_equal(sel, want_sel)
        assert_close("o", o, O, TOL[shape.dtype])
        assert_close("lse", lse, LSE, TOL[shape.dtype])


def tied_score_inputs(shape, seed, nvalues):
    """Keys of history block x all equal to v_x e_0 and queries equal to e_0:
    the block summary is v_x e_0 and the step's query mean e_0 exactly, so
    every selection score is the small integer v_x on both sides, and with
    far more blocks than values the k-th boundary falls inside a run of
    equal scores that spans several 256-block groups.  V is random."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, S, D = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim
    vals = rng.integers(0, nvalues, size=(B, Hkv, S // shape.hist_block)).astype(np.float32)
    k = np.zeros((B, Hkv, S, D), np.float32)
    k[..., 0] = np.repeat(vals, shape.hist_block, axis=2)
    q = np.zeros((B, Hq, S, D), np.float32)
    q[..., 0] = 1.0
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    return {"q": q, "k": k, "v": v}


# (top-k, first new token, new tokens): 1,016 candidates (four scoring
# blocks) with lists of 8 to 256, and 264 / 300 candidates, whose last
# scoring block holds fewer than k and keeps them all
# (top-k, first new token, new tokens): 1,016 history blocks with lists of 8
# to 256 entries per scoring block; 264 and 300 blocks; 96 blocks (one
# scoring block)
TWO_STAGE_CASES = [(8, 16256, 1), (30, 16300, 4), (60, 16383, 1), (100, 16256, 16),
                   (256, 16383, 1), (256, 4224, 2), (200, 4800, 1), (8, 1650, 1), (30, 1650, 3)]


@pytest.mark.parametrize("top_k,pos,n", TWO_STAGE_CASES)
def test_decode_two_stage_topk_ties(top_k, pos, n):
    """The two-stage top-k of the bf16 decode step (each scoring block keeps
    its own k best, the attention blocks pick the k best of those lists)
    against the oracle's single top-k over all candidates, with exact integer
    scores and ties at the k-th boundary: the selection bit for bit (the
    lower block index wins every tie), O and LSE within the tolerance."""
    shape = shp(seq_len=16384, seg_len=128, hist_block=16, query_block=16, top_k=top_k,
                n_q_heads=2, n_kv_heads=1, head_dim=64)
    inp = tied_score_inputs(shape, 5, 40)
    dev = upload(inp, shape)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    nb = pos // shape.seg_len * shape.seg_len // shape.hist_block
    sc = kbar[0, 0, :nb, 0]
    kth = np.sort(sc)[::-1][top_k - 1]
    assert (sc > kth).sum() < top_k < (sc >= kth).sum()  # a tie at the boundary
    q_new = inp["q"][:, :, pos:pos + n]
    sel, o, lse, _ = run_decode(shape, dev, pos, n)
    want_sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos, kbar=kbar)
    np.testing.assert_array_equal(sel, want_sel)
    assert_close("o", o, O, TOL["bf16"])
    assert_close("lse", lse, LSE, TOL["bf16"])


# (top-k, sequence length, first new token, new tokens) of the bf16 steps
# that do not take the two-stage top-k: k above 256 (the scores, then one
# top-k launch), and more than 1,024 candidates (the LDS sort of the
# selection kernel)
FALLBACK_CASES = [(300, 16384, 16383, 1), (300, 16384, 12000, 4), (8, 20480, 20479, 1),
                  (64, 20480, 20000, 16)]


@pytest.mark.parametrize("top_k,seq_len,pos,n", FALLBACK_CASES)
def test_decode_fallback_selection_ties(top_k, seq_len, pos, n):
    """The bf16 decode step's other selection paths against the oracle, with
    exact integer scores and ties at the k-th boundary: selection bit for
    bit, O and LSE within the tolerance."""
    shape = shp(seq_len=seq_len, seg_len=128, hist_block=16, query_block=16, top_k=top_k,
                n_q_heads=2, n_kv_heads=1, head_dim=64)
    inp = tied_score_inputs(shape, 7, 40)
    dev = upload(inp, shape)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    nb = pos // shape.seg_len * shape.seg_len // shape.hist_block
    assert nb > top_k and (top_k > 256 or nb > 1024)
    sc = kbar[0, 0, :nb, 0]
    kth = np.sort(sc)[::-1][top_k - 1]
    assert (sc > kth).sum() < top_k < (sc >= kth).sum()  # a tie at the boundary
    q_new = inp["q"][:, :, pos:pos + n]
    sel, o, lse, _ = run_decode(shape, dev, pos, n)
    want_sel, O, LSE = orc.decode_step(q_new, inp["k"], inp["v"], shape, pos, kbar=kbar)
    np.testing.assert_array_equal(sel, want_sel)
    assert_close("o", o, O, TOL["bf16"])
    assert_close("lse", lse, LSE, TOL["bf16"])
