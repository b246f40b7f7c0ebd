"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs.  Selection, gather and summaries-driven indices are
compared bit for bit; floating-point outputs by max-abs-relative error,
max|x - ref| / max|ref|, at 1e-5 (fp32) and 2e-2 (bf16)."""

import numpy as np
import pytest

from oracle import hga_oracle as orc
from synth import HGAShape, WORKLOADS, make_inputs

from gpu_util import TOL, assert_close, max_abs_rel, run_pass, to_np, upload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_long_context_query_amd as hga  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


def shp(**kw):
    base = dict(name="t", batch=1, seq_len=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                seg_len=128, hist_block=32, query_block=32, top_k=3, dtype="bf16")
    base.update(kw)
    return HGAShape(**base)


def compare_all(shape, inp, buf, segments=None, tol=None):
    tol = tol or TOL[shape.dtype]
    ref = orc.run(inp, shape, segments=segments, bwd=buf.dq is not None)
    np.testing.assert_array_equal(to_np(buf.sel), ref["sel"])
    errs = {}
    for key in ("o", "lse") + (("dq", "dk", "dv") if buf.dq is not None else ()):
        errs[key] = assert_close(key, to_np(getattr(buf, key)), ref[key], tol)
    nblk_hist = (shape.seq_len - shape.seg_len) // shape.hist_block
    if nblk_hist > 0:
        assert_close("summ", to_np(buf.summ)[:, :, :nblk_hist], ref["kbar"][:, :, :nblk_hist],
                     1e-6)
    return errs


# ------------------------------------------------------------ whole passes
@pytest.mark.parametrize("name", ["tiny_f32", "qwen3_2k"])
def test_workload_pass_full_parity(name):
    shape = WORKLOADS[name]
    inp = make_inputs(shape, seed=0)
    for s in range(shape.nseg):
        assert orc.selection_gap(inp["q"], inp["k"], shape, s) >= 1e-3
    buf = run_pass(shape, upload(inp, shape))
    errs = compare_all(shape, inp, buf)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("shape", [
    shp(),                                                     # several tiles, G=4
    shp(query_block=16, hist_block=16, top_k=5),               # half-filled 32-row waves
    shp(query_block=48, hist_block=48, seg_len=96, seq_len=480, top_k=2),  # ragged tiles
    shp(n_q_heads=2, n_kv_heads=2, top_k=2),                   # G = 1
    shp(n_q_heads=16, n_kv_heads=2, top_k=4),                  # G = 8
    shp(head_dim=64, query_block=64, hist_block=64, seg_len=128, top_k=2),  # D = 64
    shp(batch=2, seq_len=256, top_k=2),                        # batch 2
    shp(seq_len=128, seg_len=128),                             # one segment, no history
    shp(top_k=40),                                             # k covers all history
    shp(seq_len=128, seg_len=32, hist_block=16, query_block=16, top_k=2),  # one 32-key tile
    shp(seq_len=192, seg_len=48, hist_block=16, query_block=16, top_k=3),  # ragged key tile
    shp(seq_len=480, seg_len=160, top_k=4),                    # odd number of key tiles
    shp(seq_len=1024, seg_len=256, hist_block=16, query_block=64, top_k=24),  # many candidates
    shp(seq_len=1152, seg_len=384, hist_block=64, query_block=64, top_k=3),  # 3 key blocks
    shp(seq_len=960, seg_len=320, top_k=4),                    # 3 key blocks, last one ragged
    shp(head_dim=64, seq_len=1152, seg_len=384, hist_block=64, query_block=64, top_k=2),  # D=64
    shp(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2),
    shp(dtype="f32", head_dim=128, query_block=16, hist_block=8, top_k=5, seq_len=256),
])
def test_shape_variants_full_parity(shape):
    inp = make_inputs(shape, seed=5)
    buf = run_pass(shape, upload(inp, shape))
    compare_all(shape, inp, buf)


def test_k_all_equals_dense_causal():
    """With k covering every history block the HGA forward is dense causal
    attention (checked against torch SDPA in float64 on the CPU)."""
    shape = WORKLOADS["qwen3_2k"].replace(top_k=WORKLOADS["qwen3_2k"].seq_len // 64)
    inp = make_inputs(shape, seed=0)
    buf = run_pass(shape, upload(inp, shape))
    G = shape.group
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(inp["q"], dtype=torch.float64),
        torch.tensor(inp["k"], dtype=torch.float64).repeat_interleave(G, 1),
        torch.tensor(inp["v"], dtype=torch.float64).repeat_interleave(G, 1),
        is_causal=True).numpy()
    assert_close("o vs dense", to_np(buf.o), ref, TOL["bf16"])
    compare_all(shape, inp, buf)


def test_forward_only_without_lse():
    shape = shp(seq_len=256)
    inp = make_inputs(shape, seed=1, with_do=False)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg, bwd=False)
    for s in range(shape.nseg):
        if s > 0:
            hga.summarize(cfg, dev["k"], (s - 1) * shape.seg_len // shape.hist_block,
                          s * shape.seg_len // shape.hist_block, buf.summ)
        hga.select(cfg, dev["q"], buf.summ, s, buf.sel)
        hga.attn_fwd(cfg, dev["q"], dev["k"], dev["v"], buf.sel, s, buf.o, None)
    torch.cuda.synchronize()
    ref = orc.run(inp, shape, bwd=False)
    np.testing.assert_array_equal(to_np(buf.sel), ref["sel"])
    assert_close("o", to_np(buf.o), ref["o"], TOL["bf16"])


# ------------------------------------------------------ kernels one by one
def test_selection_crafted_ties_and_order():
    """Keys whose blocks repeat one of three integer patterns and integer
    queries: every score is exact in fp32 and many scores tie exactly, also
    at the k-th boundary, where the lower block index must win."""
    shape = shp(seq_len=1024, seg_len=128, hist_block=32, query_block=32, top_k=5,
                n_q_heads=4, n_kv_heads=2)
    rng = np.random.default_rng(3)
    q = rng.integers(-1, 2, size=(1, 4, 1024, 128)).astype(np.float32)
    pat = rng.integers(-1, 2, size=(3, 128))
    idx = rng.integers(0, 3, size=(2, 32))
    k = np.repeat(pat[idx][None, :, :, None, :], 32, axis=3).reshape(1, 2, 1024, 128)
    k = k.astype(np.float32)
    v = rng.standard_normal((1, 2, 1024, 128)).astype(np.float32)
    inp = {"q": q, "k": k, "v": v, "do": None, "shape": shape}
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg, bwd=False)
    hga.summarize(cfg, dev["k"], 0, 1024 // 32, buf.summ)
    for s in range(shape.nseg):
        hga.select(cfg, dev["q"], buf.summ, s, buf.sel)
    torch.cuda.synchronize()
    nqb = shape.n_qblocks
    boundary_ties = 0
    for s in range(shape.nseg):
        want = orc.select_segment(q, k, shape, s)
        got = to_np(buf.sel)[:, :, s * nqb:(s + 1) * nqb]
        np.testing.assert_array_equal(got, want)
        if s == 0:
            continue
        sc = orc.block_scores(orc.query_means(q, 2, s * 128, 128, 32),
                              orc.block_summaries(k, 32), s * 128 // 32)
        for row in sc.reshape(-1, sc.shape[-1]):
            if len(row) > shape.top_k:
                srt = np.sort(row)[::-1]
                boundary_ties += srt[shape.top_k - 1] == srt[shape.top_k]
    assert boundary_ties > 20  # the case really exercises ties at the boundary


@pytest.mark.parametrize("shape", [
    # > 1024 candidates: the LDS sort path
    shp(seq_len=20480, seg_len=2048, hist_block=16, query_block=64, top_k=8, n_q_heads=2,
        n_kv_heads=1, head_dim=64),
    # 64 < candidates <= 1024 with k spanning several lanes' registers
    shp(seq_len=8192, seg_len=1024, hist_block=16, query_block=128, top_k=100, n_q_heads=4,
        n_kv_heads=2),
])
def test_selection_many_candidates(shape):
    """Selection only (summaries + top-k) against the oracle, bit-exact."""
    inp = make_inputs(shape, seed=12, with_do=False)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg, bwd=False)
    nblk = shape.seq_len // shape.hist_block
    hga.summarize(cfg, dev["k"], 0, nblk, buf.summ)
    for s in range(shape.nseg):
        hga.select(cfg, dev["q"], buf.summ, s, buf.sel)
    torch.cuda.synchronize()
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    nqb = shape.n_qblocks
    for s in range(shape.nseg):
        assert orc.selection_gap(inp["q"], inp["k"], shape, s) >= 1e-3
        want = orc.select_segment(inp["q"], inp["k"], shape, s, kbar=kbar)
        np.testing.assert_array_equal(to_np(buf.sel)[:, :, s * nqb:(s + 1) * nqb], want,
                                      err_msg=f"segment {s}")


def test_summarize_matches_closed_form():
    """K[t, d] = t//64 + 0.25*(t%64) - (d%16)/8 (all bf16-exact): the mean of
    block i is i + 7.875 - (d%16)/8 exactly; rows outside the requested
    block range stay untouched."""
    shape = shp(seq_len=1024, hist_block=64, query_block=64, seg_len=256)
    t = np.arange(1024)[None, None, :, None]
    d = np.arange(128)[None, None, None, :]
    k = np.broadcast_to((t // 64) + 0.25 * (t % 64) - (d % 16) / 8.0, (1, 2, 1024, 128))
    k = k.astype(np.float32).copy()
    dev = upload({"k": k}, shape)
    cfg = hga.Config.from_shape(shape)
    summ = torch.full(hga.Shapes(cfg).summ, -7.0, device="cuda")
    hga.summarize(cfg, dev["k"], 3, 11, summ)
    torch.cuda.synchronize()
    got = to_np(summ)
    i = np.arange(16)[:, None]
    want = i + 7.875 - (np.arange(128)[None, :] % 16) / 8.0
    for g in range(2):
        np.testing.assert_array_equal(got[0, g, 3:11], want[3:11])
    assert np.all(got[0, :, :3] == -7.0) and np.all(got[0, :, 11:] == -7.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_bit_exact(dtype):
    shape = shp(dtype=dtype, top_k=4, seq_len=1024, seg_len=256, hist_block=32,
                query_block=64, head_dim=64 if dtype == "f32" else 128)
    inp = make_inputs(shape, seed=2, with_do=False)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    s_ = hga.Shapes(cfg)
    seg = 3
    sel = torch.full(s_.sel, -1, dtype=torch.int32, device="cuda")
    nqb = shape.n_qblocks
    rows = np.array([[5, 0, 17, -1], [23, 3, -1, -1], [1, 2, 3, 4], [-1, -1, -1, -1]],
                    dtype=np.int32)
    sel_np = np.full(s_.sel, -1, dtype=np.int32)
    sel_np[:, :, seg * nqb:(seg + 1) * nqb] = rows[None, None]
    sel_np[0, 1, seg * nqb] = [7, 99, -5, 2]  # out-of-range entries read as padding
    sel.copy_(torch.from_numpy(sel_np))
    ko = torch.empty(s_.gather, dtype=dev["k"].dtype, device="cuda")
    vo = torch.empty_like(ko)
    hga.gather(cfg, dev["k"], dev["v"], sel, seg, ko, vo)
    torch.cuda.synchronize()
    cleaned = sel_np[:, :, seg * nqb:(seg + 1) * nqb].copy()
    cleaned[(cleaned < 0) | (cleaned >= seg * 256 // 32)] = -1
    np.testing.assert_array_equal(to_np(ko), orc.gather_blocks(inp["k"], cleaned, 32))
    np.testing.assert_array_equal(to_np(vo), orc.gather_blocks(inp["v"], cleaned, 32))


def test_attention_with_arbitrary_selection():
    """Forward/backward with a selection that is not top-k (unsorted,
    repeated-free, padded): the kernels attend exactly the listed blocks."""
    shape = shp(seq_len=512, seg_len=128, top_k=4)
    inp = make_inputs(shape, seed=8)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg)
    seg = 3
    rng = np.random.default_rng(0)
    nqb = shape.n_qblocks
    sel_np = np.full(hga.Shapes(cfg).sel, -1, dtype=np.int32)
    for g in range(2):
        for j in range(nqb):
            n = rng.integers(0, 5)
            sel_np[0, g, seg * nqb + j, :n] = rng.choice(12, size=n, replace=False)
    buf.sel.copy_(torch.from_numpy(sel_np))
    hga.attn_fwd(cfg, dev["q"], dev["k"], dev["v"], buf.sel, seg, buf.o, buf.lse)
    hga.attn_bwd(cfg, dev["q"], dev["k"], dev["v"], buf.o, buf.lse, dev["do"], buf.sel, seg,
                 buf.dq, buf.dk, buf.dv, buf.ws)
    torch.cuda.synchronize()
    sel_seg = sel_np[:, :, seg * nqb:(seg + 1) * nqb]
    O, LSE = orc.segment_forward(inp["q"], inp["k"], inp["v"], sel_seg, shape, seg)
    dQ, dK, dV = orc.segment_backward(inp["q"], inp["k"], inp["v"], inp["do"], sel_seg, shape,
                                      seg, O, LSE)
    t0, L = seg * 128, 128
    assert_close("o", to_np(buf.o)[:, :, t0:t0 + L], O, TOL["bf16"])
    assert_close("lse", to_np(buf.lse)[:, :, t0:t0 + L], LSE, TOL["bf16"])
    assert_close("dq", to_np(buf.dq)[:, :, t0:t0 + L], dQ, TOL["bf16"])
    assert_close("dk", to_np(buf.dk)[:, :, t0:t0 + L], dK, TOL["bf16"])
    assert_close("dv", to_np(buf.dv)[:, :, t0:t0 + L], dV, TOL["bf16"])
    # rows outside the segment untouched
    assert not to_np(buf.o)[:, :, :t0].any() and not to_np(buf.dk)[:, :, :t0].any()


# ------------------------------------------------------- determinism, resume
def test_bitwise_deterministic():
    shape = WORKLOADS["qwen3_2k"]
    inp = make_inputs(shape, seed=0)
    dev = upload(inp, shape)
    a = run_pass(shape, dev)
    b = run_pass(shape, dev)
    for key in ("summ", "sel", "o", "lse", "dq", "dk", "dv"):
        assert torch.equal(getattr(a, key), getattr(b, key)), key


def test_resume_from_segment_state():
    """The resumable state of a segmented pass is the summary table (plus
    the inputs): restarting at segment s with a copy of it gives the same
    outputs as the uninterrupted pass."""
    shape = WORKLOADS["qwen3_2k"]
    inp = make_inputs(shape, seed=0)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    full = hga.Buffers(cfg)
    full.run_pass(dev["q"], dev["k"], dev["v"], dev["do"], per_step=True)
    first = hga.Buffers(cfg)
    first.run_pass(dev["q"], dev["k"], dev["v"], dev["do"], segments=range(0, 2))
    second = hga.Buffers(cfg)
    second.summ.copy_(first.summ)
    second.run_pass(dev["q"], dev["k"], dev["v"], dev["do"], segments=range(2, shape.nseg))
    torch.cuda.synchronize()
    t = 2 * shape.seg_len
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(getattr(second, key)[:, :, t:], getattr(full, key)[:, :, t:]), key


# ------------------------------------------------------- pass vs steps
@pytest.mark.parametrize("shape", [shp(), shp(dtype="f32", head_dim=64, n_q_heads=4,
                                                n_kv_heads=2), shp(seq_len=128, seg_len=128)])
@pytest.mark.parametrize("bwd", [True, False])
def test_pass_streams_and_steps(shape, bwd):
    """hga_segment_pass gives the same results bit for bit on two streams
    and on one; hga_segment_step called for each segment in order gives the
    same selections and, within the dtype's tolerance, the same outputs
    (the bf16 pass runs its forward as one launch over all segments, whose
    blocks walk all keys of a unit themselves, so its float sums are added
    in another order); both match the oracle."""
    inp = make_inputs(shape, seed=31, with_do=bwd)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    a, b, c = (hga.Buffers(cfg, bwd=bwd) for _ in range(3))
    a.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd, two_streams=True)
    b.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd, per_step=True)
    c.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd, two_streams=False)
    torch.cuda.synchronize()
    keys = ("sel", "o", "lse") + (("dq", "dk", "dv") if bwd else ())
    for key in keys:
        assert torch.equal(getattr(a, key), getattr(c, key)), key
    assert torch.equal(a.sel, b.sel)
    tol = TOL[shape.dtype]
    for key in keys[1:]:
        assert_close(key, to_np(getattr(a, key)), to_np(getattr(b, key)).astype(np.float64), tol)
    compare_all(shape, inp, a)
    compare_all(shape, inp, b)

# ------------------------------------------------------- limits of the sizes
def exact_score_inputs(shape, seed, nvalues):
    """Inputs whose selection scores are exact small integers: every key of
    block x is v_x * e_0 (so its summary is exactly v_x e_0), every query is
    e_0 (so every query-block mean is exactly e_0), hence score_x = v_x with
    no rounding on either side.  v_x in [0, nvalues) with many blocks per
    value, so the k-th boundary falls inside a group of ties and the
    lower-index rule decides."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, S, D = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_len, shape.head_dim
    nblk = S // shape.hist_block
    vals = rng.integers(0, nvalues, size=(B, Hkv, nblk)).astype(np.float32)
    k = np.zeros((B, Hkv, S, D), np.float32)
    k[..., 0] = np.repeat(vals, shape.hist_block, axis=2)
    q = np.zeros((B, Hq, S, D), np.float32)
    q[..., 0] = 1.0
    return {"q": q, "k": k, "v": np.zeros_like(k)}


@pytest.mark.parametrize("dtype,nvalues", [("bf16", 200), ("f32", 2000)])
def test_selection_at_the_size_limits(dtype, nvalues):
    """The largest selection the library takes: 8,192 history blocks in the
    sequence (8,128 candidates for the last segment, the LDS-sort path) and
    top-k 1,024, with exact integer scores and ties at the k-th boundary;
    bit-exact against the oracle for the last and a middle segment."""
    shape = shp(seq_len=131072, seg_len=1024, hist_block=16, query_block=256, top_k=1024,
                n_q_heads=2, n_kv_heads=1, head_dim=64, dtype=dtype)
    assert shape.seq_len // shape.hist_block == 8192
    inp = exact_score_inputs(shape, 3, nvalues)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg, bwd=False)
    nblk = shape.seq_len // shape.hist_block
    hga.summarize(cfg, dev["k"], 0, nblk, buf.summ)
    nqb = shape.n_qblocks
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    for s in (shape.nseg - 1, shape.nseg // 2):
        hga.select(cfg, dev["q"], buf.summ, s, buf.sel)
        torch.cuda.synchronize()
        want = orc.select_segment(inp["q"], inp["k"], shape, s, kbar=kbar)
        got = to_np(buf.sel)[:, :, s * nqb:(s + 1) * nqb]
        np.testing.assert_array_equal(got, want, err_msg=f"segment {s}")
        # the k-th score is shared by blocks on both sides of the cut
        nb = s * shape.seg_len // shape.hist_block
        sc = kbar[0, 0, :nb, 0]
        kth = np.sort(sc)[::-1][shape.top_k - 1]
        assert (sc == kth).sum() > (sc[want[0, 0, 0]] == kth).sum()


def test_attention_with_top_k_1024():
    """Forward and backward of one segment whose query blocks each attend to
    1,024 history blocks (the top-k limit; 16,384 history keys) plus their
    local keys, against the oracle."""
    shape = shp(seq_len=24576, seg_len=2048, hist_block=16, query_block=128, top_k=1024,
                n_q_heads=2, n_kv_heads=1, head_dim=64, dtype="bf16")
    inp = make_inputs(shape, seed=21)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg)
    s = shape.nseg - 1
    t0, L = s * shape.seg_len, shape.seg_len
    hga.summarize(cfg, dev["k"], 0, t0 // shape.hist_block, buf.summ)
    hga.select(cfg, dev["q"], buf.summ, s, buf.sel)
    hga.attn_fwd(cfg, dev["q"], dev["k"], dev["v"], buf.sel, s, buf.o, buf.lse)
    hga.attn_bwd(cfg, dev["q"], dev["k"], dev["v"], buf.o, buf.lse, dev["do"], buf.sel, s,
                 buf.dq, buf.dk, buf.dv, buf.ws)
    torch.cuda.synchronize()
    nqb = shape.n_qblocks
    sel = to_np(buf.sel)[:, :, s * nqb:(s + 1) * nqb]
    assert (sel >= 0).sum(axis=-1).min() == 1024
    # 1,408 candidates: the register radix-select path; the planted inputs
    # keep the k-th boundary clear, so the chosen set is checked bit for bit
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    assert orc.selection_gap(inp["q"], inp["k"], shape, s, kbar=kbar) >= 1e-3
    np.testing.assert_array_equal(sel, orc.select_segment(inp["q"], inp["k"], shape, s,
                                                          kbar=kbar))
    O, LSE = orc.segment_forward(inp["q"], inp["k"], inp["v"], sel, shape, s)
    dQ, dK, dV = orc.segment_backward(inp["q"], inp["k"], inp["v"], inp["do"], sel, shape, s,
                                      O, LSE)
    tol = TOL["bf16"]
    assert_close("o", to_np(buf.o)[:, :, t0:t0 + L], O, tol)
    assert_close("lse", to_np(buf.lse)[:, :, t0:t0 + L], LSE, tol)
    assert_close("dq", to_np(buf.dq)[:, :, t0:t0 + L], dQ, tol)
    assert_close("dk", to_np(buf.dk)[:, :, t0:t0 + L], dK, tol)
    assert_close("dv", to_np(buf.dv)[:, :, t0:t0 + L], dV, tol)


@pytest.mark.parametrize("shape,scale", [
    (shp(), 0.05),                                                   # bf16 whole-pass kernels
    (shp(head_dim=64, query_block=64, hist_block=64, seg_len=128, top_k=2), 0.3),
    (shp(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2), 0.3),  # f32 kernels
])
@pytest.mark.parametrize("per_step", [False, True])
def test_softmax_scale_non_default(shape, scale, per_step):
    """A softmax scale other than 1/sqrt(D), through hga_segment_pass (bf16:
    the whole-pass kernels) and hga_segment_step (the one-segment kernels),
    against the oracle at the same scale.  The selection score is unscaled,
    so the chosen blocks are those of the default scale; the outputs are
    not, which shows that the scale reached the kernels."""
    inp = make_inputs(shape, seed=7)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape, softmax_scale=scale)
    buf = hga.Buffers(cfg)
    buf.run_pass(dev["q"], dev["k"], dev["v"], dev["do"], per_step=per_step)
    torch.cuda.synchronize()
    ref = orc.run(inp, shape, scale=scale)
    np.testing.assert_array_equal(to_np(buf.sel), ref["sel"])
    tol = TOL[shape.dtype]
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert_close(key, to_np(getattr(buf, key)), ref[key], tol)
    default = orc.run(inp, shape)
    np.testing.assert_array_equal(default["sel"], ref["sel"])
    assert max_abs_rel(to_np(buf.o), default["o"]) > 10 * tol
