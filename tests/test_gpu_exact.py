"""GPU parity of the exact-gradient backward (hga_segment_step_exact,
history not detached) against the oracle's backward_exact: selection bit for
bit, O, LSE and the full-sequence dQ, dK, dV by max-abs-relative error at
2e-2 (bf16; the step is bf16 only)."""

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
    base = dict(name="x", batch=1, seq_len=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                seg_len=128, hist_block=32, query_block=32, top_k=3, dtype="bf16")
    base.update(kw)
    return HGAShape(**base)


def run_exact(shape, dev):
    """Summaries of every block, then the exact steps from the last segment
    to the first; returns the output tensors on the host."""
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    z = lambda shp_, dt: torch.zeros(shp_, dtype=dt, device="cuda")  # noqa: E731
    out = {"summ": z(s.summ, torch.float32), "sel": z(s.sel, torch.int32), "o": z(s.q, s.dt),
           "lse": z(s.lse, torch.float32), "dq": z(s.q, s.dt), "dk": z(s.kv, s.dt),
           "dv": z(s.kv, s.dt)}
    hdk, hdv = z(s.kv, torch.float32), z(s.kv, torch.float32)
    ws = torch.empty(max(hga.workspace_size(cfg, hga.HGA_OP_STEP_EXACT), 256), dtype=torch.uint8,
                     device="cuda")
    hga.summarize(cfg, dev["k"], 0, shape.seq_len // shape.hist_block, out["summ"])
    for seg in reversed(range(shape.nseg)):
        hga.segment_step_exact(cfg, seg, dev["q"], dev["k"], dev["v"], dev["do"], out["summ"],
                               out["sel"], out["o"], out["lse"], out["dq"], out["dk"],
                               out["dv"], hdk, hdv, ws)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


def run_exact_pass(shape, dev):
    """hga_segment_pass_exact; returns the output tensors on the host."""
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    z = lambda shp_, dt: torch.zeros(shp_, dtype=dt, device="cuda")  # noqa: E731
    out = {"summ": z(s.summ, torch.float32), "sel": z(s.sel, torch.int32), "o": z(s.q, s.dt),
           "lse": z(s.lse, torch.float32), "dq": z(s.q, s.dt), "dk": z(s.kv, s.dt),
           "dv": z(s.kv, s.dt)}
    hga.segment_pass_exact(cfg, dev["q"], dev["k"], dev["v"], dev["do"], out["summ"],
                           out["sel"], out["o"], out["lse"], out["dq"], out["dk"], out["dv"])
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


EXACT_SHAPES = [
    shp(),                                                      # G = 4, D = 128
    shp(top_k=40),                                              # k covers all history
    shp(hist_block=16, query_block=16, top_k=5),                # 16-row blocks (half tiles)
    shp(hist_block=64, query_block=64, top_k=2, n_q_heads=16),  # 2 key tiles per block, G = 8
    shp(head_dim=64, seq_len=384, seg_len=96, hist_block=48, query_block=48, top_k=2),
    shp(head_dim=64, seq_len=768, seg_len=256, hist_block=64, query_block=64, top_k=2),
    shp(batch=2, seq_len=256, n_q_heads=2, n_kv_heads=2, top_k=2),  # G = 1, batch 2
    shp(seq_len=128, seg_len=128),                              # one segment: no history
]


@pytest.mark.parametrize("shape", EXACT_SHAPES)
def test_exact_backward_parity(shape):
    inp = make_inputs(shape, seed=23)
    got = run_exact(shape, upload(inp, shape))
    ref = orc.run(inp, shape, bwd=False)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    dQ, dK, dV = orc.backward_exact(inp["q"], inp["k"], inp["v"], inp["do"], ref["sel"], shape,
                                    ref["o"], ref["lse"])
    tol = TOL[shape.dtype]
    errs = {}
    for key, want in (("o", ref["o"]), ("lse", ref["lse"]), ("dq", dQ), ("dk", dK), ("dv", dV)):
        errs[key] = assert_close(key, got[key], want, tol)
    print({k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_exact_backward_full_size_16k():
    """The 16K training workload in the exact form; dK/dV compared in full
    for one KV head (the oracle recomputes that group only)."""
    shape = WORKLOADS["train_16k"]
    print("[exact 16k] generating inputs", flush=True)
    inp = make_inputs(shape, seed=0)
    print("[exact 16k] GPU", flush=True)
    got = run_exact(shape, upload(inp, shape))
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    nqb = shape.n_qblocks
    sel = np.full(got["sel"].shape, -1, dtype=np.int32)
    for s in range(shape.nseg):
        sel[:, :, s * nqb:(s + 1) * nqb] = orc.select_segment(inp["q"], inp["k"], shape, s,
                                                              kbar=kbar if s else None)
    np.testing.assert_array_equal(got["sel"], sel)
    g, G = 3, shape.group
    print("[exact 16k] oracle forward + exact backward, one KV head", flush=True)
    O = np.zeros(inp["q"].shape)
    LSE = np.zeros(inp["q"].shape[:3])
    for s in range(shape.nseg):
        t0, L = s * shape.seg_len, shape.seg_len
        o_s, l_s = orc.segment_forward(inp["q"], inp["k"], inp["v"], sel[:, :, s * nqb:(s + 1) * nqb],
                                       shape, s, groups=[(0, g)])
        O[:, :, t0:t0 + L] = o_s
        LSE[:, :, t0:t0 + L] = l_s
    dQ, dK, dV = orc.backward_exact(inp["q"], inp["k"], inp["v"], inp["do"], sel, shape, O, LSE,
                                    groups=[(0, g)])
    hs = slice(g * G, (g + 1) * G)
    tol = TOL[shape.dtype]
    assert_close("o", got["o"][0, hs], O[0, hs], tol)
    assert_close("dq", got["dq"][0, hs], dQ[0, hs], tol)
    assert_close("dk", got["dk"][0, g], dK[0, g], tol)
    assert_close("dv", got["dv"][0, g], dV[0, g], tol)
    # the exact pass (whole-pass kernels) on the same inputs: the same
    # selections, the same gradient within the tolerance, for every head
    print("[exact 16k] exact pass", flush=True)
    dev = upload(inp, shape)
    pas = run_exact_pass(shape, dev)
    np.testing.assert_array_equal(pas["sel"], got["sel"])
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert_close(f"pass {key}", pas[key], got[key].astype(np.float64), tol)
    assert_close("pass dk (oracle head)", pas["dk"][0, g], dK[0, g], tol)


@pytest.mark.parametrize("shape", EXACT_SHAPES + [
    shp(seq_len=1024, seg_len=256, hist_block=64, query_block=64, top_k=3),  # 2 key blocks
    shp(seq_len=480, seg_len=160, hist_block=32, query_block=32, top_k=4),   # ragged key block
])
def test_exact_pass_parity(shape):
    """hga_segment_pass_exact against the oracle's backward_exact, and
    against the exact steps (selection bit for bit; outputs within the
    dtype's tolerance: the pass adds float sums in another order)."""
    inp = make_inputs(shape, seed=29)
    dev = upload(inp, shape)
    got = run_exact_pass(shape, dev)
    ref = orc.run(inp, shape, bwd=False)
    np.testing.assert_array_equal(got["sel"], ref["sel"])
    dQ, dK, dV = orc.backward_exact(inp["q"], inp["k"], inp["v"], inp["do"], ref["sel"], shape,
                                    ref["o"], ref["lse"])
    tol = TOL[shape.dtype]
    errs = {}
    for key, want in (("o", ref["o"]), ("lse", ref["lse"]), ("dq", dQ), ("dk", dK), ("dv", dV)):
        errs[key] = assert_close(key, got[key], want, tol)
    steps = run_exact(shape, dev)
    np.testing.assert_array_equal(got["sel"], steps["sel"])
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert_close(key, got[key], steps[key].astype(np.float64), tol)
    print({k: f"{v:.2e}" for k, v in errs.items()})
