"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (hga_segment_pass: one launch per kernel over all segments).  Selection and
summaries are compared in full; O, LSE and gradients on sampled (segment,
sequence, KV head) groups that the fp64 oracle recomputes one by one."""

import numpy as np
import pytest

from oracle import hga_oracle as orc
from synth import WORKLOADS, make_inputs

from gpu_util import TOL, assert_close, run_pass, to_np, upload

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import sparse_long_context_query_amd as hga  # noqa: E402

# (segment, sequence, KV head) groups the oracle recomputes: a few early and
# middle ones, and every KV head of the last segment (its query blocks carry
# the most history)
SAMPLES = {
    "train_16k": [(1, 0, 0), (7, 0, 5)] + [(15, 0, g) for g in range(8)],
    "infer_131k": [(1, 0, 3), (64, 0, 0), (127, 0, 6)],
    "batch4_32k": [(1, 0, 0), (8, 1, 2)] + [(15, 3, g) for g in range(8)],
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["train_16k", "infer_131k", "batch4_32k"])
def test_full_size(name):
    shape = WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    inp = make_inputs(shape, seed=0)
    print(f"[{name}] GPU pass", flush=True)
    buf = run_pass(shape, upload(inp, shape))
    L, Bh, nqb = shape.seg_len, shape.hist_block, shape.n_qblocks

    print(f"[{name}] summaries + selection (all segments)", flush=True)
    kbar = orc.block_summaries(inp["k"], Bh)
    nh = (shape.seq_len - L) // Bh
    assert_close("summ", to_np(buf.summ)[:, :, :nh], kbar[:, :, :nh], 1e-6)
    sel_gpu = to_np(buf.sel)
    for s in range(shape.nseg):
        assert orc.selection_gap(inp["q"], inp["k"], shape, s, kbar=kbar) >= 1e-3
        want = orc.select_segment(inp["q"], inp["k"], shape, s, kbar=kbar)
        np.testing.assert_array_equal(sel_gpu[:, :, s * nqb:(s + 1) * nqb], want, err_msg=f"seg {s}")

    tol = TOL[shape.dtype]
    G = shape.group
    outs = {k: to_np(getattr(buf, k)) for k in ("o", "lse", "dq", "dk", "dv")
            if getattr(buf, k) is not None}
    for s, b, g in SAMPLES[name]:
        print(f"[{name}] oracle sample seg={s} b={b} g={g}", flush=True)
        t0 = s * L
        sel = sel_gpu[:, :, s * nqb:(s + 1) * nqb]
        O, LSE = orc.segment_forward(inp["q"], inp["k"], inp["v"], sel, shape, s, groups=[(b, g)])
        hs = slice(g * G, (g + 1) * G)
        assert_close(f"o s{s}", outs["o"][b, hs, t0:t0 + L], O[b, hs], tol)
        assert_close(f"lse s{s}", outs["lse"][b, hs, t0:t0 + L], LSE[b, hs], tol)
        if shape.bwd:
            dQ, dK, dV = orc.segment_backward(inp["q"], inp["k"], inp["v"], inp["do"], sel, shape,
                                              s, O, LSE, groups=[(b, g)])
            assert_close(f"dq s{s}", outs["dq"][b, hs, t0:t0 + L], dQ[b, hs], tol)
            assert_close(f"dk s{s}", outs["dk"][b, g, t0:t0 + L], dK[b, g], tol)
            assert_close(f"dv s{s}", outs["dv"][b, g, t0:t0 + L], dV[b, g], tol)
