"""GPU: hga_segment_pass_noalloc (scratch in the library's fixed per-GPU
array) against hga_segment_pass (scratch in a caller workspace), through the
C ABI.  Two calls in a row, the second with a smaller input (the array keeps
the first call's contents), bf16 and f32, forward + backward and forward
only.  Both entry points run the same kernels in the same order on one
stream, so every output is compared bit for bit."""

import pytest

from synth import HGAShape, make_inputs

from gpu_util import upload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_long_context_query_amd as hga  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


def shp(**kw):
    base = dict(name="t", batch=1, seq_len=2048, n_q_heads=32, n_kv_heads=8, head_dim=128,
                seg_len=512, hist_block=64, query_block=64, top_k=8, dtype="bf16")
    base.update(kw)
    return HGAShape(**base)


CALLS = {
    "bf16": [shp(),
             shp(seq_len=1024, n_q_heads=8, n_kv_heads=2, seg_len=256, top_k=4)],
    "f32": [shp(dtype="f32", seq_len=512, n_q_heads=4, n_kv_heads=2, head_dim=64, seg_len=128,
                hist_block=32, query_block=32, top_k=3),
            shp(dtype="f32", seq_len=256, n_q_heads=2, n_kv_heads=1, head_dim=64, seg_len=64,
                hist_block=16, query_block=16, top_k=2)],
}


def one_call(shape, seed, bwd):
    print(f"[noalloc] {shape.dtype} S={shape.seq_len} Hq={shape.n_q_heads} bwd={bwd}", flush=True)
    inp = make_inputs(shape, seed=seed, with_do=bwd)
    dev = upload(inp, shape)
    cfg = hga.Config.from_shape(shape)
    ref = hga.Buffers(cfg, bwd=bwd)
    ref.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd, two_streams=False)
    got = hga.Buffers(cfg, bwd=bwd)
    hga.segment_pass_noalloc(cfg, dev["q"], dev["k"], dev["v"], got.summ, got.sel, got.o,
                             got.lse, dev.get("do"), got.dq, got.dk, got.dv, bwd=bwd)
    torch.cuda.synchronize()
    keys = ("summ", "sel", "o", "lse") + (("dq", "dk", "dv") if bwd else ())
    for key in keys:
        a, b = getattr(got, key), getattr(ref, key)
        assert torch.equal(a, b), f"{key}: max diff {(a.float() - b.float()).abs().max().item()}"
    assert got.o.float().abs().max().item() > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_pass_equals_pass_two_calls(dtype):
    big, small = CALLS[dtype]
    one_call(big, 1, bwd=True)
    one_call(small, 2, bwd=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_pass_forward_only(dtype):
    big, small = CALLS[dtype]
    one_call(small, 3, bwd=False)
    one_call(big, 4, bwd=False)
