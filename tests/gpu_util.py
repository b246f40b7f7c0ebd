"""Helpers for the GPU parity tests: upload generator inputs, run the HIP
path through the C ABI, and compare against the fp64 oracle."""

from __future__ import annotations

import numpy as np

import sparse_long_context_query_amd as hga

TOL = {"f32": 1e-5, "bf16": 2e-2}


def torch_dtype(shape):
    import torch
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def upload(inp, shape, device="cuda"):
    """Generator arrays (float32 holding dtype-exact values) -> device tensors."""
    import torch
    dt = torch_dtype(shape)
    out = {}
    for key in ("q", "k", "v", "do"):
        if inp.get(key) is not None:
            out[key] = torch.from_numpy(inp[key]).to(device).to(dt).contiguous()
    return out


def run_pass(shape, dev, bwd=None, cfg=None):
    """Whole segmented pass through hga_segment_step; returns Buffers."""
    import torch
    if bwd is None:
        bwd = shape.bwd and "do" in dev
    cfg = cfg or hga.Config.from_shape(shape)
    buf = hga.Buffers(cfg, bwd=bwd)
    buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd)
    torch.cuda.synchronize()
    return buf


def to_np(t):
    import torch
    return t.detach().float().cpu().numpy() if t.dtype != torch.int32 else t.cpu().numpy()


def max_abs_rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / den)


def assert_close(name, x, ref, tol):
    err = max_abs_rel(x, ref)
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: max-abs-relative error {err:.3e} > {tol:.1e}"
    return err
