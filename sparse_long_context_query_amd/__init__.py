"""Python binding of the HGA hot-path library (``libhga.so``, gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/hga.h``.  PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: if the
library is missing, every call raises.

Layouts (see the header): q, o, dO, dq [B,Hq,S,D]; k, v, dk, dv
[B,Hkv,S,D]; lse [B,Hq,S] float32; summ [B,Hkv,S/Bh,D] float32;
sel [B,Hkv,S/Bq,k] int32.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# HGA_LIB names another build of the same library (the host-sanitized one
# used by the CPU checks); the default is the package's own libhga.so
LIB_PATH = os.environ.get("HGA_LIB") or os.path.join(_PKG, "libhga.so")

HGA_OK = 0
HGA_ERR_ARG = -1
HGA_ERR_UNSUPPORTED = -2
HGA_ERR_WORKSPACE = -3
HGA_ERR_HIP = -4
HGA_F32 = 0
HGA_BF16 = 1
HGA_STEP_BWD = 1
(HGA_OP_FWD, HGA_OP_BWD, HGA_OP_STEP, HGA_OP_DECODE, HGA_OP_STEP_EXACT, HGA_OP_PASS,
 HGA_OP_PASS_EXACT, HGA_OP_STEP_HOST, HGA_OP_PASS_HOST) = range(9)
HGA_STEP_SUMMARIES_READY = 2
KERNEL_CLASSES = ("summarize", "select", "gather", "fwd", "bwd_pre", "bwd_dq", "bwd_dkdv",
                  "decode", "decode_merge", "bwd_hist", "tier_plan", "tier_fetch")


class HGAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"HGA error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    """Mirror of ``hga_config``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("seg_len", ctypes.c_int32),
        ("hist_block", ctypes.c_int32),
        ("query_block", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]

    @classmethod
    def from_shape(cls, shape, softmax_scale: float = 0.0) -> "Config":
        """From any object with the HGAShape attribute names."""
        return cls(shape.batch, shape.seq_len, shape.seg_len, shape.hist_block,
                   shape.query_block, shape.top_k, shape.n_q_heads, shape.n_kv_heads,
                   shape.head_dim, HGA_BF16 if shape.dtype == "bf16" else HGA_F32,
                   softmax_scale)


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_CP = ctypes.POINTER(Config)

_SIGNATURES = {
    "hga_summarize": (ctypes.c_int, [_CP, _P, ctypes.c_int32, ctypes.c_int32, _P, _P]),
    "hga_select": (ctypes.c_int, [_CP, _P, _P, ctypes.c_int32, _P, _P]),
    "hga_gather": (ctypes.c_int, [_CP, _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "hga_attn_fwd": (ctypes.c_int, [_CP, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "hga_attn_bwd": (ctypes.c_int, [_CP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                    _P, _P, ctypes.c_size_t, _P]),
    "hga_segment_step": (ctypes.c_int, [_CP, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "hga_segment_pass": (ctypes.c_int, [_CP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "hga_segment_pass_noalloc": (ctypes.c_int, [_CP, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                                _P, _P, _P, _P, _P, _P]),
    "hga_segment_step_host": (ctypes.c_int, [_CP, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "hga_segment_pass_host": (ctypes.c_int, [_CP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "hga_segment_step_exact": (ctypes.c_int, [_CP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                              _P]),
    "hga_segment_pass_exact": (ctypes.c_int, [_CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, ctypes.c_size_t, _P]),
    "hga_decode_step": (ctypes.c_int, [_CP, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P]),
    "hga_workspace_size": (ctypes.c_size_t, [_CP, ctypes.c_int32]),
    "hga_last_error": (ctypes.c_char_p, []),
    "hga_version": (ctypes.c_char_p, []),
    "hga_profile_begin": (ctypes.c_int, [ctypes.c_uint32]),
    "hga_profile_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m sparse_long_context_query_amd.build_lib)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().hga_last_error().decode()


def version() -> str:
    return lib().hga_version().decode()


def _check(rc: int) -> None:
    if rc != HGA_OK:
        raise HGAError(rc, last_error())


# ---------------------------------------------------------------- tensors
def _torch():
    import torch
    return torch


def _ptr(t, name, dtype=None, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _host_ptr(t, name, dtype, shape):
    """A pinned host tensor (the host tier's K / V)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor (pin_memory=True)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Shapes:
    """Expected tensor shapes and dtypes for a Config."""

    def __init__(self, cfg: Config):
        torch = _torch()
        B, S, D = cfg.batch, cfg.seq_len, cfg.head_dim
        self.dt = torch.bfloat16 if cfg.dtype == HGA_BF16 else torch.float32
        self.q = (B, cfg.n_q_heads, S, D)
        self.kv = (B, cfg.n_kv_heads, S, D)
        self.lse = (B, cfg.n_q_heads, S)
        self.summ = (B, cfg.n_kv_heads, S // cfg.hist_block, D)
        self.sel = (B, cfg.n_kv_heads, S // cfg.query_block, cfg.top_k)
        self.gather = (B, cfg.n_kv_heads, cfg.seg_len // cfg.query_block, cfg.top_k,
                       cfg.hist_block, D)


def workspace_size(cfg: Config, op: int = HGA_OP_STEP) -> int:
    return int(lib().hga_workspace_size(ctypes.byref(cfg), op))


def summarize(cfg: Config, k, blk_begin: int, blk_end: int, summ) -> None:
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_summarize(ctypes.byref(cfg), _ptr(k, "k", s.dt, s.kv), blk_begin,
                               blk_end, _ptr(summ, "summ", torch.float32, s.summ), _stream()))


def select(cfg: Config, q, summ, seg: int, sel) -> None:
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_select(ctypes.byref(cfg), _ptr(q, "q", s.dt, s.q),
                            _ptr(summ, "summ", torch.float32, s.summ), seg,
                            _ptr(sel, "sel", torch.int32, s.sel), _stream()))


def gather(cfg: Config, k, v, sel, seg: int, k_out, v_out) -> None:
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_gather(ctypes.byref(cfg), _ptr(k, "k", s.dt, s.kv), _ptr(v, "v", s.dt, s.kv),
                            _ptr(sel, "sel", torch.int32, s.sel), seg,
                            _ptr(k_out, "k_out", s.dt, s.gather),
                            _ptr(v_out, "v_out", s.dt, s.gather), _stream()))


def attn_fwd(cfg: Config, q, k, v, sel, seg: int, o, lse=None) -> None:
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_attn_fwd(ctypes.byref(cfg), _ptr(q, "q", s.dt, s.q),
                              _ptr(k, "k", s.dt, s.kv), _ptr(v, "v", s.dt, s.kv),
                              _ptr(sel, "sel", torch.int32, s.sel), seg,
                              _ptr(o, "o", s.dt, s.q),
                              _ptr(lse, "lse", torch.float32, s.lse, allow_none=True),
                              None, 0, _stream()))


def attn_bwd(cfg: Config, q, k, v, o, lse, do, sel, seg: int, dq, dk, dv, ws) -> None:
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_attn_bwd(ctypes.byref(cfg), _ptr(q, "q", s.dt, s.q),
                              _ptr(k, "k", s.dt, s.kv), _ptr(v, "v", s.dt, s.kv),
                              _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse),
                              _ptr(do, "do", s.dt, s.q), _ptr(sel, "sel", torch.int32, s.sel),
                              seg, _ptr(dq, "dq", s.dt, s.q), _ptr(dk, "dk", s.dt, s.kv),
                              _ptr(dv, "dv", s.dt, s.kv), _ptr(ws, "ws"),
                              ws.numel() * ws.element_size(), _stream()))


def segment_step(cfg: Config, seg: int, q, k, v, summ, sel, o, lse=None, do=None, dq=None,
                 dk=None, dv=None, ws=None, bwd: bool = True,
                 summaries_ready: bool = False) -> None:
    """hga_segment_step on the current stream; summaries_ready sets
    HGA_STEP_SUMMARIES_READY (summ already holds every block before the
    segment, so the step does not summarize)."""
    s = Shapes(cfg)
    torch = _torch()
    flags = (HGA_STEP_BWD if bwd else 0) | (HGA_STEP_SUMMARIES_READY if summaries_ready else 0)
    _check(lib().hga_segment_step(
        ctypes.byref(cfg), seg, flags, _ptr(q, "q", s.dt, s.q), _ptr(k, "k", s.dt, s.kv),
        _ptr(v, "v", s.dt, s.kv), _ptr(do, "do", s.dt, s.q, allow_none=not bwd),
        _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
        _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse, allow_none=not bwd),
        _ptr(dq, "dq", s.dt, s.q, allow_none=not bwd),
        _ptr(dk, "dk", s.dt, s.kv, allow_none=not bwd),
        _ptr(dv, "dv", s.dt, s.kv, allow_none=not bwd),
        _ptr(ws, "ws", allow_none=not bwd),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()))


def segment_step_exact(cfg: Config, seg: int, q, k, v, do, summ, sel, o, lse, dq, dk, dv,
                       hist_dk, hist_dv, ws) -> None:
    """Exact-gradient step (history not detached); see hga_segment_step_exact:
    summ must be complete, hist_dk / hist_dv float32 [B, Hkv, S, D] zeroed
    before the first call, segments visited in descending order."""
    s = Shapes(cfg)
    torch = _torch()
    _check(lib().hga_segment_step_exact(
        ctypes.byref(cfg), seg, _ptr(q, "q", s.dt, s.q), _ptr(k, "k", s.dt, s.kv),
        _ptr(v, "v", s.dt, s.kv), _ptr(do, "do", s.dt, s.q),
        _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
        _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse),
        _ptr(dq, "dq", s.dt, s.q), _ptr(dk, "dk", s.dt, s.kv), _ptr(dv, "dv", s.dt, s.kv),
        _ptr(hist_dk, "hist_dk", torch.float32, s.kv),
        _ptr(hist_dv, "hist_dv", torch.float32, s.kv),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def segment_pass_exact(cfg: Config, q, k, v, do, summ, sel, o, lse, dq, dk, dv, ws=None) -> None:
    """The whole exact-gradient pass (history not detached); see
    hga_segment_pass_exact.  ws defaults to a fresh buffer of
    workspace_size(cfg, HGA_OP_PASS_EXACT) bytes."""
    s = Shapes(cfg)
    torch = _torch()
    if ws is None:
        ws = torch.empty(max(workspace_size(cfg, HGA_OP_PASS_EXACT), 256), dtype=torch.uint8,
                         device=q.device)
    _check(lib().hga_segment_pass_exact(
        ctypes.byref(cfg), _ptr(q, "q", s.dt, s.q), _ptr(k, "k", s.dt, s.kv),
        _ptr(v, "v", s.dt, s.kv), _ptr(do, "do", s.dt, s.q),
        _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
        _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse),
        _ptr(dq, "dq", s.dt, s.q), _ptr(dk, "dk", s.dt, s.kv), _ptr(dv, "dv", s.dt, s.kv),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def decode_step(cfg: Config, pos: int, q_new, k, v, summ, sel, o, lse=None, ws=None) -> None:
    """n = q_new.shape[2] new tokens at positions pos .. pos+n-1 (one
    segment): q_new and o [B, Hq, n, D], sel [B, Hkv, k] int32, lse
    [B, Hq, n] float32 or None; k, v the full caches.  ws defaults to a fresh
    buffer of workspace_size(cfg, HGA_OP_DECODE) bytes."""
    s = Shapes(cfg)
    torch = _torch()
    if q_new.dim() != 4:
        raise ValueError("q_new must be [B, Hq, n, D]")
    n = int(q_new.shape[2])
    B, Hq, Hkv, D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    if ws is None:
        ws = torch.empty(max(workspace_size(cfg, HGA_OP_DECODE), 256), dtype=torch.uint8,
                         device=q_new.device)
    _check(lib().hga_decode_step(
        ctypes.byref(cfg), pos, n, _ptr(q_new, "q_new", s.dt, (B, Hq, n, D)),
        _ptr(k, "k", s.dt, s.kv), _ptr(v, "v", s.dt, s.kv),
        _ptr(summ, "summ", torch.float32, s.summ),
        _ptr(sel, "sel", torch.int32, (B, Hkv, cfg.top_k)),
        _ptr(o, "o", s.dt, (B, Hq, n, D)),
        _ptr(lse, "lse", torch.float32, (B, Hq, n), allow_none=True),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream()))


def profile_begin(classes=None) -> None:
    """Start bracketing launches of the given kernel classes (names from
    KERNEL_CLASSES; default all) with HIP events on their stream."""
    names = KERNEL_CLASSES if classes is None else classes
    mask = 0
    for n in names:
        mask |= 1 << KERNEL_CLASSES.index(n)
    _check(lib().hga_profile_begin(mask))


def profile_end() -> dict:
    """{kernel class: (total ms, launches)} since profile_begin()."""
    ms = (ctypes.c_double * len(KERNEL_CLASSES))()
    cnt = (ctypes.c_int64 * len(KERNEL_CLASSES))()
    _check(lib().hga_profile_end(ms, cnt))
    return {name: (ms[i], int(cnt[i])) for i, name in enumerate(KERNEL_CLASSES)}


def segment_pass(cfg: Config, q, k, v, summ, sel, o, lse=None, do=None, dq=None, dk=None,
                 dv=None, ws=None, bwd: bool = True, stream2=None) -> None:
    """hga_segment_pass on the current stream (and stream2, a torch stream at
    default priority, when given); ws of workspace_size(cfg, HGA_OP_PASS) bytes."""
    s = Shapes(cfg)
    torch = _torch()
    flags = HGA_STEP_BWD if bwd else 0
    _check(lib().hga_segment_pass(
        ctypes.byref(cfg), flags, _ptr(q, "q", s.dt, s.q), _ptr(k, "k", s.dt, s.kv),
        _ptr(v, "v", s.dt, s.kv), _ptr(do, "do", s.dt, s.q, allow_none=not bwd),
        _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
        _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse, allow_none=not bwd),
        _ptr(dq, "dq", s.dt, s.q, allow_none=not bwd),
        _ptr(dk, "dk", s.dt, s.kv, allow_none=not bwd),
        _ptr(dv, "dv", s.dt, s.kv, allow_none=not bwd),
        _ptr(ws, "ws", allow_none=not bwd),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(),
        None if stream2 is None else ctypes.c_void_p(stream2.cuda_stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # HGA_NOALLOC_SCRATCH_BYTES


def segment_pass_noalloc(cfg: Config, q, k, v, summ, sel, o, lse=None, do=None, dq=None,
                         dk=None, dv=None, bwd: bool = True) -> None:
    """hga_segment_pass_noalloc on the current stream: the pass with its
    scratch in the library's fixed per-GPU array instead of a workspace."""
    s = Shapes(cfg)
    torch = _torch()
    flags = HGA_STEP_BWD if bwd else 0
    _check(lib().hga_segment_pass_noalloc(
        ctypes.byref(cfg), flags, _ptr(q, "q", s.dt, s.q), _ptr(k, "k", s.dt, s.kv),
        _ptr(v, "v", s.dt, s.kv), _ptr(do, "do", s.dt, s.q, allow_none=not bwd),
        _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
        _ptr(o, "o", s.dt, s.q), _ptr(lse, "lse", torch.float32, s.lse, allow_none=not bwd),
        _ptr(dq, "dq", s.dt, s.q, allow_none=not bwd),
        _ptr(dk, "dk", s.dt, s.kv, allow_none=not bwd),
        _ptr(dv, "dv", s.dt, s.kv, allow_none=not bwd), _stream()))


def _host_args(cfg: Config, q, k_host, v_host, summ, sel, o, lse, do, dq, dk, dv, ws, bwd):
    s = Shapes(cfg)
    torch = _torch()
    return [_ptr(q, "q", s.dt, s.q), _host_ptr(k_host, "k_host", s.dt, s.kv),
            _host_ptr(v_host, "v_host", s.dt, s.kv),
            _ptr(do, "do", s.dt, s.q, allow_none=not bwd),
            _ptr(summ, "summ", torch.float32, s.summ), _ptr(sel, "sel", torch.int32, s.sel),
            _ptr(o, "o", s.dt, s.q),
            _ptr(lse, "lse", torch.float32, s.lse, allow_none=not bwd),
            _ptr(dq, "dq", s.dt, s.q, allow_none=not bwd),
            _ptr(dk, "dk", s.dt, s.kv, allow_none=not bwd),
            _ptr(dv, "dv", s.dt, s.kv, allow_none=not bwd),
            _ptr(ws, "ws"), ws.numel() * ws.element_size()]


def host_workspace(cfg: Config, op: int = HGA_OP_PASS_HOST):
    """A device workspace for hga_segment_step_host / hga_segment_pass_host."""
    torch = _torch()
    return torch.empty(max(workspace_size(cfg, op), 256), dtype=torch.uint8, device="cuda")


def segment_step_host(cfg: Config, seg: int, q, k_host, v_host, summ, sel, o, lse=None,
                      do=None, dq=None, dk=None, dv=None, ws=None, bwd: bool = True,
                      summaries_ready: bool = False) -> None:
    """hga_segment_step_host: k_host / v_host pinned host tensors [B, Hkv, S, D];
    ws of workspace_size(cfg, HGA_OP_STEP_HOST) bytes."""
    if ws is None:
        ws = host_workspace(cfg, HGA_OP_STEP_HOST)
    flags = (HGA_STEP_BWD if bwd else 0) | (HGA_STEP_SUMMARIES_READY if summaries_ready else 0)
    _check(lib().hga_segment_step_host(
        ctypes.byref(cfg), seg, flags,
        *_host_args(cfg, q, k_host, v_host, summ, sel, o, lse, do, dq, dk, dv, ws, bwd),
        _stream()))


def segment_pass_host(cfg: Config, q, k_host, v_host, summ, sel, o, lse=None, do=None,
                      dq=None, dk=None, dv=None, ws=None, bwd: bool = True,
                      stream2=None) -> None:
    """hga_segment_pass_host on the current stream, the fetches on stream2 (a torch
    stream at default priority) when given; ws of workspace_size(cfg,
    HGA_OP_PASS_HOST) bytes."""
    if ws is None:
        ws = host_workspace(cfg, HGA_OP_PASS_HOST)
    _check(lib().hga_segment_pass_host(
        ctypes.byref(cfg), HGA_STEP_BWD if bwd else 0,
        *_host_args(cfg, q, k_host, v_host, summ, sel, o, lse, do, dq, dk, dv, ws, bwd),
        _stream(), None if stream2 is None else ctypes.c_void_p(stream2.cuda_stream)))


class Buffers:
    """Device tensors of one layer's segmented pass (allocated with torch)."""

    def __init__(self, cfg: Config, device="cuda", bwd: bool = True, stream2=None):
        torch = _torch()
        s = Shapes(cfg)
        self.cfg = cfg
        self.summ = torch.zeros(s.summ, dtype=torch.float32, device=device)
        self.sel = torch.full(s.sel, -1, dtype=torch.int32, device=device)
        self.o = torch.zeros(s.q, dtype=s.dt, device=device)
        self.lse = torch.zeros(s.lse, dtype=torch.float32, device=device)
        if bwd:
            self.dq = torch.zeros(s.q, dtype=s.dt, device=device)
            self.dk = torch.zeros(s.kv, dtype=s.dt, device=device)
            self.dv = torch.zeros(s.kv, dtype=s.dt, device=device)
            # one workspace for the whole pass and for per-segment steps
            nbytes = max(workspace_size(cfg, HGA_OP_PASS), workspace_size(cfg, HGA_OP_STEP), 256)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        else:
            self.dq = self.dk = self.dv = self.ws = None
        # the second stream of the two-stream forms (default priority); a new
        # one unless the caller passes its own
        self.stream2 = stream2 if stream2 is not None else torch.cuda.Stream(device=device)

    def run_pass(self, q, k, v, do=None, bwd: bool = True, segments=None,
                 two_streams: bool = True, per_step: bool = False) -> None:
        """One layer's segmented pass: hga_segment_pass (segments alternating
        over two streams, or on the current stream only with two_streams=False),
        or, with per_step=True or a segment subset, hga_segment_step for each
        segment in order."""
        if segments is None and not per_step:
            segment_pass(self.cfg, q, k, v, self.summ, self.sel, self.o, self.lse, do,
                         self.dq, self.dk, self.dv, self.ws, bwd=bwd,
                         stream2=self.stream2 if two_streams else None)
            return
        nseg = self.cfg.seq_len // self.cfg.seg_len
        for s in (range(nseg) if segments is None else segments):
            segment_step(self.cfg, s, q, k, v, self.summ, self.sel, self.o, self.lse, do,
                         self.dq, self.dk, self.dv, self.ws, bwd=bwd)
