"""C-ABI checks that need no GPU: the library loads, exports every symbol
the header declares, and rejects bad arguments on the host with the
documented status before anything is enqueued (only invalid calls are made
here, so no kernel is ever launched)."""

import ctypes
import os
import re

import pytest

import sparse_long_context_query_amd as hga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hga.LIB_PATH):
        from sparse_long_context_query_amd import build_lib
        build_lib.build()
    return hga.lib()


def header_functions():
    with open(os.path.join(ROOT, "include", "hga.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hga_[a-z_]+)\s*\(", text)))


def test_exports_every_header_function(L):
    names = header_functions()
    assert {"hga_summarize", "hga_select", "hga_gather", "hga_attn_fwd", "hga_attn_bwd",
            "hga_segment_step", "hga_workspace_size", "hga_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def good_cfg(**kw):
    c = hga.Config(1, 16384, 1024, 64, 64, 32, 32, 8, 128, hga.HGA_BF16, 0.0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code,frag", [
    ("seq_len", 1000, hga.HGA_ERR_ARG, "multiple of seg_len"),
    ("hist_block", 48, hga.HGA_ERR_ARG, "multiple of hist_block"),
    ("query_block", 48, hga.HGA_ERR_ARG, "multiple of query_block"),
    ("n_q_heads", 30, hga.HGA_ERR_ARG, "multiple of n_kv_heads"),
    ("top_k", 0, hga.HGA_ERR_ARG, ">= 1"),
    ("batch", 0, hga.HGA_ERR_ARG, ">= 1"),
    ("head_dim", 96, hga.HGA_ERR_UNSUPPORTED, "head_dim"),
    ("dtype", 7, hga.HGA_ERR_UNSUPPORTED, "dtype"),
    ("top_k", 2000, hga.HGA_ERR_UNSUPPORTED, "top_k"),
    ("hist_block", 8, hga.HGA_ERR_UNSUPPORTED, "multiples of 16"),
])
def test_bad_config_rejected(L, field, value, code, frag):
    cfg = good_cfg(**{field: value})
    rc = L.hga_select(ctypes.byref(cfg), FAKE, FAKE, 1, FAKE, None)
    assert rc == code
    assert frag in hga.last_error()
    assert L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_STEP) == 0


def test_too_many_history_blocks(L):
    cfg = good_cfg(seq_len=1 << 20, seg_len=1024, hist_block=64)
    rc = L.hga_attn_fwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None, 0, None)
    assert rc == hga.HGA_ERR_UNSUPPORTED and "history blocks" in hga.last_error()


def test_null_config(L):
    assert L.hga_select(None, FAKE, FAKE, 0, FAKE, None) == hga.HGA_ERR_ARG
    assert "config is NULL" in hga.last_error()


@pytest.mark.parametrize("seg", [-1, 16, 1000])
def test_segment_out_of_range(L, seg):
    cfg = good_cfg()
    assert L.hga_select(ctypes.byref(cfg), FAKE, FAKE, seg, FAKE, None) == hga.HGA_ERR_ARG
    assert "out of range" in hga.last_error()
    rc = L.hga_segment_step(ctypes.byref(cfg), seg, 0, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                            FAKE, None, None, None, None, None, 0, None)
    assert rc == hga.HGA_ERR_ARG


def test_null_pointers(L):
    cfg = good_cfg()
    assert L.hga_select(ctypes.byref(cfg), None, FAKE, 1, FAKE, None) == hga.HGA_ERR_ARG
    assert "q is NULL" in hga.last_error()
    assert L.hga_attn_fwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, None, 1, FAKE, None, None, 0,
                          None) == hga.HGA_ERR_ARG
    assert "sel is NULL" in hga.last_error()
    rc = L.hga_attn_bwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, FAKE,
                        FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == hga.HGA_ERR_ARG and "dO is NULL" in hga.last_error()
    # backward step needs its gradient buffers
    rc = L.hga_segment_step(ctypes.byref(cfg), 1, hga.HGA_STEP_BWD, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == hga.HGA_ERR_ARG and "dq is NULL" in hga.last_error()
    assert L.hga_gather(ctypes.byref(cfg), FAKE, FAKE, FAKE, 1, None, FAKE, None) == hga.HGA_ERR_ARG


def test_bad_summary_range(L):
    cfg = good_cfg()
    for b0, b1 in [(-1, 3), (5, 4), (0, 257)]:
        assert L.hga_summarize(ctypes.byref(cfg), FAKE, b0, b1, FAKE, None) == hga.HGA_ERR_ARG
        assert "block range" in hga.last_error()


def test_workspace_too_small(L):
    cfg = good_cfg()
    need = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_BWD)
    # one fp32 row-sum per query row of a segment, then per mirror pair of
    # 32-key tiles (16 per KV head) two fp32 partial dK/dV tiles
    assert need == 1 * 32 * 1024 * 4 + 8 * 16 * 2 * 64 * 128 * 4
    rc = L.hga_attn_bwd(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE,
                        FAKE, FAKE, FAKE, need - 1, None)
    assert rc == hga.HGA_ERR_WORKSPACE
    rc = L.hga_segment_step(ctypes.byref(cfg), 1, hga.HGA_STEP_BWD, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert rc == hga.HGA_ERR_WORKSPACE
    assert L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_FWD) == 0
    assert L.hga_workspace_size(ctypes.byref(cfg), 9) == 0 and "unknown op" in hga.last_error()


def test_unknown_step_flags(L):
    cfg = good_cfg()
    rc = L.hga_segment_step(ctypes.byref(cfg), 1, 6, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == hga.HGA_ERR_ARG and "flags" in hga.last_error()


def test_profile_hooks_without_launches(L):
    hga.profile_begin()
    stats = hga.profile_end()
    assert set(stats) == set(hga.KERNEL_CLASSES)
    assert all(v == (0.0, 0) for v in stats.values())


def test_binding_rejects_cpu_tensors(L):
    import torch
    cfg = good_cfg(seq_len=2048, seg_len=512, top_k=8)
    s = hga.Shapes(cfg)
    q = torch.zeros(s.q, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        hga.select(cfg, q, torch.zeros(s.summ), 1, torch.zeros(s.sel, dtype=torch.int32))


def test_version(L):
    assert "gfx950" in hga.version()


def test_decode_step_validation(L):
    cfg = good_cfg()  # S 16384, L 1024, G 4
    ws = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_DECODE)
    # per (b, g): 32 history chunks (k 32 x Bh 64 / 64) + 16 local chunks of
    # 64 keys, 64 query rows each, D + 2 floats per row; then one score per
    # history block; then the two-stage top-k's candidate lists, one slot of
    # k (score, index) pairs per 128 history blocks (256 blocks: 2 slots)
    assert ws == (1 * 8 * (32 + 16) * 64 * (128 + 2) * 4 + 1 * 8 * 256 * 4
                  + 1 * 8 * 2 * 32 * (4 + 4))

    def call(pos, n, ws_bytes=ws, sel=FAKE):
        return L.hga_decode_step(ctypes.byref(cfg), pos, n, FAKE, FAKE, FAKE, FAKE, sel, FAKE,
                                 None, FAKE, ws_bytes, None)

    assert call(-1, 1) == hga.HGA_ERR_ARG and "outside" in hga.last_error()
    assert call(16383, 2) == hga.HGA_ERR_ARG and "outside" in hga.last_error()
    assert call(5, 0) == hga.HGA_ERR_ARG
    assert call(1020, 8) == hga.HGA_ERR_ARG and "segment boundary" in hga.last_error()
    assert call(0, 17) == hga.HGA_ERR_UNSUPPORTED and "G*n" in hga.last_error()
    assert call(2048, 4, sel=None) == hga.HGA_ERR_ARG and "sel is NULL" in hga.last_error()
    assert call(2048, 4, ws_bytes=ws - 1) == hga.HGA_ERR_WORKSPACE


def test_exact_step_validation(L):
    cfg = good_cfg()
    need = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_STEP_EXACT)
    assert need > L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_STEP)

    def call(c, seg=1, ws_bytes=need, hdk=FAKE):
        return L.hga_segment_step_exact(ctypes.byref(c), seg, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, FAKE, hdk, FAKE, FAKE, ws_bytes,
                                        None)

    assert call(cfg, seg=16) == hga.HGA_ERR_ARG
    assert call(cfg, hdk=None) == hga.HGA_ERR_ARG and "hist_dk is NULL" in hga.last_error()
    assert call(cfg, ws_bytes=need - 1) == hga.HGA_ERR_WORKSPACE
    f32 = good_cfg(dtype=hga.HGA_F32)
    assert call(f32) == hga.HGA_ERR_UNSUPPORTED and "bf16" in hga.last_error()
    wide = good_cfg(seg_len=2048, query_block=16)  # 128 query blocks per segment (> 64)
    assert call(wide) == hga.HGA_ERR_UNSUPPORTED and "64" in hga.last_error()


def test_exact_pass_validation(L):
    cfg = good_cfg()
    need = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_PASS_EXACT)
    # every segment's delta rows, the fp32 history sums of dK and dV, the list
    sums = 2 * cfg.batch * cfg.n_kv_heads * cfg.seq_len * cfg.head_dim * 4
    assert need >= (cfg.seq_len // cfg.seg_len) * cfg.batch * cfg.n_q_heads * cfg.seg_len * 4 + sums

    def call(c, ws_bytes=need, dk=FAKE):
        return L.hga_segment_pass_exact(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, dk, FAKE, FAKE, ws_bytes, None)

    assert call(cfg, dk=None) == hga.HGA_ERR_ARG and "dk is NULL" in hga.last_error()
    assert call(cfg, ws_bytes=need - 1) == hga.HGA_ERR_WORKSPACE
    f32 = good_cfg(dtype=hga.HGA_F32)
    assert call(f32) == hga.HGA_ERR_UNSUPPORTED and "bf16" in hga.last_error()
    wide = good_cfg(seg_len=2048, query_block=16)  # 128 query blocks per segment (> 64)
    assert call(wide) == hga.HGA_ERR_UNSUPPORTED and "64" in hga.last_error()


def _r256(x):
    return (x + 255) // 256 * 256


def test_host_tier_validation(L):
    cfg = good_cfg()
    B, Hkv, D, Bh, Lseg = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.hist_block, cfg.seg_len
    # window slots: the most one segment's query blocks can choose together
    C = min((Lseg // cfg.query_block) * cfg.top_k, (cfg.seq_len - Lseg) // Bh)
    assert C == 240
    window = 2 * _r256(B * Hkv * (C * Bh + Lseg) * D * 2) + _r256(B * Hkv * C * 4) + _r256(B * Hkv * 4)
    wsel = _r256(B * Hkv * (cfg.seq_len // cfg.query_block) * cfg.top_k * 4)
    step = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_STEP_HOST)
    two = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_PASS_HOST)
    bwd = _r256(L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_STEP))
    assert step == bwd + wsel + window and two == step + window
    # the window does not grow with the sequence once the selection bounds it
    long = good_cfg(seq_len=131072, hist_block=128, query_block=128, top_k=16)
    C2 = min(8 * 16, (131072 - 1024) // 128)
    assert C2 == 128
    win2 = 2 * _r256(B * Hkv * (C2 * 128 + 1024) * D * 2)
    need_long = L.hga_workspace_size(ctypes.byref(long), hga.HGA_OP_STEP_HOST)
    assert win2 < need_long < win2 + (12 << 20)  # + the backward's scratch and wsel
    assert need_long < (2 * B * Hkv * 131072 * D * 2) // 6  # vs K and V resident: 512 MiB
    f32 = good_cfg(dtype=hga.HGA_F32)
    assert L.hga_workspace_size(ctypes.byref(f32), hga.HGA_OP_STEP_HOST) == 0
    assert "bf16" in hga.last_error()

    def step_call(c, flags=hga.HGA_STEP_BWD, ws_bytes=step, seg=1, dq=FAKE):
        return L.hga_segment_step_host(ctypes.byref(c), seg, flags, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, FAKE, dq, FAKE, FAKE, FAKE, ws_bytes, None)

    def pass_call(c, flags=hga.HGA_STEP_BWD, ws_bytes=two, dq=FAKE):
        return L.hga_segment_pass_host(ctypes.byref(c), flags, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, FAKE, dq, FAKE, FAKE, FAKE, ws_bytes, None, FAKE)

    assert step_call(f32) == hga.HGA_ERR_UNSUPPORTED and "bf16" in hga.last_error()
    assert pass_call(f32) == hga.HGA_ERR_UNSUPPORTED
    assert step_call(cfg, seg=16) == hga.HGA_ERR_ARG
    assert step_call(cfg, dq=None) == hga.HGA_ERR_ARG and "dq is NULL" in hga.last_error()
    assert step_call(cfg, ws_bytes=step - 1) == hga.HGA_ERR_WORKSPACE
    # the forward alone needs the window too
    assert step_call(cfg, flags=0, ws_bytes=step - 1) == hga.HGA_ERR_WORKSPACE
    assert pass_call(cfg, ws_bytes=two - 1) == hga.HGA_ERR_WORKSPACE
    assert pass_call(cfg, flags=hga.HGA_STEP_BWD | hga.HGA_STEP_SUMMARIES_READY) == hga.HGA_ERR_ARG
    assert pass_call(cfg, flags=8) == hga.HGA_ERR_ARG and "flags" in hga.last_error()


def test_segment_pass_validation(L):
    cfg = good_cfg()
    two = L.hga_workspace_size(ctypes.byref(cfg), hga.HGA_OP_PASS)
    # bf16: the fp32 delta rows of every segment
    assert two == (cfg.seq_len // cfg.seg_len) * cfg.batch * cfg.n_q_heads * cfg.seg_len * 4
    f32 = good_cfg(dtype=hga.HGA_F32)
    step32 = L.hga_workspace_size(ctypes.byref(f32), hga.HGA_OP_STEP)
    assert L.hga_workspace_size(ctypes.byref(f32), hga.HGA_OP_PASS) >= 2 * step32

    def call(flags=hga.HGA_STEP_BWD, ws_bytes=two, stream2=FAKE, dq=FAKE):
        return L.hga_segment_pass(ctypes.byref(cfg), flags, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, dq, FAKE, FAKE, FAKE, ws_bytes, None, stream2)

    assert call(flags=hga.HGA_STEP_BWD | hga.HGA_STEP_SUMMARIES_READY) == hga.HGA_ERR_ARG
    assert call(flags=8) == hga.HGA_ERR_ARG and "flags" in hga.last_error()
    assert call(dq=None) == hga.HGA_ERR_ARG and "dq is NULL" in hga.last_error()
    assert call(ws_bytes=two - 1) == hga.HGA_ERR_WORKSPACE
    # on one stream the pass needs the same workspace
    assert call(ws_bytes=two - 1, stream2=None) == hga.HGA_ERR_WORKSPACE


def test_segment_pass_noalloc_validation(L):
    """The no-allocation pass: host-side rejections before anything is
    enqueued, including a scratch need beyond the fixed per-GPU array."""
    cfg = good_cfg()

    def call(c, flags=hga.HGA_STEP_BWD, dq=FAKE):
        return L.hga_segment_pass_noalloc(ctypes.byref(c), flags, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, dq, FAKE, FAKE, None)

    assert call(cfg, flags=8) == hga.HGA_ERR_ARG and "flags" in hga.last_error()
    assert call(cfg, dq=None) == hga.HGA_ERR_ARG and "dq is NULL" in hga.last_error()
    assert call(cfg, flags=hga.HGA_STEP_BWD | hga.HGA_STEP_SUMMARIES_READY) == hga.HGA_ERR_ARG
    # bf16: the delta rows of every segment, B*Hq*S*4 bytes; 2^20 tokens x 32
    # heads x 4 bytes is 128 MiB, beyond the 64 MiB array
    big = good_cfg(seq_len=1 << 20, seg_len=1024, hist_block=128)
    need = L.hga_workspace_size(ctypes.byref(big), hga.HGA_OP_PASS)
    assert need > hga.NOALLOC_SCRATCH_BYTES
    assert call(big) == hga.HGA_ERR_WORKSPACE and "scratch" in hga.last_error()
