#!/usr/bin/env python3
"""HGA hot-path benchmark on one MI355X.

One step = one whole segmented pass of one attention layer over the
16,384-token training workload (Qwen3-8B attention shape: 32 query heads,
8 KV heads, head_dim 128; segments of 1,024, history blocks of 64, top-k
32): the history blocks' summaries, then select, forward and backward of
every segment, through hga_segment_pass (bf16: one launch per kernel over
all segments).  Inputs are synthetic
(planted-direction N(0,1), seeded) and already resident in HBM when the
timed region starts.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HGA fwd+bwd tokens/s per layer at 16K (Qwen3-8B shape); % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="train_16k")
    ap.add_argument("--mode", default="planted", choices=["planted", "diverse"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-self", action="store_true")
    ap.add_argument("--no-diverse", action="store_true",
                    help="skip the extra timing on diverse-selection inputs")
    ap.add_argument("--no-dense-sdpa", action="store_true",
                    help="skip torch SDPA (flash backend) dense causal fwd+bwd at the same shape")
    ap.add_argument("--no-sequential", action="store_true",
                    help="skip the segment-by-segment form (hga_segment_step per segment)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 131K inference and 4 x 32K training workloads")
    ap.add_argument("--only", default=None,
                    help="comma-separated legs to run without the headline (for profiler runs): "
                         "hbm, sequential, infer_131k, batch4_32k, exact, decode, host_tier, "
                         "peaks; "
                         "prints one JSON line with those legs only")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV",
                    help="no GPU: per-kernel statistics (median over warm launches) of rocprofv3 "
                         "--kernel-trace CSV files, as a markdown table")
    ap.add_argument("--pmc-table", nargs="+", metavar="CSV",
                    help="no GPU: per-kernel averages of rocprofv3 --pmc counter CSV files, as a "
                         "markdown table")
    ap.add_argument("--skip-launches", type=int, default=1,
                    help="--trace-summary: launches of each kernel left out at the start (warm-up)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-step timing at the 131,072-token inference shape")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--streams", type=int, choices=(1, 2), default=2,
                    help="streams the timed passes use (1: every kernel of the pass on one "
                         "stream, as in the kernel-timing loops; used for kernel traces)")
    ap.add_argument("--no-exact", action="store_true",
                    help="skip the exact-gradient (history not detached) pass timing")
    ap.add_argument("--no-tier-131k", action="store_true",
                    help="skip the host-tier pass at the 131K inference shape")
    ap.add_argument("--no-fwd-only", action="store_true",
                    help="skip the forward-only pass timing (fwd_only_ms_per_pass)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured bf16 GEMM and copy rates (measured_peaks)")
    ap.add_argument("--no-hbm", action="store_true",
                    help="skip the summaries-at-131K and standalone-gather measurements")
    ap.add_argument("--no-host-tier", action="store_true",
                    help="skip the pass with K and V in pinned host memory")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a known-size "
                         "reference for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter CSVs of two rocprofv3 --pmc runs of "
                         "'bench.py --copy-calibration' (FETCH_SIZE, then WRITE_SIZE) into "
                         "per-launch HBM bytes, write profiles/traffic.json, print a table")
    return ap.parse_args()


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_CLASS_OF = {"tier_fetch_kernel": "tier_fetch", "tier_plan_kernel": "tier_plan",
                   "fwd_pass_kernel": "fwd", "dq_pass_kernel": "bwd_dq",
                   "dkdv_pass_kernel": "bwd_dkdv", "fwd_bf16_kernel": "fwd",
                   "dq_bf16_kernel": "bwd_dq", "dkdv_bf16_kernel": "bwd_dkdv",
                   "delta_kernel": "bwd_pre", "select_kernel": "select",
                   "select_multi_kernel": "select", "summarize_kernel": "summarize"}


def sources_sha256() -> str:
    """Hash of the kernel sources and the public header (the counters in
    profiles/traffic.json are used only for the sources they were taken on)."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "sparse_long_context_query_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def pmc_summary(fetch_csv, write_csv, workload):
    """Per-dispatch HBM bytes of each library kernel class from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, summed over the 8 XCDs), each scaled by what
    the same counter reads for the run's plain 256 MiB device copy."""
    import csv
    import re

    def load(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy_kib = 256 * 1024
    cf = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs]
    cw = [v for k, vs in write.items() if "copyBuffer" in k for v in vs]
    if not cf or not cw:
        raise SystemExit("no 256 MiB calibration copy in the counter files (run with --copy-calibration)")
    f_scale, w_scale = copy_kib / cf[0], copy_kib / cw[0]
    classes = {}
    for name in fetch:
        m = re.search("(" + "|".join(KERNEL_CLASS_OF) + ")", name)
        if not m:
            continue
        c = classes.setdefault(KERNEL_CLASS_OF[m.group(1)], {"fetch": [], "write": []})
        c["fetch"] += fetch[name]
        c["write"] += write.get(name, [])
    out = {"workload": workload, "sources_sha256": sources_sha256(),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "calibration": {"copy_kib": copy_kib, "fetch_kib": cf[0], "write_kib": cw[0]},
           "kernels": {}}
    for c, v in sorted(classes.items()):
        fk = sum(v["fetch"]) / len(v["fetch"])
        wk = sum(v["write"]) / len(v["write"]) if v["write"] else 0.0
        out["kernels"][c] = {"dispatches": len(v["fetch"]), "fetch_kib_raw": round(fk, 1),
                             "write_kib_raw": round(wk, 1),
                             "hbm_bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024))}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(f"calibration: 256 MiB copy reads FETCH_SIZE {cf[0]:.1f} KiB (scale {f_scale:.3f}), "
          f"WRITE_SIZE {cw[0]:.1f} KiB (scale {w_scale:.3f})")
    print("| kernel class | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MiB per launch |")
    print("|---|---:|---:|---:|---:|")
    for c, v in out["kernels"].items():
        print(f"| {c} | {v['dispatches']} | {v['fetch_kib_raw']:.1f} | {v['write_kib_raw']:.1f} | "
              f"{v['hbm_bytes_per_launch'] / 2**20:.2f} |")


def measured_traffic(kernel_class, workload):
    """HBM bytes per launch of a kernel class from profiles/traffic.json, or
    None when absent or taken on other sources or another workload."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("sources_sha256") != sources_sha256():
        return None
    k = t.get("kernels", {}).get(kernel_class)
    return k["hbm_bytes_per_launch"] if k else None


def timed_passes(buf, dev, bwd, n, profile_classes=None, two_streams=True):
    import torch
    import sparse_long_context_query_amd as hga
    torch.cuda.synchronize()
    if profile_classes:
        hga.profile_begin(profile_classes)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd,
                     two_streams=two_streams)
    end.record()
    torch.cuda.synchronize()
    prof = hga.profile_end() if profile_classes else None
    return start.elapsed_time(end) / n, prof


def single_passes(buf, dev, bwd, n, two_streams=True):
    """Median, minimum and maximum of n passes, each timed between its own
    pair of events on the current stream."""
    import statistics
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd,
                     two_streams=two_streams)
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in evs]
    return {"median_ms": round(statistics.median(t), 4), "min_ms": round(min(t), 4),
            "max_ms": round(max(t), 4), "passes": n}


def exact_bench(shape, dev, steps, warmup):
    """The exact-gradient pass (hga_segment_pass_exact): summaries, selection
    and forward of every segment, then every segment's queries (last
    segment first) give their dK/dV to the history blocks they selected,
    then local dK/dV plus those sums, and dQ.  Same inputs as the headline
    pass.  `steps_ms_per_step` times the same gradient through
    hga_segment_step_exact per segment."""
    import torch
    import sparse_long_context_query_amd as hga
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    z = lambda shp_, dt: torch.zeros(shp_, dtype=dt, device="cuda")  # noqa: E731
    summ, sel = z(s.summ, torch.float32), z(s.sel, torch.int32)
    o, lse, dq = z(s.q, s.dt), z(s.lse, torch.float32), z(s.q, s.dt)
    dk, dv = z(s.kv, s.dt), z(s.kv, s.dt)
    ws = torch.empty(hga.workspace_size(cfg, hga.HGA_OP_PASS_EXACT), dtype=torch.uint8,
                     device="cuda")
    hdk, hdv = z(s.kv, torch.float32), z(s.kv, torch.float32)
    ws_step = torch.empty(hga.workspace_size(cfg, hga.HGA_OP_STEP_EXACT), dtype=torch.uint8,
                          device="cuda")

    def one_pass():
        hga.segment_pass_exact(cfg, dev["q"], dev["k"], dev["v"], dev["do"], summ, sel, o, lse,
                               dq, dk, dv, ws)

    def one_step_pass():
        hdk.zero_()
        hdv.zero_()
        hga.summarize(cfg, dev["k"], 0, shape.seq_len // shape.hist_block, summ)
        for seg in reversed(range(shape.nseg)):
            hga.segment_step_exact(cfg, seg, dev["q"], dev["k"], dev["v"], dev["do"], summ, sel,
                                   o, lse, dq, dk, dv, hdk, hdv, ws_step)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(steps):
            fn()
        en.record()
        torch.cuda.synchronize()
        return st.elapsed_time(en) / steps

    ms = timed(one_pass)
    ms_steps = timed(one_step_pass)
    hga.profile_begin()
    one_pass()
    prof = hga.profile_end()
    return {"ms_per_step": round(ms, 4),
            "tokens_per_s": round(shape.batch * shape.seq_len / (ms * 1e-3), 1),
            "kernels_ms_per_pass": {c: round(v[0], 4) for c, v in prof.items() if v[1]},
            "steps_ms_per_step": round(ms_steps, 4),
            "note": "history not detached: later segments' queries also give dK/dV to the "
                    "blocks they selected (hga_segment_pass_exact)"}


PCIE5_X16_GBPS = 64.0  # host link of the MI355X: PCIe 5.0 x16, per direction


def host_tier_bench(shape, dev, steps, warmup):
    """The pass with K and V in pinned host memory (hga_segment_pass_host):
    per segment the summaries of the previous segment's blocks are read from
    the host, the selection is made, the union of the chosen blocks and the
    segment's own rows are fetched into an HBM window, and the attention
    reads the window; the next segment's fetch runs on a second stream
    meanwhile.  The fetch kernel reads host memory over the PCIe link: its
    roofline is the link's bandwidth, not HBM."""
    import numpy as np
    import torch
    import sparse_long_context_query_amd as hga
    cfg = hga.Config.from_shape(shape)
    buf = buffers(cfg, bwd=True)
    kh, vh = dev["k"].cpu().pin_memory(), dev["v"].cpu().pin_memory()
    ws2 = hga.host_workspace(cfg, hga.HGA_OP_PASS_HOST)
    ws1 = hga.host_workspace(cfg, hga.HGA_OP_STEP_HOST)

    def run_pass(stream2):
        hga.segment_pass_host(cfg, dev["q"], kh, vh, buf.summ, buf.sel, buf.o, buf.lse,
                              dev["do"], buf.dq, buf.dk, buf.dv, ws=ws2, stream2=stream2)

    def run_steps():
        for seg in range(shape.nseg):
            hga.segment_step_host(cfg, seg, dev["q"], kh, vh, buf.summ, buf.sel, buf.o, buf.lse,
                                  dev["do"], buf.dq, buf.dk, buf.dv, ws=ws1)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(steps):
            fn()
        en.record()
        torch.cuda.synchronize()
        return st.elapsed_time(en) / steps

    ms2 = timed(lambda: run_pass(buf.stream2))
    ms1 = timed(lambda: run_pass(None))
    ms_steps = timed(run_steps)
    torch.cuda.synchronize()
    hga.profile_begin()
    for _ in range(steps):
        run_pass(None)
    prof = {c: (v[0] / steps, v[1] // steps) for c, v in hga.profile_end().items()}
    # bytes the fetches move per pass: each segment's union of chosen blocks
    # and its own rows, K and V (the summaries are taken from the window)
    sel = buf.sel.cpu().numpy()
    nqb = shape.seg_len // shape.query_block
    rows = 0
    for seg in range(shape.nseg):
        part = sel[:, :, seg * nqb:(seg + 1) * nqb, :]
        for b in range(part.shape[0]):
            for g in range(part.shape[1]):
                u = part[b, g]
                rows += len(np.unique(u[u >= 0])) * shape.hist_block + shape.seg_len
    esz = 2
    fetch_bytes = rows * shape.head_dim * esz * 2
    fetch_ms, fetch_n = prof["tier_fetch"]
    achieved = fetch_bytes / (fetch_ms * 1e-3) / 1e9
    # a plain host-to-device copy of the whole K (hipMemcpyAsync from pinned
    # memory; the runtime runs it as a copy kernel) for comparison
    dst = torch.empty_like(dev["k"])
    for _ in range(2):
        dst.copy_(kh, non_blocking=True)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(5):
        dst.copy_(kh, non_blocking=True)
    en.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * kh.numel() * esz / (st.elapsed_time(en) * 1e-3) / 1e9
    kv_bytes = 2 * kh.numel() * esz
    return {"ms_per_step": round(ms2, 4),
            "tokens_per_s": round(shape.batch * shape.seq_len / (ms2 * 1e-3), 1),
            "one_stream_ms_per_step": round(ms1, 4),
            "steps_ms_per_step": round(ms_steps, 4),
            "kernels_ms_per_pass": {c: round(v[0], 4) for c, v in prof.items() if v[1]},
            "fetch": {"bound": "pcie", "bytes_per_pass": fetch_bytes,
                      "kernel_ms_per_pass": round(fetch_ms, 4), "launches": fetch_n,
                      "achieved": round(achieved, 1), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                      "frac": round(achieved / PCIE5_X16_GBPS, 4),
                      "h2d_memcpy_GBps": round(copy_gbps, 1)},
            "hbm_workspace_bytes": int(ws2.numel()),
            "kv_bytes_in_host_memory": kv_bytes,
            "note": "K and V in pinned host memory; per segment only the chosen blocks "
                    "and the segment's rows are fetched into HBM (hga_segment_pass_host)"}


def host_tier_131k_bench(steps):
    """The 131,072-token inference workload, forward only, with K and V in
    pinned host memory (hga_segment_pass_host, fetches on a second stream)
    against the resident pass (hga_segment_pass) on the same inputs.  Inputs
    are N(0,1) drawn on the GPU with no planted directions, so the 8 query
    blocks of a segment mostly choose different blocks and the window is
    near its 128-block capacity: the tier's heaviest case."""
    import numpy as np
    import torch
    import sparse_long_context_query_amd as hga
    from synth import WORKLOADS
    shape = WORKLOADS["infer_131k"]
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    q = torch.randn(s.q, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(s.kv, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(s.kv, generator=gen, device="cuda").to(torch.bfloat16)
    kh, vh = k.cpu().pin_memory(), v.cpu().pin_memory()
    buf = buffers(cfg, bwd=False)
    ws = hga.host_workspace(cfg, hga.HGA_OP_PASS_HOST)

    def tier():
        hga.segment_pass_host(cfg, q, kh, vh, buf.summ, buf.sel, buf.o, buf.lse, bwd=False,
                              ws=ws, stream2=buf.stream2)

    def resident():
        buf.run_pass(q, k, v, None, bwd=False)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(steps):
            fn()
        en.record()
        torch.cuda.synchronize()
        return st.elapsed_time(en) / steps

    ms_tier = timed(tier)
    sel = buf.sel.cpu().numpy()
    ms_res = timed(resident)
    nqb = shape.seg_len // shape.query_block
    rows = 0
    unions = []
    for seg in range(shape.nseg):
        part = sel[:, :, seg * nqb:(seg + 1) * nqb, :]
        for b in range(part.shape[0]):
            for g in range(part.shape[1]):
                u = part[b, g]
                n = len(np.unique(u[u >= 0]))
                unions.append(n)
                rows += n * shape.hist_block + shape.seg_len
    fetch_bytes = rows * shape.head_dim * 2 * 2
    tokens = shape.batch * shape.seq_len
    return {"workload": "infer_131k forward (K, V in pinned host memory)",
            "data": "synthetic N(0,1) drawn on the GPU, no planted directions",
            "ms_per_pass": round(ms_tier, 3),
            "tokens_per_s": round(tokens / (ms_tier * 1e-3), 1),
            "resident_ms_per_pass": round(ms_res, 3),
            "resident_tokens_per_s": round(tokens / (ms_res * 1e-3), 1),
            "fetch_bytes_per_pass": fetch_bytes,
            "fetch_GBps_over_pass": round(fetch_bytes / (ms_tier * 1e-3) / 1e9, 1),
            "mean_union_blocks": round(float(np.mean(unions)), 1),
            "window_slots": min(nqb * shape.top_k,
                                (shape.seq_len - shape.seg_len) // shape.hist_block),
            "hbm_workspace_bytes": int(ws.numel()),
            "kv_bytes_in_host_memory": 2 * kh.numel() * 2}


def hbm_kernels_bench(shape, dev, buf, steps):
    """The HBM-bound rows on their own, against the 8 TB/s HBM peak (launch
    times stamped by the kernels' own dispatches):
      - a1, summaries of every block of the 131K workload's K (256 MiB);
      - a4, the standalone gather of the last 16K segment's chosen blocks
        (K and V read and written once), on the headline pass's selection."""
    import torch
    import sparse_long_context_query_amd as hga
    from synth import WORKLOADS
    out = {}
    big = WORKLOADS["infer_131k"]
    bcfg = hga.Config.from_shape(big)
    bs = hga.Shapes(bcfg)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    kb = torch.randn(bs.kv, generator=gen, device="cuda").to(torch.bfloat16)
    summ = torch.zeros(bs.summ, dtype=torch.float32, device="cuda")
    nblk = big.seq_len // big.hist_block

    def stamped(cls, fn):
        fn()
        torch.cuda.synchronize()
        hga.profile_begin([cls])
        for _ in range(steps):
            fn()
        prof = hga.profile_end()
        ms, n = prof[cls]
        return ms / n

    ms = stamped("summarize", lambda: hga.summarize(bcfg, kb, 0, nblk, summ))
    nbytes = kb.numel() * 2 + summ.numel() * 4
    out["summarize_131k"] = {"bytes": nbytes, "us_per_launch": round(ms * 1e3, 2),
                             "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del kb, summ
    cfg = hga.Config.from_shape(shape)
    s = hga.Shapes(cfg)
    seg = shape.nseg - 1
    ko = torch.empty(s.gather, dtype=s.dt, device="cuda")
    vo = torch.empty(s.gather, dtype=s.dt, device="cuda")
    ms = stamped("gather", lambda: hga.gather(cfg, dev["k"], dev["v"], buf.sel, seg, ko, vo))
    # HBM bytes at the least: each distinct chosen block's K and V read once
    # (query blocks that chose the same block re-read it from the caches),
    # and everything written; the per-query-block count reads every copy
    import numpy as np
    nqb = shape.seg_len // shape.query_block
    rows = buf.sel[:, :, seg * nqb:(seg + 1) * nqb].cpu().numpy()
    distinct = sum(len(np.unique(r[r >= 0])) for r in rows.reshape(-1, nqb * shape.top_k))
    written = 2 * ko.numel() * ko.element_size()
    nbytes = distinct * shape.hist_block * shape.head_dim * 2 * 2 + written
    out["gather_16k_last_segment"] = {"bytes": nbytes, "per_query_block_bytes": 2 * written,
                                      "distinct_blocks": distinct,
                                      "us_per_launch": round(ms * 1e3, 2),
                                      "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                    4)}
    return out


def decode_bench(n_steps, news=(1, 16)):
    """Decode steps (hga_decode_step) at the 131,072-token inference shape:
    B 1, 32 query / 8 KV heads, D 128, segments of 1,024, blocks of 128,
    top-k 16, bf16.  The steps lie in the last segment, whose history is the
    1,016 summarized blocks before it; positions are spread evenly over the
    segment so that the local part averages half a segment.  Inputs are
    N(0,1) drawn on the GPU: a step's work is fixed by the shapes (k*Bh
    history keys plus the local keys), not by which blocks win.  Reports
    microseconds per step and, for the attention kernel, algorithmic HBM
    bytes (K/V rows of the key set, the query rows, the chunk partial sums
    written) over its measured time against the 8 TB/s peak."""
    import ctypes
    import torch
    import sparse_long_context_query_amd as hga
    from synth import WORKLOADS
    shape = WORKLOADS["infer_131k"]
    cfg = hga.Config.from_shape(shape)
    B, S, L, Bh, K = shape.batch, shape.seq_len, shape.seg_len, shape.hist_block, shape.top_k
    Hq, Hkv, D = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    G = Hq // Hkv
    gen = torch.Generator(device="cuda").manual_seed(0)
    kv = (B, Hkv, S, D)
    k = torch.randn(kv, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(kv, generator=gen, device="cuda").to(torch.bfloat16)
    qseg = torch.randn((B, Hq, L, D), generator=gen, device="cuda").to(torch.bfloat16)
    t0 = S - L
    s = hga.Shapes(cfg)
    summ = torch.zeros(s.summ, dtype=torch.float32, device="cuda")
    hga.summarize(cfg, k, 0, t0 // Bh, summ)
    sel = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(hga.workspace_size(cfg, hga.HGA_OP_DECODE), dtype=torch.uint8, device="cuda")
    nht = min(K, t0 // Bh) * Bh
    res = {"workload": "infer_131k decode (last segment, history 1,016 blocks)",
           "data": "synthetic N(0,1) drawn on the GPU"}
    for n in news:
        steps = min(n_steps, (L - 1) // n)
        stride = (L - 1 - n) // max(steps - 1, 1)
        pos = [t0 + 1 + i * stride for i in range(steps)]
        qs = [qseg[:, :, p - t0:p - t0 + n].contiguous() for p in pos]
        o = torch.empty((B, Hq, n, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device="cuda")
        for i in range(3):
            hga.decode_step(cfg, pos[i], qs[i], k, v, summ, sel, o, lse, ws)
        torch.cuda.synchronize()
        # whole steps, timed with events around the loop: through the C ABI
        # with each step's arguments prepared beforehand (the shapes were
        # checked by the binding's calls above), then through the binding
        clib = hga.lib()
        vp = ctypes.c_void_p
        stream = vp(torch.cuda.current_stream().cuda_stream)
        fixed = [vp(t.data_ptr()) for t in (k, v, summ, sel, o, lse, ws)]
        calls = [(ctypes.byref(cfg), p, n, vp(q.data_ptr()), *fixed, ws.numel(), stream)
                 for p, q in zip(pos, qs)]
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for a in calls:
            if clib.hga_decode_step(*a) != 0:
                raise RuntimeError(hga.last_error())
        en.record()
        torch.cuda.synchronize()
        step_ms = st.elapsed_time(en) / steps
        st.record()
        for p, q in zip(pos, qs):
            hga.decode_step(cfg, p, q, k, v, summ, sel, o, lse, ws)
        en.record()
        torch.cuda.synchronize()
        binding_ms = st.elapsed_time(en) / steps
        # per-kernel times in a second loop (events around each launch)
        hga.profile_begin(["select", "decode", "decode_merge"])
        for p, q in zip(pos, qs):
            hga.decode_step(cfg, p, q, k, v, summ, sel, o, lse, ws)
        prof = hga.profile_end()
        R = G * n
        ck = 64 if R <= 32 else 128  # keys per chunk of the bf16 attention launch
        nbytes = 0
        for p in pos:
            nloc = p + n - t0
            nc = -(-nht // ck) + -(-nloc // ck)
            nbytes += B * Hkv * ((nht + nloc) * D * 2 * 2 + R * D * 2 + nc * R * (D + 2) * 4)
        attn_ms = prof["decode"][0]
        gbs = nbytes / (attn_ms * 1e-3) / 1e9
        res[f"n{n}"] = {
            "steps": steps, "us_per_step": round(step_ms * 1e3, 2),
            "tokens_per_s": round(B * n / (step_ms * 1e-3), 1),
            "us_per_step_python_binding": round(binding_ms * 1e3, 2),
            "kernel_us_per_step": {c: round(prof[c][0] * 1e3 / prof[c][1], 2)
                                   for c in ("select", "decode", "decode_merge") if prof[c][1]},
            "attn_bytes_per_step": int(nbytes / steps),
            "attn_hbm_gbs": round(gbs, 1), "attn_frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        }
        log(f"[bench] decode n={n}: {res[f'n{n}']}")
    del k, v, qseg, summ, ws
    return res


def cpu_baseline(inp, shape, budget_s):
    """The fp64 oracle on the host over a bounded sample of the workload:
    whole segments of one (sequence, KV head) group, forward + backward,
    scaled to the full pass by the sample's share of the algorithmic FLOPs."""
    import numpy as np
    from oracle import hga_oracle as orc
    from sparse_long_context_query_amd import work
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    total = work.flops(shape)
    kbar = orc.block_summaries(inp["k"], shape.hist_block)
    t_start = time.perf_counter()
    # whole segments of one (sequence, KV head) group after another until the
    # time budget is spent; the selection of a segment covers every group
    order = [1, shape.nseg - 1] + list(range(2, shape.nseg - 1))
    groups = [(b, g) for b in range(shape.batch) for g in range(shape.n_kv_heads)]
    sels = {}
    sample_fl = 0.0
    done = []
    for b, g in groups:
        for s in order:
            if time.perf_counter() - t_start > budget_s and done:
                break
            if s not in sels:
                sels[s] = orc.select_segment(inp["q"], inp["k"], shape, s, kbar=kbar)
            O, LSE = orc.segment_forward(inp["q"], inp["k"], inp["v"], sels[s], shape, s,
                                         groups=[(b, g)])
            if shape.bwd:
                orc.segment_backward(inp["q"], inp["k"], inp["v"], inp["do"], sels[s], shape, s,
                                     O, LSE, groups=[(b, g)])
            f = work.flops(shape, segments=[s], groups=1)
            sample_fl += f["fwd"] + (f["bwd"] if shape.bwd else 0)
            done.append((b, g, s))
    elapsed = time.perf_counter() - t_start
    frac = sample_fl / (total["fwd"] + (total["bwd"] if shape.bwd else 0))
    t_full = elapsed / frac
    del np
    ngroups = len({(b, g) for b, g, _ in done})
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "")
    except OSError:
        pass
    return {
        "value": shape.batch * shape.seq_len / t_full,
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": model,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, fwd{'+bwd' if shape.bwd else ''} of {len(done)} "
                   f"(segment, sequence, KV head) groups over {ngroups} KV heads, segment "
                   f"selection included ({elapsed:.1f} s), scaled by their {frac:.4f} share "
                   f"of the pass FLOPs"),
    }


def short_kernel_name(name: str) -> str:
    """Kernel name without namespace and arguments, template arguments kept
    (works on both the mangled and the demangled forms rocprofv3 prints)."""
    import re
    m = re.search(r"_GLOBAL__N_1(\d+)", name)
    if m:  # mangled: _ZN3hga12_GLOBAL__N_1<len><name>I<args>E...
        n = int(m.group(1))
        base, rest = name[m.end():m.end() + n], name[m.end() + n:]
        args = []
        if rest.startswith("I"):
            for a in re.finditer(r"DF16b|Li(\d+)E|f(?=[ELi])", rest[1:rest.find("EE") + 1]):
                args.append("bf16" if a.group(0) == "DF16b" else (a.group(1) or "float"))
        return base + (f"<{','.join(args)}>" if args else "")
    m = re.search(r"(\w+)(<[^()]*>)?\(", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:40]


def trace_summary(paths, skip):
    """Per-kernel statistics of rocprofv3 kernel-trace CSVs: every launch,
    and the launches after the first `skip` of each kernel (warm), with
    median and mean; for the whole-pass kernels of the 16K training
    workload also the algorithmic TFLOP/s and fraction of the bf16 peak at
    the warm median."""
    import csv
    import statistics
    from sparse_long_context_query_amd import work
    from synth import WORKLOADS
    durs = {}
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            durs.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(d)
    fl = work.flops(WORKLOADS["train_16k"])
    flop_of = {"fwd_pass_kernel<128>": fl["fwd"], "dq_pass_kernel<128>": fl["bwd_dq"],
               "dkdv_pass_kernel<128>": fl["bwd_dkdv"]}
    print(f"| kernel | launches | mean us | warm launches | warm median us | warm mean us | "
          f"warm min us | algorithmic TFLOP/s at warm median | fraction of 2.5 PFLOP/s |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for k, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        w = v[skip:] if len(v) > skip else v
        med = statistics.median(w)
        f = flop_of.get(k)
        tf = f"{f / (med * 1e-6) / 1e12:.1f}" if f else ""
        fr = f"{f / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f}" if f else ""
        print(f"| {k} | {len(v)} | {statistics.mean(v):.1f} | {len(w)} | {med:.1f} | "
              f"{statistics.mean(w):.1f} | {min(w):.1f} | {tf} | {fr} |")


# counters whose per-dispatch value is a sum over the 8 XCDs of a per-XCD
# clock count (GRBM) or a sum over SIMDs (SQ_*_CYCLES), and derived ones
PMC_DERIVED_NOTE = ("MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * "
                    "SIMDs); LDSBankConflict = 100 * sum(SQ_LDS_BANK_CONFLICT) / "
                    "max(GRBM_GUI_ACTIVE) / CUs (rocprofv3's own definitions); clock = "
                    "GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration, for dispatches of 100 us "
                    "or more")


def pmc_table(paths):
    """Per-kernel averages of rocprofv3 --pmc counter CSVs (one row per
    kernel, one column per counter), with the clock the dispatches ran at."""
    import csv
    vals, durs = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_kernel_name(r["Kernel_Name"])
            if "at::" in r["Kernel_Name"] or "copyBuffer" in r["Kernel_Name"]:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            durs.setdefault(k, {})[(path, r["Dispatch_Id"])] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    counters = sorted({c for v in vals.values() for c in v})
    print("| kernel | dispatches | mean us | clock GHz | " + " | ".join(counters) + " |")
    print("|---|---:|---:|---:|" + "---:|" * len(counters))
    for k in sorted(vals, key=lambda k: -sum(durs[k].values())):
        d = sum(durs[k].values()) / len(durs[k])
        gui = vals[k].get("GRBM_GUI_ACTIVE")
        # GRBM_GUI_ACTIVE also counts a little time around the dispatch, so
        # the clock is shown for long dispatches only
        clk = f"{sum(gui) / len(gui) / 8 / d:.2f}" if gui and d >= 100e3 else ""
        cells = []
        for c in counters:
            x = vals[k].get(c)
            cells.append("" if not x else f"{sum(x) / len(x):.4g}")
        print(f"| {k} | {len(durs[k])} | {d / 1e3:.1f} | {clk} | " + " | ".join(cells) + " |")
    print()
    print(PMC_DERIVED_NOTE)


def stamped_kernels(fn, n):
    """Runs fn() n times with every library kernel's dispatches stamping HIP
    events; {class: (ms per call, launches per call)}."""
    import torch
    import sparse_long_context_query_amd as hga
    torch.cuda.synchronize()
    hga.profile_begin()
    for _ in range(n):
        fn()
    prof = hga.profile_end()
    return {c: (v[0] / n, v[1] // n) for c, v in prof.items() if v[1]}


_STREAM2 = None


def buffers(cfg, bwd: bool = True):
    """hga.Buffers whose second stream is one stream shared by every leg.
    HIP runs streams on a few hardware queues (four by default), and two
    streams that share a queue run one after the other.  With a new second
    stream per leg, which queue it shared depended on how many legs had run
    before, and in the full run the host-RAM tier's two streams lost their
    overlap (6.5 ms per pass against 4.4 ms when that leg ran alone); one
    second stream for the whole run keeps the pairing the same in every
    leg."""
    global _STREAM2
    import torch
    import sparse_long_context_query_amd as hga
    if _STREAM2 is None:
        _STREAM2 = torch.cuda.Stream()  # default priority
    return hga.Buffers(cfg, bwd=bwd, stream2=_STREAM2)


def event_timed(fn, n, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(n):
        fn()
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) / n


def fractions(shape, kern, bwd):
    """fwd / bwd algorithmic TFLOP/s and fractions of the bf16 peak from
    per-class kernel times (ms per pass)."""
    from sparse_long_context_query_amd import work
    fl = work.flops(shape)
    out = {"kernels_ms_per_pass": {c: round(v[0], 4) for c, v in kern.items()},
           "launches_per_pass": {c: v[1] for c, v in kern.items()}}
    fwd_ms = kern["fwd"][0]
    out["fwd_tflops"] = round(fl["fwd"] / (fwd_ms * 1e-3) / 1e12, 1)
    out["fwd_frac_peak"] = round(fl["fwd"] / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    if bwd:
        bwd_ms = sum(kern[c][0] for c in ("bwd_pre", "bwd_dq", "bwd_dkdv") if c in kern)
        out["bwd_tflops"] = round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12, 1)
        out["bwd_frac_peak"] = round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    return out


def sequential_bench(shape, dev, steps, warmup):
    """The workload's segment-by-segment form: hga_segment_step for segment
    0, 1, ... in order, each step summarizing the blocks the previous
    segment closed, then selecting, running the forward and the backward of
    its own segment (the one-segment kernels), all on one stream.  Also on
    two streams: the summaries of every block first (hga_summarize), then
    the steps alternate between the streams (HGA_STEP_SUMMARIES_READY, one
    workspace per stream), so a step's kernels can fill the CUs the
    previous step's leave idle."""
    import torch
    import sparse_long_context_query_amd as hga
    from sparse_long_context_query_amd import work
    cfg = hga.Config.from_shape(shape)
    bwd = shape.bwd
    buf = buffers(cfg, bwd=bwd)
    ws2 = torch.empty_like(buf.ws) if bwd else None
    nseg = shape.nseg
    nblk = (shape.seq_len - shape.seg_len) // shape.hist_block

    def one_stream():
        for s_ in range(nseg):
            hga.segment_step(cfg, s_, dev["q"], dev["k"], dev["v"], buf.summ, buf.sel, buf.o,
                             buf.lse, dev.get("do"), buf.dq, buf.dk, buf.dv, buf.ws, bwd=bwd)

    main = torch.cuda.current_stream()
    other = buf.stream2

    def two_streams():
        hga.summarize(cfg, dev["k"], 0, nblk, buf.summ)
        other.wait_stream(main)
        for s_ in range(nseg):
            st, ws = (main, buf.ws) if s_ % 2 == 0 else (other, ws2)
            with torch.cuda.stream(st):
                hga.segment_step(cfg, s_, dev["q"], dev["k"], dev["v"], buf.summ, buf.sel,
                                 buf.o, buf.lse, dev.get("do"), buf.dq, buf.dk, buf.dv, ws,
                                 bwd=bwd, summaries_ready=True)
        main.wait_stream(other)

    ms1 = event_timed(one_stream, steps, warmup)
    ms2 = event_timed(two_streams, steps, warmup)
    kern = stamped_kernels(one_stream, steps)
    fl = work.flops(shape)
    tokens = shape.batch * shape.seq_len
    out = {"ms_per_pass": round(ms1, 4), "tokens_per_s": round(tokens / (ms1 * 1e-3), 1),
           "two_streams_ms_per_pass": round(ms2, 4),
           "two_streams_tokens_per_s": round(tokens / (ms2 * 1e-3), 1),
           "pass_frac_peak": round((fl["fwd"] + (fl["bwd"] if bwd else 0)) / (ms1 * 1e-3)
                                   / 1e12 / PEAK_BF16_TFLOPS, 4)}
    out.update(fractions(shape, kern, bwd))
    out["note"] = ("hga_segment_step per segment in order (summarize the blocks the previous "
                   "segment closed, select, forward, backward), one-segment kernels; "
                   "kernel times from one-stream passes")
    del buf, ws2
    return out


WORKLOAD_NOTES = {
    "infer_131k": ("forward only; local causal window of 1,024 read as segment-aligned (segments "
                   "of 1,024 tokens, causal within the segment, history = whole blocks before "
                   "the segment); a sliding token window is not the reading taken"),
    "batch4_32k": "four sequences of 32,768 tokens, per-sequence seeds and planted directions",
}


def workload_bench(name, steps, warmup):
    """A whole segmented pass (hga_segment_pass) of another workload on its
    planted-direction inputs, resident in HBM: tokens/s, and the forward and
    backward kernels' fractions of the bf16 peak from stamped passes."""
    import torch
    import sparse_long_context_query_amd as hga
    from sparse_long_context_query_amd import work
    from synth import WORKLOADS, make_inputs
    shape = WORKLOADS[name]
    log(f"[bench] {name}: generating inputs")
    inp = make_inputs(shape, seed=0)
    dev = {k: torch.from_numpy(inp[k]).cuda().to(torch.bfloat16)
           for k in ("q", "k", "v", "do") if inp.get(k) is not None}
    del inp
    cfg = hga.Config.from_shape(shape)
    bwd = shape.bwd
    buf = buffers(cfg, bwd=bwd)

    def one():
        buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd)

    log(f"[bench] {name}: timing")
    ms = event_timed(one, steps, warmup)
    kern = stamped_kernels(one, steps)
    fl = work.flops(shape)
    tokens = shape.batch * shape.seq_len
    out = {"workload": name, "batch": shape.batch, "seq_len": shape.seq_len,
           "seg_len": shape.seg_len, "hist_block": shape.hist_block,
           "query_block": shape.query_block, "top_k": shape.top_k,
           "step": "summarize + select + fwd" + (" + bwd" if bwd else "") +
                   " of all segments (hga_segment_pass)",
           "data": "synthetic (planted-direction N(0,1), seed 0)",
           "ms_per_pass": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
           "algorithmic_flop_per_pass": fl["fwd"] + (fl["bwd"] if bwd else 0),
           "pass_frac_peak": round((fl["fwd"] + (fl["bwd"] if bwd else 0)) / (ms * 1e-3)
                                   / 1e12 / PEAK_BF16_TFLOPS, 4),
           "note": WORKLOAD_NOTES[name]}
    out.update(fractions(shape, kern, bwd))
    del buf, dev
    torch.cuda.empty_cache()
    return out



def only_legs(args, shape):
    """The legs named by --only, without the headline (profiler runs)."""
    import torch
    import sparse_long_context_query_amd as hga
    from synth import make_inputs
    legs = [x.strip() for x in args.only.split(",") if x.strip()]
    out = {"only": legs}
    dev = buf = None
    if {"hbm", "sequential", "exact", "host_tier"} & set(legs):
        inp = make_inputs(shape, seed=0, mode=args.mode)
        dev = {k: torch.from_numpy(inp[k]).cuda().to(torch.bfloat16)
               for k in ("q", "k", "v", "do") if inp.get(k) is not None}
        buf = buffers(hga.Config.from_shape(shape), bwd=shape.bwd)
        for _ in range(2):
            buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=shape.bwd)
        torch.cuda.synchronize()
    for leg in legs:
        log(f"[bench] leg {leg}")
        if leg == "hbm":
            out[leg] = hbm_kernels_bench(shape, dev, buf, args.steps)
        elif leg == "sequential":
            out[leg] = sequential_bench(shape, dev, args.steps, args.warmup)
        elif leg in ("infer_131k", "batch4_32k"):
            out[leg] = workload_bench(leg, args.steps, args.warmup)
        elif leg == "exact":
            out[leg] = exact_bench(shape, dev, args.steps, args.warmup)
        elif leg == "host_tier":
            out[leg] = host_tier_bench(shape, dev, args.steps, args.warmup)
        elif leg == "decode":
            out[leg] = decode_bench(args.decode_steps)
        elif leg == "peaks":
            out[leg] = measured_peaks()
        else:
            raise SystemExit(f"unknown leg {leg!r}")
    return out


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.skip_launches)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the HGA hot "
              "path here has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_long_context_query_amd as hga
    from sparse_long_context_query_amd import work
    from synth import WORKLOADS, make_inputs

    if not os.path.exists(hga.LIB_PATH):
        from sparse_long_context_query_amd import build_lib
        build_lib.build()
    hga.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    shape = WORKLOADS[args.workload]
    bwd = shape.bwd
    if args.only:
        print(json.dumps(only_legs(args, shape)), flush=True)
        return
    log(f"[bench] generating {shape.name} inputs ({args.mode})")
    inp = make_inputs(shape, seed=0, mode=args.mode)
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    dev = {k: torch.from_numpy(inp[k]).cuda().to(dt)
           for k in ("q", "k", "v", "do") if inp.get(k) is not None}
    cfg = hga.Config.from_shape(shape)
    buf = buffers(cfg, bwd=bwd)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        buf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd,
                     two_streams=args.streams == 2)
    torch.cuda.synchronize()

    # value: K passes (hga_segment_pass), nothing profiled
    log(f"[bench] timing {args.steps} passes ({args.streams} stream(s))")
    ms, _ = timed_passes(buf, dev, bwd, args.steps, two_streams=args.streams == 2)
    # the same passes one by one, each between its own pair of events: the
    # median and the spread of single passes (ms_per_step stays the loop's)
    per_pass = single_passes(buf, dev, bwd, args.steps, two_streams=args.streams == 2)
    # kernel times: a second loop of K one-stream passes in which every
    # kernel's own dispatch stamps HIP start / stop events (the stamps add a
    # little idle time between kernels, so the pass time above never comes
    # from this loop; with the f32 pass on two streams neighbouring
    # segments' kernels would overlap and share the CUs)
    log(f"[bench] timing {args.steps} one-stream passes with every kernel's dispatches "
        f"stamping events")
    ms_prof, prof = timed_passes(buf, dev, bwd, args.steps, profile_classes=hga.KERNEL_CLASSES,
                                 two_streams=False)
    prof_all = {c: (v[0] / args.steps, v[1] // args.steps) for c, v in prof.items()}
    dominant = max(prof_all, key=lambda c: prof_all[c][0])
    log(f"[bench] per-kernel ms per pass: "
        + ", ".join(f"{c}={v[0]:.3f}/{v[1]}" for c, v in prof_all.items() if v[1]))
    dom_ms, dom_n = prof[dominant]

    fl = work.flops(shape)
    tokens = shape.batch * shape.seq_len
    value = tokens / (ms / 1e3)
    dom_flops = {"fwd": fl["fwd"], "bwd_dq": fl["bwd_dq"], "bwd_dkdv": fl["bwd_dkdv"]}.get(dominant)
    per_launch_flop = dom_flops * args.steps / dom_n if dom_flops else None
    avg_launch_ms = dom_ms / dom_n
    achieved = per_launch_flop / (avg_launch_ms * 1e-3) / 1e12 if per_launch_flop else None

    fwd_ms = prof_all["fwd"][0]
    bwd_ms = sum(prof_all[c][0] for c in ("bwd_pre", "bwd_dq", "bwd_dkdv"))
    extras = {
        "kernels_ms_per_pass": {c: round(v[0], 4) for c, v in prof_all.items() if v[1]},
        "launches_per_pass": {c: v[1] for c, v in prof_all.items() if v[1]},
        "fwd_tflops": round(fl["fwd"] / (fwd_ms * 1e-3) / 1e12, 1),
        "fwd_frac_peak": round(fl["fwd"] / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }
    if bwd:
        extras["bwd_tflops"] = round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12, 1)
        extras["bwd_frac_peak"] = round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    pass_tf = (fl["fwd"] + (fl["bwd"] if bwd else 0)) / (ms * 1e-3) / 1e12
    extras["pass_tflops_algorithmic"] = round(pass_tf, 1)
    extras["pass_frac_peak"] = round(pass_tf / PEAK_BF16_TFLOPS, 4)

    if not args.no_hbm and shape.name == "train_16k":
        log("[bench] HBM-bound rows (summaries at 131K, standalone gather)")
        extras["hbm_kernels"] = hbm_kernels_bench(shape, dev, buf, args.steps)
    if not args.no_dense_self:
        dshape = shape.replace(seg_len=shape.seq_len, top_k=1)
        dcfg = hga.Config.from_shape(dshape)
        dbuf = buffers(dcfg, bwd=bwd)
        for _ in range(2):
            dbuf.run_pass(dev["q"], dev["k"], dev["v"], dev.get("do"), bwd=bwd)
        dms, _ = timed_passes(dbuf, dev, bwd, 3)
        extras["dense_causal_same_kernels_ms"] = round(dms, 3)
        extras["speedup_vs_dense_same_kernels"] = round(dms / ms, 2)
        del dbuf
    if not args.no_dense_sdpa:
        log("[bench] torch SDPA dense causal comparator")
        extras.update(dense_sdpa(dev, shape, bwd, ms))
    if bwd and not args.no_fwd_only:
        # the forward on its own (summaries, selection, forward: no dO, so no
        # row sums for the backward either)
        fms = event_timed(lambda: buf.run_pass(dev["q"], dev["k"], dev["v"], None, bwd=False),
                          args.steps, 3)
        extras["fwd_only_ms_per_pass"] = round(fms, 4)
    if not args.no_diverse and args.mode == "planted":
        # the same pass on inputs whose query blocks pick different history
        # sets (less reuse of K/V tiles across blocks); throughput only
        log("[bench] diverse-selection inputs")
        dinp = make_inputs(shape, seed=0, mode="diverse")
        ddev = {k: torch.from_numpy(dinp[k]).cuda().to(dt)
                for k in ("q", "k", "v", "do") if dinp.get(k) is not None}
        for _ in range(args.warmup):
            buf.run_pass(ddev["q"], ddev["k"], ddev["v"], ddev.get("do"), bwd=bwd)
        dms, _ = timed_passes(buf, ddev, bwd, args.steps)
        extras["diverse"] = {"tokens_per_s": round(tokens / (dms / 1e3), 1),
                             "ms_per_step": round(dms, 4),
                             "data": "synthetic (one planted direction per query block)"}
        del ddev, dinp

    if not args.no_sequential and shape.dtype == "bf16":
        log("[bench] segment-by-segment form (hga_segment_step per segment)")
        extras["sequential_steps"] = sequential_bench(shape, dev, args.steps, 3)
    if not args.no_workloads and shape.name == "train_16k":
        extras["workloads"] = {}
        for wname in ("infer_131k", "batch4_32k"):
            extras["workloads"][wname] = workload_bench(wname, max(3, args.steps // 4), 2)
        if not args.no_dense_sdpa:
            log("[bench] HGA against dense attention at 2K and 131K")
            try:
                extras["dense_by_length"] = dense_by_length(
                    ms if bwd else None, extras.get("dense_sdpa_flash_ms"),
                    extras["workloads"]["infer_131k"]["ms_per_pass"])
            except Exception as ex:  # noqa: BLE001 -- a comparator, never the result
                extras["dense_by_length"] = {"error": str(ex)[:200]}
                torch.cuda.empty_cache()
    if not args.no_exact and bwd and shape.dtype == "bf16":
        log("[bench] exact-gradient pass")
        # three warm-up passes: the first passes over the freshly allocated
        # history sums and workspace run slower (0.2-0.3 ms per pass with one)
        extras["exact_gradient"] = exact_bench(shape, dev, max(5, args.steps // 4), 3)
    if not args.no_host_tier and bwd and shape.dtype == "bf16":
        log("[bench] host-RAM history tier pass")
        extras["host_tier"] = host_tier_bench(shape, dev, max(3, args.steps // 4), 2)
        if shape.name == "train_16k" and not args.no_tier_131k:
            log("[bench] host-RAM tier at 131K (forward)")
            extras["host_tier_131k"] = host_tier_131k_bench(3)
    if not args.no_decode:
        log("[bench] decode steps at 131K")
        del buf
        extras["decode_131k"] = decode_bench(args.decode_steps)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "single_pass_ms": per_pass,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": f"synthetic ({args.mode}-direction N(0,1), seed 0)",
        "config": {"workload": shape.name, "batch": shape.batch, "seq_len": shape.seq_len,
                   "seg_len": shape.seg_len, "hist_block": shape.hist_block,
                   "query_block": shape.query_block, "top_k": shape.top_k,
                   "n_q_heads": shape.n_q_heads, "n_kv_heads": shape.n_kv_heads,
                   "head_dim": shape.head_dim, "segments": shape.nseg,
                   "step": ("summarize + select + fwd" + (" + bwd" if bwd else "") +
                            " of all segments (hga_segment_pass: one launch per kernel)")},
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
            "traffic": measured_traffic(dominant, shape.name),
            "avg_launch_us": round(avg_launch_ms * 1e3, 2),
            "launches": dom_n,
            "algorithmic_flop_per_launch": per_launch_flop,
            "timing": (f"HIP start/stop events stamped by every kernel's own dispatches "
                       f"(hipExtLaunchKernel) on its launch stream over a loop of "
                       f"{args.steps} one-stream passes ({ms_prof:.4f} ms per pass with the "
                       f"stamps); kernels_ms_per_pass averages the same loop"),
        },
    }
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count,
                     "memory_gib": round(props.total_memory / 2**30, 1)}
    out.update(extras)
    if not args.no_peaks:
        log("[bench] measured peaks (bf16 GEMM, device copy)")
        mp = measured_peaks()
        if achieved:
            mp["dominant_frac_of_gemm"] = round(achieved / mp["bf16_gemm_tflops"], 4)
        out["measured_peaks"] = mp
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(inp, shape, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def measured_peaks(steps=20):
    """What the machine sustains, to read the fractions against beside the
    published peaks: a square bf16 GEMM through torch (hipBLASLt; plain 2-D
    mm on contiguous tensors) and a 1 GiB device-to-device copy (bytes read
    + written)."""
    import torch
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 / (e0.elapsed_time(e1) / steps * 1e-3) / 1e12
    del a, b, c
    src = torch.empty(1 << 30, device="cuda", dtype=torch.uint8)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / steps * 1e-3) / 1e9
    del src, dst
    return {"bf16_gemm_tflops": round(gemm_tflops, 1), "gemm": f"torch.mm bf16 {n}^3",
            "copy_gbs": round(copy_gbs, 1), "copy": "1 GiB device-to-device, read + written"}


def dense_by_length(hga_16k_ms, sdpa_16k_ms, hga_131k_fwd_ms):
    """HGA against dense causal attention (torch SDPA, flash backend) as the
    sequence grows: the 2K training workload (fwd + bwd, both timed here),
    the 16K headline (the figures above) and the 131K inference workload
    (forward only; the HGA figure is its pass, the dense one runs on
    N(0,1) tensors of the same shape, its cost not depending on the
    values)."""
    import torch
    import sparse_long_context_query_amd as hga
    from synth import WORKLOADS, make_inputs
    out = {}
    shape = WORKLOADS["qwen3_2k"]
    inp = make_inputs(shape, seed=0)
    dev = {k: torch.from_numpy(inp[k]).cuda().to(torch.bfloat16) for k in ("q", "k", "v", "do")}
    buf = buffers(hga.Config.from_shape(shape))
    h2 = event_timed(lambda: buf.run_pass(dev["q"], dev["k"], dev["v"], dev["do"]), 20, 5)
    d2 = dense_sdpa(dev, shape, True, h2)
    out["2k_fwd_bwd"] = {"hga_ms": round(h2, 4), "dense_sdpa_flash_ms": d2["dense_sdpa_flash_ms"],
                         "dense_over_hga": d2.get("speedup_vs_dense_sdpa")}
    del buf, dev
    if hga_16k_ms and sdpa_16k_ms:
        out["16k_fwd_bwd"] = {"hga_ms": round(hga_16k_ms, 4), "dense_sdpa_flash_ms": sdpa_16k_ms,
                              "dense_over_hga": round(sdpa_16k_ms / hga_16k_ms, 2)}
    shape = WORKLOADS["infer_131k"]
    gen = torch.Generator(device="cuda").manual_seed(0)
    qs = (shape.batch, shape.n_q_heads, shape.seq_len, shape.head_dim)
    ks = (shape.batch, shape.n_kv_heads, shape.seq_len, shape.head_dim)
    dev = {"q": torch.randn(qs, generator=gen, device="cuda").to(torch.bfloat16),
           "k": torch.randn(ks, generator=gen, device="cuda").to(torch.bfloat16),
           "v": torch.randn(ks, generator=gen, device="cuda").to(torch.bfloat16)}
    d131 = dense_sdpa(dev, shape, False, hga_131k_fwd_ms)
    out["131k_fwd"] = {"hga_ms": round(hga_131k_fwd_ms, 4),
                       "dense_sdpa_flash_ms": d131["dense_sdpa_flash_ms"],
                       "dense_over_hga": d131.get("speedup_vs_dense_sdpa")}
    if d131.get("dense_sdpa_error"):
        out["131k_fwd"]["dense_sdpa_error"] = d131["dense_sdpa_error"]
    del dev
    torch.cuda.empty_cache()
    return out


def dense_sdpa(dev, shape, bwd, hga_ms):
    """torch SDPA, flash backend only (errors instead of falling back to the
    math path), dense causal over the whole sequence at the same shape."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    G = shape.group
    try:
        q = dev["q"].detach().clone().requires_grad_(bwd)
        k = dev["k"].repeat_interleave(G, 1).contiguous().requires_grad_(bwd)
        v = dev["v"].repeat_interleave(G, 1).contiguous().requires_grad_(bwd)
        do = dev.get("do")

        def once():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
                if bwd:
                    o.backward(do)

        for _ in range(2):
            once()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(3):
            once()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / 3
        return {"dense_sdpa_flash_ms": round(ms, 3), "speedup_vs_dense_sdpa": round(ms / hga_ms, 2)}
    except Exception as ex:  # noqa: BLE001
        return {"dense_sdpa_flash_ms": None, "dense_sdpa_error": str(ex)[:200]}


if __name__ == "__main__":
    main()
