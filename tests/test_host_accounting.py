"""Host-side accounting behind the benchmark's figures (CPU only).

- The algorithmic work that throughput and roofline fractions divide by
  (`sparse_long_context_query_amd.work`) against a count made key by key
  from the oracle's selections: every history block the oracle selects
  contributes all of its Bh tokens to every query of the query block, and
  each query sees the local tokens of its segment up to itself.
- The kernel-trace summary (warm launches, median, fraction of peak) and
  the HBM-counter summary (scaling by the calibration copy, per-launch
  bytes, the source hash that gates their use) on synthetic CSV files.
- The one-GPU guard of bench.py.
"""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import hga_oracle as orc  # noqa: E402
from sparse_long_context_query_amd import work  # noqa: E402
from synth import HGAShape, WORKLOADS, make_inputs  # noqa: E402


def shp(**kw):
    base = dict(name="t", batch=1, seq_len=256, seg_len=64, hist_block=16, query_block=16,
                top_k=3, n_q_heads=4, n_kv_heads=2, head_dim=16, dtype="f32")
    base.update(kw)
    return HGAShape(**base)


def counted_pairs(shape, seed=3):
    """(history pairs, local pairs) summed over query heads, counted from
    the oracle's selection of every segment."""
    inp = make_inputs(shape, seed=seed)
    G = shape.n_q_heads // shape.n_kv_heads
    L, Bq, Bh = shape.seg_len, shape.query_block, shape.hist_block
    hist = loc = 0
    for s in range(shape.seq_len // L):
        t0 = s * L
        sel = orc.select_segment(inp["q"], inp["k"], shape, s)
        for b in range(shape.batch):
            for g in range(shape.n_kv_heads):
                for j in range(L // Bq):
                    blocks = [x for x in sel[b, g, j] if x >= 0]
                    assert all(0 <= x < t0 // Bh for x in blocks)  # whole history blocks
                    for tau in range(t0 + j * Bq, t0 + (j + 1) * Bq):
                        hist += G * len(blocks) * Bh
                        loc += G * (tau - t0 + 1)
    return hist, loc


@pytest.mark.parametrize("shape", [
    shp(),                                                   # k reached from segment 1 on
    shp(top_k=1),
    shp(top_k=40),                                           # k covers all history
    shp(hist_block=32, query_block=16, top_k=2),             # Bh != Bq
    shp(batch=2, n_q_heads=2, n_kv_heads=2, seq_len=192),    # G = 1, B = 2
])
def test_pair_counts_match_the_oracle_selection(shape):
    h, l_ = work.pair_counts(shape)
    assert (h, l_) == counted_pairs(shape)
    # per segment and per group, as the CPU-baseline sample uses them
    ngroups = shape.batch * shape.n_kv_heads
    for s in range(shape.seq_len // shape.seg_len):
        hs, ls = work.pair_counts(shape, segments=[s], groups=1)
        hall, lall = work.pair_counts(shape, segments=[s])
        assert (hs * ngroups, ls * ngroups) == (hall, lall)


def test_flop_formulas():
    shape = shp()
    h, l_ = work.pair_counts(shape)
    D = shape.head_dim
    f = work.flops(shape)
    assert f["fwd"] == 4 * D * (h + l_)
    assert f["bwd_dq"] == 4 * D * (h + l_)
    assert f["bwd_dkdv"] == 4 * D * l_
    assert f["bwd"] == f["bwd_dq"] + f["bwd_dkdv"]


def test_flops_of_the_16k_workload():
    """The per-launch figures the benchmark and the profiles divide by."""
    f = work.flops(WORKLOADS["train_16k"])
    assert f["fwd"] == 635_789_377_536
    assert f["bwd_dq"] == 635_789_377_536
    assert f["bwd_dkdv"] == 137_573_171_200


def test_dense_causal_flops_count_every_causal_pair():
    shape = shp(seq_len=96, batch=2)
    S = shape.seq_len
    pairs = shape.batch * shape.n_q_heads * sum(tau + 1 for tau in range(S))
    f = work.dense_causal_flops(shape)
    assert f["fwd"] == 4 * shape.head_dim * pairs
    assert f["bwd"] == 8 * shape.head_dim * pairs


def write_csv(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


DQ_MANGLED = ("_ZN3hga12_GLOBAL__N_114dq_pass_kernelILi128EEEvPKDF16bS3_S3_PKfS3_S5_PKiPDF16b"
              "NS0_7BwdArgsE")


def test_short_kernel_names():
    assert bench.short_kernel_name(DQ_MANGLED) == "dq_pass_kernel<128>"
    assert bench.short_kernel_name(
        "_ZN3hga12_GLOBAL__N_112score_kernelIDF16bLi128ELi128EEEvPKT_PKfPfNS0_7SelGeomE"
    ) == "score_kernel<bf16,128,128>"
    assert bench.short_kernel_name(
        "hga::(anonymous namespace)::tier_plan_kernel(int const*, int*)") == "tier_plan_kernel"


def test_trace_summary_warm_median_and_fraction(tmp_path, capsys):
    # launches of 2000 (the cold first one), then 900, 1000, 1100 us
    rows, t = [], 0
    for us in (2000, 900, 1000, 1100):
        rows.append({"Kernel_Name": DQ_MANGLED, "Start_Timestamp": t,
                     "End_Timestamp": t + us * 1000})
        t += us * 1000 + 5000
    p = tmp_path / "trace.csv"
    write_csv(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary([str(p)], skip=1)
    line = [x for x in capsys.readouterr().out.splitlines() if x.startswith("| dq_pass_kernel")]
    cells = [c.strip() for c in line[0].strip("|").split("|")]
    assert cells[1] == "4" and cells[3] == "3"
    assert float(cells[4]) == 1000.0                      # warm median
    flop = work.flops(WORKLOADS["train_16k"])["bwd_dq"]
    assert float(cells[8]) == pytest.approx(flop / 1e-3 / 1e12 / 2500.0, abs=1e-4)


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the 256 MiB copy: FETCH_SIZE sees half of it, WRITE_SIZE all of it
    write_csv(tmp_path / "f.csv", fields, [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
         "Counter_Value": 131072.0},
        {"Kernel_Name": DQ_MANGLED, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
        {"Kernel_Name": DQ_MANGLED, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000.0}])
    write_csv(tmp_path / "w.csv", fields, [
        {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
         "Counter_Value": 262144.0},
        {"Kernel_Name": DQ_MANGLED, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0},
        {"Kernel_Name": DQ_MANGLED, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "train_16k")
    t = json.loads(out.read_text())
    k = t["kernels"]["bwd_dq"]
    assert k["dispatches"] == 2
    assert k["hbm_bytes_per_launch"] == (2000 * 2 + 500) * 1024
    # used while the sources are those it was taken on, for its workload only
    assert bench.measured_traffic("bwd_dq", "train_16k") == (2000 * 2 + 500) * 1024
    assert bench.measured_traffic("bwd_dq", "infer_131k") is None
    t["sources_sha256"] = "0" * 64
    out.write_text(json.dumps(t))
    assert bench.measured_traffic("bwd_dq", "train_16k") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
