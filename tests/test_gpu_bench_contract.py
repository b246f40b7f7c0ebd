"""The benchmark's output line (GPU): a short run of bench.py with the
optional legs off prints one JSON line carrying the fields a reader of it
relies on -- the metric and its unit, whole-job throughput consistent with
ms_per_step, the roofline object of the dominant kernel (its algorithmic
rate against the published bf16 peak) and the CPU-oracle baseline."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

LEGS_OFF = ["--no-dense-self", "--no-dense-sdpa", "--no-decode", "--no-diverse",
            "--no-host-tier", "--no-hbm", "--no-sequential", "--no-workloads", "--no-exact",
            "--no-tier-131k", "--no-peaks", "--no-fwd-only"]


def test_bench_prints_one_contract_line():
    print("case: bench.py --steps 3 --warmup 1 --cpu-seconds 1, optional legs off", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--cpu-seconds", "1"] + LEGS_OFF,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and d["config"]["workload"] == "train_16k"
    assert d["device"]["compute_units"] > 0 and "gfx950" in d["device"]["arch"]
    # whole-job throughput: the 16,384 tokens of one pass over its time
    assert d["value"] == pytest.approx(16384 / (d["ms_per_step"] * 1e-3), rel=1e-3)
    sp = d["single_pass_ms"]
    assert sp["passes"] == 3 and sp["min_ms"] <= sp["median_ms"] <= sp["max_ms"]
    assert sp["median_ms"] == pytest.approx(d["ms_per_step"], rel=0.25)
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["achieved"] < rf["peak"]
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-3)
    # achieved = algorithmic FLOP per launch / average launch time
    assert rf["achieved"] == pytest.approx(
        rf["algorithmic_flop_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e12, rel=2e-3)
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
