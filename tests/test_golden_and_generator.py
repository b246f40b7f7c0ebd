"""Generator properties and the stored tiny oracle fixture."""

import json
import os

import numpy as np
import pytest

from oracle import hga_oracle as orc
from synth import WORKLOADS, HGAShape, make_inputs, round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_hga.json")


def load_golden():
    with open(GOLDEN) as f:
        doc = json.load(f)
    shp = HGAShape(name="golden_tiny", **doc["shape"])
    inputs = {k: np.array(v["data"], dtype=np.float32).reshape(v["shape"])
              for k, v in doc["inputs"].items()}
    outputs = {k: np.array(v) for k, v in doc["outputs"].items()}
    return shp, doc["seed"], inputs, outputs


def test_generator_reproduces_golden_inputs():
    shp, seed, inputs, _ = load_golden()
    inp = make_inputs(shp, seed=seed)
    for k in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(inp[k], inputs[k])


def test_oracle_reproduces_golden_outputs():
    shp, _, inputs, outputs = load_golden()
    out = orc.run(dict(inputs, shape=shp))
    np.testing.assert_array_equal(out["sel"], outputs["sel"].astype(np.int32))
    for k in ("o", "lse", "dq", "dk", "dv", "kbar"):
        np.testing.assert_allclose(out[k], outputs[k], rtol=0, atol=1e-13, err_msg=k)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5e-3,
                  3.3895314e38], dtype=np.float32)
    import torch
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(x.copy()), want)
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000).astype(np.float32) * 100
    want = torch.tensor(y).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(y.copy()), want)


def test_generator_deterministic_and_streams_independent():
    shp = WORKLOADS["tiny_f32"]
    a = make_inputs(shp, seed=0)
    b = make_inputs(shp, seed=0, with_do=False)
    for k in ("q", "k", "v"):
        np.testing.assert_array_equal(a[k], b[k])
    c = make_inputs(shp, seed=1)
    assert not np.array_equal(a["q"], c["q"])


def test_generator_planting_counts():
    shp = WORKLOADS["qwen3_2k"]
    inp = make_inputs(shp, seed=0, with_do=False)
    pl = inp["planted"][0]
    assert len(pl) == shp.nseg and len(pl[0]) == 0
    for s in range(1, shp.nseg):
        assert len(pl[s]) == min(shp.top_k, shp.n_hist_blocks(s))
        assert np.all(np.diff(pl[s]) > 0)
    assert inp["q"].dtype == np.float32
    # bf16 workloads hold bf16-representable values
    bits = inp["q"].view(np.uint32)
    assert not np.any(bits & 0xFFFF)


def test_batched_workload_uses_independent_sequences():
    shp = WORKLOADS["batch4_32k"].replace(seq_len=4096, seg_len=1024, batch=2)
    a = make_inputs(shp, seed=0, with_do=False)
    one = make_inputs(shp.replace(batch=1), seed=1, with_do=False)
    np.testing.assert_array_equal(a["q"][1], one["q"][0])
    assert [list(x) for x in a["planted"][1]] == [list(x) for x in one["planted"][0]]


def test_diverse_mode_plants_per_query_block():
    shp = WORKLOADS["qwen3_2k"].replace(seq_len=2048, seg_len=256)
    inp = make_inputs(shp, seed=0, mode="diverse", with_do=False)
    s = shp.nseg - 1
    assert shp.n_hist_blocks(s) > shp.top_k
    sel = orc.select_segment(inp["q"], inp["k"], shp, s)
    # query blocks of one segment do not all share one set in this mode
    rows = {tuple(sel[0, 0, j]) for j in range(shp.n_qblocks)}
    assert len(rows) > 1
