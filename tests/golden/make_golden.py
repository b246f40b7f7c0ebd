"""Writes tests/golden/tiny_hga.json: a tiny HGA case whose inputs come from
the seeded generator and whose expected outputs come from the fp64 oracle
(and nothing else).  Re-run only when a change to the oracle's arithmetic is
justified by a reading of the pages, and say which in the commit message.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import hga_oracle  # noqa: E402
from synth import HGAShape, make_inputs  # noqa: E402

SHAPE = HGAShape("golden_tiny", 1, 48, 4, 2, 4, 16, 8, 8, 2, "f32")
SEED = 7


def _f32_list(a):
    import numpy as np
    flat = [float(np.format_float_positional(x, unique=True)) for x in a.ravel()]
    return {"shape": list(a.shape), "data": flat}


def main():
    inp = make_inputs(SHAPE, seed=SEED)
    out = hga_oracle.run(inp)
    doc = {
        "about": "Tiny HGA case: inputs from synth.make_inputs, outputs from "
                 "the fp64 oracle (oracle/hga_oracle.py run()).",
        "shape": {k: getattr(SHAPE, k) for k in (
            "batch", "seq_len", "n_q_heads", "n_kv_heads", "head_dim",
            "seg_len", "hist_block", "query_block", "top_k", "dtype")},
        "seed": SEED,
        # float32 inputs in their shortest round-tripping decimal form
        "inputs": {k: _f32_list(inp[k]) for k in ("q", "k", "v", "do")},
        "outputs": {k: out[k].tolist() for k in ("sel", "o", "lse", "dq", "dk", "dv", "kbar")},
    }
    with open(os.path.join(HERE, "tiny_hga.json"), "w") as f:
        json.dump(doc, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
