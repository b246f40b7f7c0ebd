"""Seeded synthetic inputs for the HGA hot path (shared by the oracle tests,
the GPU tests, the smoke check and the benchmark).

This package holds no arithmetic of the attention method itself: it only
draws random tensors, plants directions and rounds values to the storage
dtype.  The method's arithmetic lives in ``oracle/`` (CPU, fp64) and in the
HIP library (GPU); the two never import each other.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    HGAShape,
    make_inputs,
    round_to_bf16,
    shape_by_name,
)
