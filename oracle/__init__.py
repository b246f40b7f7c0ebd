"""CPU fp64 oracle of the HGA hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the benchmark's CPU-baseline leg, never by the library or its binding.
Holds no C code: nothing here needs compiling.
"""

from . import hga_loop, hga_oracle  # noqa: F401
