"""CPU oracle for the ZeRO-sharded Adam step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path never does. It shares no code with
the HIP path.
"""
from .oracle import (Oracle, MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16,  # noqa: F401
                     MIXED_MODES)
