"""CPU oracle for block-scaled FP4 quantization and FP4 attention.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it; the GPU library never does.  See fp4_oracle.c for
the definitions it implements and the readings of the source pages.
"""
from .oracle import *  # noqa: F401,F403
