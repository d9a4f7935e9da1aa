"""CPU oracle for the MoE layer forward (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library or its binding.
"""
from .moe_oracle import *  # noqa: F401,F403
