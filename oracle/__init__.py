"""CPU oracle of the sparse MoE layer forward (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It is independent of the HIP library and must stay so.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
