"""CPU oracle for the MoE-layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
calls it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
