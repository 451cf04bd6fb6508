"""CPU oracle for the dots3-note preview MoE layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package. The
GPU library never calls it and shares no code with it.

See ``oracle.moe`` for what each function computes and which passage of the
pages it follows.
"""
from .moe import *  # noqa: F401,F403
