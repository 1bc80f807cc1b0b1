"""CPU oracle for the MoE block-verify layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP product path never does.
"""
from .oracle import *  # noqa: F401,F403
