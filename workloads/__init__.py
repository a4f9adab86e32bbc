"""Seeded synthetic workloads for the FASA decode path.

This package only draws inputs: random numbers, sampled dominant-FC sets,
planted salient positions and dtype rounding of what it draws.  It holds none
of the method's arithmetic (no TIP, no selection, no attention), and both the
HIP path's tests/benchmark and the oracle receive its arrays unchanged.
"""

from .configs import Workload, CONFIGS, get, shrink  # noqa: F401
from .generate import generate, to_bf16_bits, round_bf16, random_scores, head_budgets  # noqa: F401
