"""CPU oracle of the per-rank ZeRO-1/2 mixed-precision shard step.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  Plain numpy, one IEEE fp32 operation per
array expression, no code shared with the HIP library.
"""
from . import accounting, flatten, loss_scale, ring, zero_step  # noqa: F401
