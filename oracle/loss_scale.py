"""CPU oracle of the dynamic loss-scale state machine.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; it shares no code with the HIP library.

The pages name loss scaling only as the "scale" step of the ZeRO-1 update
(ZeRO notes, rkmt.cn/news/44736, section "Deepspeed ZeRO-1", step 更新) and say
nothing of how the scale moves.  Reading taken: on a step whose unscaled
gradient holds inf/NaN the update is skipped, the scale is multiplied by the
backoff factor (0.5) down to a floor, and the run of clean steps restarts;
after ``growth_interval`` clean steps in a row the scale is multiplied by the
growth factor (2) up to a ceiling.  The scale is an fp32 value.

Pins: the halving on overflow and the untouched state are fixed by the
overflow workload.  The growth rule and the restart of the clean run are
checked against torch's GradScaler on forced sequences; that is a library
with the same reading, not the pages, so growth stays a reading.  The floor
and ceiling are parity unpinned beyond the closed form of this state machine
on forced flag sequences.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = np.float32


@dataclasses.dataclass
class ScalerState:
    scale: float = 65536.0
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    min_scale: float = 1.0
    max_scale: float = float(2 ** 24)
    growth_interval: int = 1000
    good_steps: int = 0
    skipped_steps: int = 0


def update_loss_scale(s: ScalerState, overflow: bool) -> bool:
    """Advance ``s`` in place after a step's flag is known; return skip."""
    if overflow:
        s.scale = float(max(F32(s.scale) * F32(s.backoff_factor), F32(s.min_scale)))
        s.good_steps = 0
        s.skipped_steps += 1
        return True
    s.good_steps += 1
    if s.good_steps >= s.growth_interval:
        s.scale = float(min(F32(s.scale) * F32(s.growth_factor), F32(s.max_scale)))
        s.good_steps = 0
    return False
