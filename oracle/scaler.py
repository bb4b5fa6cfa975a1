"""Oracle of the dynamic loss-scale policy around the step (test infrastructure).

The pages show the GradScaler calls only -- scale the loss, step (skipped when
a gradient overflows), update ("PaddlePaddle ZeRO优化…", section
"工程落地中的真实权衡", item "混合精度才是最佳拍档").  The update rule is a
reading: after an overflow the scale is multiplied by backoff_factor and the
count of clean steps restarts; after growth_interval clean steps in a row it is
multiplied by growth_factor, unless that product is not finite.  The scale is
an fp32 value and every product is one fp32 rounding.
"""
from __future__ import annotations

import dataclasses

import numpy as np

F32 = np.float32


@dataclasses.dataclass
class ScalerState:
    scale: np.float32
    growth_tracker: int          # clean steps since the scale last changed
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    growth_interval: int = 2000


def update(s: ScalerState, overflow: bool) -> ScalerState:
    """One update after a step whose gradients did (overflow) or did not overflow."""
    if overflow:
        return dataclasses.replace(s, scale=F32(s.scale * F32(s.backoff_factor)), growth_tracker=0)
    n = s.growth_tracker + 1
    if n == s.growth_interval:
        with np.errstate(over="ignore"):            # growth past the fp32 range is data here
            grown = F32(s.scale * F32(s.growth_factor))
        return dataclasses.replace(s, scale=grown if np.isfinite(grown) else s.scale, growth_tracker=0)
    return dataclasses.replace(s, growth_tracker=n)


def inv_scale(s: ScalerState) -> np.float32:
    """fp32(1 / scale): what the step multiplies the averaged gradient by (IEEE
    division: a scale that has underflowed to 0 gives +inf)."""
    with np.errstate(divide="ignore", over="ignore"):
        return F32(np.float64(1.0) / np.float64(s.scale))
