"""Temperature schedule for BCJR-QAT (host-side helper; no kernel work).

Training anneals T from an initial T0 down to a near-zero T_end, so that the soft codeword crystallises into the
hard Viterbi code (BCJR-QAT, arXiv 2605.10655: gist.science Technical Summary, "Annealing").  The pages' schedule
correction starts at T0 = 0.3 instead of 1.0, skipping the high-temperature phase whose gradient is too smeared to
guide the weights ("Schedule Correction (Skip-High-T)").  They do not give the shape of the decay; this helper uses
the plainest one for a quantity that spans decades, a geometric sequence, and T_end = 1e-4 by default (the lowest
temperature at which the float32 recursion is exercised here).
"""
from __future__ import annotations

import math

__all__ = ["temperature_schedule"]


def temperature_schedule(num_steps: int, T0: float = 0.3, T_end: float = 1e-4) -> list[float]:
    """Temperatures T_0 .. T_{num_steps-1} with T_i = T0 * (T_end / T0) ** (i / (num_steps - 1)).

    The first equals T0 and the last T_end; consecutive ratios are equal.  One step gives [T0].
    """
    if num_steps < 1:
        raise ValueError("num_steps must be >= 1")
    if not (math.isfinite(T0) and math.isfinite(T_end) and T0 > 0 and T_end > 0):
        raise ValueError("T0 and T_end must be finite and positive")
    if T_end > T0:
        raise ValueError("annealing lowers the temperature: need T_end <= T0")
    if num_steps == 1:
        return [float(T0)]
    r = math.log(T_end / T0)
    out = [T0 * math.exp(r * i / (num_steps - 1)) for i in range(num_steps)]
    out[-1] = float(T_end)
    return out
