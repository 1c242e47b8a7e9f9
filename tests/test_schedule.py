"""The annealing schedule helper (host only): T0 -> T_end, geometric, skip-high-T default T0 = 0.3
(gist.science Technical Summary, "Annealing" and "Schedule Correction (Skip-High-T)")."""
import math

import pytest

from differentiable_bcjr_amd import temperature_schedule


def test_endpoints_and_default_start():
    Ts = temperature_schedule(300)
    assert len(Ts) == 300
    assert Ts[0] == 0.3 and Ts[-1] == 1e-4


def test_geometric_and_decreasing():
    Ts = temperature_schedule(50, T0=1.0, T_end=1e-3)
    ratios = [b / a for a, b in zip(Ts, Ts[1:])]
    assert all(r < 1 for r in ratios)
    assert max(ratios) - min(ratios) < 1e-12
    assert math.isclose(ratios[0] ** 49, 1e-3, rel_tol=1e-12)


def test_single_step_and_constant():
    assert temperature_schedule(1, T0=0.2) == [0.2]
    assert temperature_schedule(4, T0=0.5, T_end=0.5) == [0.5] * 4


@pytest.mark.parametrize("kw", [dict(num_steps=0), dict(num_steps=5, T0=0.0), dict(num_steps=5, T_end=-1.0),
                                dict(num_steps=5, T0=float("nan")), dict(num_steps=5, T0=0.1, T_end=0.2)])
def test_rejects_bad_arguments(kw):
    with pytest.raises(ValueError):
        temperature_schedule(**kw)
