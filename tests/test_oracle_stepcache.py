"""Pins of the StepCache oracle: the plan of full and extrapolated steps, exact on linear predictions,
the closed-form error on quadratic ones."""
import numpy as np
import pytest

from oracle import stepcache as SC


def test_plan_by_hand():
    third = 1.0 / 3.0
    want = [(True, -1, -1, 0.0), (False, 0, 0, 0.0), (False, 0, 0, 0.0),
            (True, -1, -1, 0.0), (False, 0, 3, third), (False, 0, 3, 2 * third),
            (True, -1, -1, 0.0), (False, 3, 6, third), (False, 3, 6, 2 * third),
            (True, -1, -1, 0.0)]
    got = SC.plan(10, 3)
    assert [g[:3] for g in got] == [w[:3] for w in want]
    assert np.allclose([g[3] for g in got], [w[3] for w in want], rtol=0, atol=1e-15)
    assert all(p[0] for p in SC.plan(7, 1))
    assert [p[0] for p in SC.plan(5, 9)] == [True, False, False, False, False]
    with pytest.raises(ValueError):
        SC.plan(4, 0)


@pytest.mark.parametrize("delta", [2, 3, 5])
def test_linear_predictions_are_reproduced(delta):
    r = np.random.default_rng(delta)
    c0, c1 = r.standard_normal((4, 6)), r.standard_normal((4, 6))
    steps = 4 * delta + 2
    out = SC.run(lambda s: c0 + c1 * s, steps, delta)
    for s in range(steps):
        want = c0 if s < delta else c0 + c1 * s  # one full prediction only before the second full step
        assert np.max(np.abs(out[s] - want)) < 1e-12


@pytest.mark.parametrize("delta", [2, 4])
def test_quadratic_error_closed_form(delta):
    """For eps_s = s^2 the line through the two last full steps misses by delta^2 w (w + 1)."""
    steps = 5 * delta
    out = SC.run(lambda s: np.array([float(s * s)]), steps, delta)
    for s, (full, a, b, w) in enumerate(SC.plan(steps, delta)):
        if full or s < delta:
            continue
        assert abs((s * s - out[s][0]) - delta * delta * w * (w + 1)) < 1e-9


def test_extrapolate_weight_zero_is_the_newer_prediction():
    r = np.random.default_rng(3)
    a, b = r.standard_normal(50), r.standard_normal(50)
    assert np.array_equal(SC.extrapolate(a, b, 0.0), b)
