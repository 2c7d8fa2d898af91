"""Closed-form pins of the SW-CFG oracle."""
import json
import os

import numpy as np
import pytest

from oracle import swcfg as G

HERE = os.path.dirname(os.path.abspath(__file__))


def _eps(C=3, Hl=8, Wl=12, seed=0):
    return np.random.default_rng(seed).standard_normal((2, C, Hl, Wl))


def test_equal_scales_is_global_cfg():
    e = _eps()
    s = np.random.default_rng(1).random(16)
    out = G.combine(e, s, 4, 4.5, 4.5)
    assert np.max(np.abs(out - (e[1] + 4.5 * (e[0] - e[1])))) < 1e-12


@pytest.mark.parametrize("sval,g", [(0.0, 2.0), (1.0, 7.0)])
def test_constant_sensitivity(sval, g):
    e = _eps(seed=2)
    out = G.combine(e, np.full(16, sval), 4, 2.0, 7.0)
    assert np.max(np.abs(out - (e[1] + g * (e[0] - e[1])))) < 1e-12


def test_unit_and_zero_scale_pick_a_branch():
    e = _eps(seed=3)
    s = np.random.default_rng(4).random(16)
    assert np.max(np.abs(G.combine(e, s, 4, 1.0, 1.0) - e[0])) < 1e-15 * 8
    assert np.array_equal(G.combine(e, s, 4, 0.0, 0.0), e[1])


def test_affine_in_s():
    e = _eps(seed=5)
    r = np.random.default_rng(6)
    s1, s2 = r.random(16), r.random(16)
    lhs = G.combine(e, s1, 4, 3.0, 6.0) + G.combine(e, s2, 4, 3.0, 6.0)
    rhs = 2 * G.combine(e, (s1 + s2) / 2, 4, 3.0, 6.0)
    assert np.max(np.abs(lhs - rhs)) < 1e-12


def test_token_map_by_pixel_loop():
    Hl, Wl, side = 8, 12, 4
    tm = G.token_map(Hl, Wl, side)
    for y in range(Hl):
        for x in range(Wl):
            assert tm[y, x] == (y // 2) * 4 + (x // 3)


def test_golden_hand_examples():
    with open(os.path.join(HERE, "golden", "swcfg_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        eps = np.array(c["eps"], dtype=np.float64)
        out = G.combine(eps, np.array(c["s"]), c["side"], c["g_ctx"], c["g_sens"])
        assert np.max(np.abs(out - np.array(c["out"]))) < 1e-12, c["why"]
