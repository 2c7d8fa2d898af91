"""Trajectory pins: anchors at multiples of the period, context rows frozen between anchors."""
import numpy as np

from oracle import attention as A
from oracle import schedule as Sch


def test_plan():
    assert Sch.plan(10, 4) == ["dense", "rows", "rows", "rows", "dense", "rows", "rows", "rows", "dense", "rows"]


def test_trajectory_rows_and_anchors():
    r = np.random.default_rng(0)
    B, H, N, T, d, k = 2, 2, 20, 6, 8, 7
    tv = (4, 4)
    per_step = [tuple(r.standard_normal(s) for s in [(B, H, N, d)] * 3 + [(B, H, T, d)] * 2) for _ in range(10)]
    warm = [(r.standard_normal((H, N, T)), np.full((H, N), 3.0)) for _ in range(2)]
    state0 = r.standard_normal((B, H, N, d))
    state, S, a, kinds = Sch.run(state0, warm, lambda t: per_step[t], k, 10, 4, tv, 0, 4)
    assert len(S) == k
    C = np.setdiff1d(np.arange(N), S)
    last_dense = A.attention(*per_step[8], tv)[0]
    last_rows = A.attention(*per_step[9], tv, rows=S)[0]
    assert np.array_equal(state[:, :, C], last_dense[:, :, C])
    assert np.max(np.abs(state[:, :, S] - last_rows)) < 1e-12
