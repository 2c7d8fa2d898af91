"""Trajectory schedule: warmup aggregation, one fixed partition, then anchor and sensitive-row steps.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the SAFE-DiT technical summary (gist.science, Korean and Italian pages), Methodology 2
(scores aggregated over a short warmup, partition then fixed for the trajectory) and Methodology 3
(sensitive-row updates in non-anchor steps, a dense refresh in periodic anchor steps).

Reading taken where the pages are silent: the warmup steps precede the scheduled steps; step t is an anchor
when t % anchor_every == 0, a sensitive-row step otherwise (anchors at 0, 4, 8 of 10 steps).
"""
from __future__ import annotations

from typing import Callable, List

import numpy as np

from . import attention as _attn
from . import pcsp as _pcsp


def plan(steps: int, anchor_every: int) -> List[str]:
    return ["dense" if t % anchor_every == 0 else "rows" for t in range(steps)]


def run(state0: np.ndarray, warmup: List[tuple], step_inputs: Callable[[int], tuple], k: int, steps: int,
        anchor_every: int, tv, c0: int, c1: int):
    """Returns (final state fp64, S, scores, kinds).

    warmup: list of (x [H,N,T], lse_img [H,N]) per warmup step.
    step_inputs(t) -> (q, k_img, v_img, k_txt, v_txt) of step t.
    """
    a = None
    for x, lse_img in warmup:
        a = _pcsp.accumulate(a, x, lse_img, tv[0], c0, c1)
    S, C, _, _ = _pcsp.partition(a, k)
    state = np.asarray(state0, dtype=np.float64)
    kinds = plan(steps, anchor_every)
    for t, kind in enumerate(kinds):
        args = step_inputs(t)
        if kind == "dense":
            state = _attn.dense_step(state, *args, tv=tv)
        else:
            state = _attn.rows_step(state, S, *args, tv=tv)
    return state, S, a, kinds
