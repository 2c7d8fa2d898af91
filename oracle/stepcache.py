"""StepCache: full model predictions every delta steps, linear extrapolation in between.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the AccelAes technical summary (Korean), gist.science, 2. Methodology B.3 StepCache: the whole
transformer runs only at a fixed step interval, and the steps between reuse the noise prediction by
linear extrapolation; the module does not depend on the model's architecture.

Readings taken where the pages are silent or ambiguous:
- the full steps are s = 0, delta, 2 delta, ...;
- a step s strictly between full steps j*delta and (j+1)*delta, j >= 1, takes the line through the last
  two full predictions, in step units: eps_s = eps_b + w (eps_b - eps_a) with a = (j-1) delta,
  b = j delta and w = (s - b) / delta;
- before the second full step (j = 0) there is one full prediction only, and it is reused (w = 0);
- delta = 1 makes every step full.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def plan(steps: int, delta: int) -> List[Tuple[bool, int, int, float]]:
    """Per step: (full, a, b, w).  Full steps carry (True, -1, -1, 0.0)."""
    if steps < 0 or delta < 1:
        raise ValueError("steps >= 0 and delta >= 1")
    out = []
    for s in range(steps):
        if s % delta == 0:
            out.append((True, -1, -1, 0.0))
            continue
        j = s // delta
        b = j * delta
        if j == 0:
            out.append((False, b, b, 0.0))
        else:
            out.append((False, b - delta, b, (s - b) / delta))
    return out


def extrapolate(eps_a: np.ndarray, eps_b: np.ndarray, w: float) -> np.ndarray:
    """eps_b + w (eps_b - eps_a) in fp64."""
    a = np.asarray(eps_a, dtype=np.float64)
    b = np.asarray(eps_b, dtype=np.float64)
    return b + float(w) * (b - a)


def run(full_prediction, steps: int, delta: int) -> List[np.ndarray]:
    """The predictions a StepCache trajectory uses: full_prediction(s) on full steps, extrapolations
    from the stored full predictions on the others."""
    done = {}
    out = []
    for s, (full, a, b, w) in enumerate(plan(steps, delta)):
        if full:
            done[s] = np.asarray(full_prediction(s), dtype=np.float64)
            out.append(done[s])
        else:
            out.append(extrapolate(done[a], done[b], w))
    return out
