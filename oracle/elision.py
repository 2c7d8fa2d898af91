"""Exact mask-elision criterion (which additive masks can be dropped without changing attention).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the SAFE-DiT technical summary (gist.science, Korean and Italian pages), Methodology 1 and
Key Contributions 2: an additive mask that only shifts each logit row by a constant c_i leaves the
normalised attention unchanged and may be removed; text padding, causal masks and non-uniform biases
are kept.

Reading taken where the pages are silent: the criterion is checked per mask slice and row, over the keys
the row actually attends to, i.e. the image block and the valid text slots of every batch entry that
uses the slice (padded slots are masked anyway).  Entries must be bitwise-equal under IEEE ==
(+0 == -0) to one finite constant; NaN or an infinity among them makes the row non-removable.  A
mask covering the image block only leaves an implicit 0 over the valid text slots, so then c_i must
be 0 unless no batch entry using the slice has valid text.  Bool masks read True as 0, False as -inf.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def row_values(mask: np.ndarray, N: int, T: int, tv: Sequence[int]) -> Tuple[list, list]:
    """The (mb, mh, i) rows of the mask restricted to their attended keys, as fp64 vectors."""
    mB, mH, Nq, Mc = mask.shape
    assert Nq == N and Mc in (N, N + T)
    B = len(tv)
    out, keys = [], []
    for mb in range(mB):
        users = list(range(B)) if mB == 1 else [mb]
        tmax = max(int(tv[b]) for b in users)
        for mh in range(mH):
            for i in range(Nq):
                row = mask[mb, mh, i]
                if row.dtype == np.bool_:
                    row = np.where(row, 0.0, -np.inf)
                row = row.astype(np.float64)
                if Mc == N:
                    vals = np.concatenate([row, np.zeros(tmax)])
                else:
                    vals = row[: N + tmax]
                out.append(vals)
                keys.append((mb, mh, i))
    return out, keys


def is_row_constant(mask: np.ndarray, N: int, T: int, tv: Sequence[int]):
    """(elidable, c) with c[mb*mH*N + mh*N + i] = the row constant, or NaN where the row is not constant."""
    rows, _ = row_values(mask, N, T, tv)
    c = np.empty(len(rows))
    ok = True
    for r, vals in enumerate(rows):
        first = vals[0]
        const = bool(np.isfinite(first)) and bool(np.all(vals == first))
        c[r] = first if const else np.nan
        ok = ok and const
    return ok, c
