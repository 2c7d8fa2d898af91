"""Prompt-conditioned sensitivity partition (PCSP): per-token scores and the S / C split.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the SAFE-DiT technical summary (gist.science, Korean and Italian pages), Methodology 2:
during a short warmup the attention weights from image tokens to text content tokens are
aggregated, and the image tokens are split into a sensitive set S and a context set C that stays
fixed for the rest of the trajectory.  Methodology 4 takes the sensitivity scores s_i from PCSP.

Readings taken where the pages are silent or ambiguous:
- the aggregated weight is the text-block mass of the joint softmax row: for head h and image row i,
  LSE = log(exp(lse_img) + sum_{t<Tv} exp(x_t)), a_i += sum_h sum_{t in [c0,c1)} exp(x_t - LSE);
  without lse_img the softmax is over the valid text slots only;
- scores add up over heads and over warmup steps (repeated calls with accumulation);
- S = the k largest scores, equal scores ordered by lower index, returned in ascending index order;
  NaN ranks below everything and -0 equals +0; C is the ascending complement;
- s_i is the min-max normalisation of the scores (0 everywhere when all scores are equal).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def scores(x: np.ndarray, lse_img: Optional[np.ndarray], tv: int, c0: int, c1: int) -> np.ndarray:
    """a [N] (fp64) from x [H,N,T] (only t < tv used) and lse_img [H,N] (or None)."""
    xv = np.asarray(x, dtype=np.float64)[:, :, :tv]
    if tv > 0:
        m = xv.max(axis=2)
        lse_txt = m + np.log(np.exp(xv - m[:, :, None]).sum(axis=2))
    else:
        lse_txt = np.full(xv.shape[:2], -np.inf)
    if lse_img is not None:
        lse = np.logaddexp(np.asarray(lse_img, dtype=np.float64), lse_txt)
    else:
        lse = lse_txt
    w = np.exp(xv[:, :, c0:c1] - lse[:, :, None])
    return w.sum(axis=2).sum(axis=0)


def accumulate(prev: Optional[np.ndarray], x, lse_img, tv, c0, c1) -> np.ndarray:
    a = scores(x, lse_img, tv, c0, c1)
    return a if prev is None else np.asarray(prev, dtype=np.float64) + a


def order(a: np.ndarray) -> np.ndarray:
    """Token indices by (score descending, index ascending), NaN last."""
    a = np.asarray(a, dtype=np.float64)
    nan = np.isnan(a)
    clean = np.where(nan, 0.0, a)
    return np.lexsort((np.arange(a.shape[0]), -clean, nan))


def partition(a: np.ndarray, k: int):
    """(S, C, is_sens, s01) for the k largest scores."""
    a = np.asarray(a, dtype=np.float64)
    N = a.shape[0]
    o = order(a)
    S = np.sort(o[:k]).astype(np.int32)
    C = np.sort(o[k:]).astype(np.int32)
    is_sens = np.zeros(N, dtype=np.uint8)
    is_sens[S] = 1
    return S, C, is_sens, normalise(a)


def normalise(a: np.ndarray) -> np.ndarray:
    """s_i = (a_i - min a) / (max a - min a), or 0 when max == min; NaN scores stay NaN."""
    a = np.asarray(a, dtype=np.float64)
    if np.all(np.isnan(a)):
        return np.full_like(a, np.nan)
    lo, hi = np.nanmin(a), np.nanmax(a)
    if hi > lo:
        with np.errstate(invalid="ignore"):
            return (a - lo) / (hi - lo)
    return np.where(np.isnan(a), np.nan, 0.0)
