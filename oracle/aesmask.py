"""AesMask: an affinity map from cross-attention to selected text tokens, and its percentile mask.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the AccelAes technical summary (Korean), gist.science, 2. Methodology B.1 AesMask: the attention
weights that a chosen set of aesthetic prompt tokens exchange with the image tokens are aggregated into
an affinity map, and a percentile threshold turns the map into a binary mask (1 = focus region), once
per generation and without training.  Choosing the tokens (CLIP similarity against a fixed anchor word
list) needs a text encoder and is an input here: a 0/1 vector over the text slots.

Readings taken where the pages are silent or ambiguous:
- the weight between image token i and text slot t is the entry of the joint softmax row of i (image
  keys and valid text keys together), the quantity the PCSP aggregation of the SAFE-DiT pages uses:
  LSE = log(exp(lse_img) + sum_{t<Tv} exp(x_t)), a_i = sum_h sum_{t<Tv, sel_t = 1} exp(x_t - LSE);
  without lse_img the softmax runs over the valid text slots only;
- the mask keeps the tokens at or above the p-th percentile of the affinities, counted as numpy's
  linearly interpolated percentile counts them for distinct scores: k = N - ceil(p (N - 1) / 100)
  tokens, with p given in hundredths of a percent (an integer, so k is exact); with equal scores the
  count is kept and the lower index wins, as in the PCSP partition.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import pcsp as _pcsp


def affinity(x: np.ndarray, lse_img: Optional[np.ndarray], tv: int, sel: np.ndarray) -> np.ndarray:
    """a [N] (fp64) from x [H,N,T] (slots t < tv used), lse_img [H,N] (or None) and sel [T] (0/1)."""
    xv = np.asarray(x, dtype=np.float64)[:, :, :tv]
    if tv > 0:
        m = xv.max(axis=2)
        lse_txt = m + np.log(np.exp(xv - m[:, :, None]).sum(axis=2))
    else:
        lse_txt = np.full(xv.shape[:2], -np.inf)
    lse = lse_txt if lse_img is None else np.logaddexp(np.asarray(lse_img, dtype=np.float64), lse_txt)
    keep = (np.asarray(sel)[:tv] != 0).astype(np.float64)
    return (np.exp(xv - lse[:, :, None]) * keep[None, None, :]).sum(axis=2).sum(axis=0)


def percentile_count(N: int, pct_bp: int) -> int:
    """Number of tokens kept at the p-th percentile, p = pct_bp / 100 (pct_bp in 0 .. 10000)."""
    if not 0 <= pct_bp <= 10000 or N < 0:
        raise ValueError("pct_bp must lie in [0, 10000] and N >= 0")
    if N == 0:
        return 0
    num = pct_bp * (N - 1)          # p (N - 1) / 100 = num / 10000
    return N - (-(-num // 10000))   # N - ceil(num / 10000)


def mask(a: np.ndarray, pct_bp: int):
    """(k, S, is_focus u8 [N]): the k = percentile_count tokens of largest affinity (ties: lower index)."""
    k = percentile_count(len(a), pct_bp)
    S, _, is_focus, _ = _pcsp.partition(a, k)
    return k, S, is_focus
