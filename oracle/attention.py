"""Plain fp64 attention over the joint image+text key set (dense anchor and sensitive-row forms).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

What it follows:
- SAFE-DiT technical summary (gist.science, Korean and Italian pages), Methodology 1: logits L of a
  row i may carry an additive mask; a row-wise constant shift L[i,:] + c_i cancels in the softmax
  normalisation, while semantic masks such as text padding are kept.
- Same pages, Methodology 3 (SRSU / CAR): in a non-anchor step only the query rows of the sensitive
  set S are updated, and they still attend to the global keys and values; an anchor step updates
  every token densely.
- AccelAes summary (gist.science, Korean page), Method B.2 SkipSparse: queries only for focus
  tokens, keys and values from the whole image.

Readings where the pages are silent: one joint softmax over the image keys
followed by the text keys; scale 1/sqrt(d); trailing text padding given per batch entry as a valid
length Tv[b], padded keys taking no part in the sum whatever they hold; a fully masked row gives a
zero output and a log-sum-exp of -inf.

Every quantity is computed in float64 from the values the device is given (bf16 inputs arrive here
already widened exactly), so a comparison measures the kernel's error, not input quantisation.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _mask_block(mask: Optional[np.ndarray], b: int, h: int, rows: np.ndarray, N: int, tv: int) -> Optional[np.ndarray]:
    """Additive fp64 mask for (b, h) over rows x [image N | valid text tv], or None.

    Bool entries map True -> 0 and False -> -inf.  A mask of N columns covers the image block only;
    its text block is 0.  A mask of N+T columns carries its own text block.
    """
    if mask is None:
        return None
    mb = 0 if mask.shape[0] == 1 else b
    mh = 0 if mask.shape[1] == 1 else h
    m = mask[mb, mh][rows]
    if m.dtype == np.bool_:
        m = np.where(m, 0.0, -np.inf)
    m = m.astype(np.float64)
    cols = m.shape[1]
    if cols == N:
        return np.concatenate([m, np.zeros((m.shape[0], tv))], axis=1)
    return m[:, : N + tv]


def attention(q: np.ndarray, k_img: np.ndarray, v_img: np.ndarray, k_txt: np.ndarray, v_txt: np.ndarray,
              tv: Sequence[int], rows: Optional[np.ndarray] = None, scale: Optional[float] = None,
              mask: Optional[np.ndarray] = None, row_block: int = 2048, want_emission: bool = False):
    """Joint-softmax attention for the image query rows `rows` (all N rows if None).

    q, k_img, v_img: [B,H,N,d]; k_txt, v_txt: [B,H,T,d]; tv: valid text length per batch entry.
    Returns (o [B,H,R,d], lse [B,H,R]) in float64, R = len(rows).  With want_emission it also returns
    x [H,R,tv[0]] (the text-block logits of batch entry 0, mask included) and lse_img [H,R] (the
    log-sum-exp of that entry's image-block logits), the per-token cross-attention responses a
    warmup step hands to the sensitivity partition.
    """
    B, H, N, d = q.shape
    if scale is None or scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.zeros((B, H, R, d))
    lse = np.full((B, H, R), -np.inf)
    x_out = np.zeros((H, R, tv[0])) if want_emission else None
    lse_img_out = np.full((H, R), -np.inf) if want_emission else None
    for b in range(B):
        t = int(tv[b])
        for h in range(H):
            keys = np.concatenate([k_img[b, h], k_txt[b, h, :t]]).astype(np.float64)
            vals = np.concatenate([v_img[b, h], v_txt[b, h, :t]]).astype(np.float64)
            for r0 in range(0, R, row_block):
                rr = rows[r0:r0 + row_block]
                L = scale * (q[b, h, rr].astype(np.float64) @ keys.T)
                m = _mask_block(mask, b, h, rr, N, t)
                if m is not None:
                    L = L + m
                mx = L.max(axis=1, keepdims=True)
                finite = np.isfinite(mx)
                safe = np.where(finite, mx, 0.0)
                p = np.exp(L - safe)
                s = p.sum(axis=1, keepdims=True)
                live = (s[:, 0] > 0) & finite[:, 0]
                o[b, h, r0:r0 + len(rr)] = np.where(live[:, None], (p @ vals) / np.where(s > 0, s, 1.0), 0.0)
                with np.errstate(divide="ignore"):
                    lse[b, h, r0:r0 + len(rr)] = np.where(live, safe[:, 0] + np.log(np.where(s[:, 0] > 0, s[:, 0], 1.0)), -np.inf)
                if want_emission and b == 0:
                    x_out[h, r0:r0 + len(rr)] = L[:, N:N + t]
                    li = L[:, :N]
                    mi = li.max(axis=1, keepdims=True)
                    fin = np.isfinite(mi)
                    si = np.exp(li - np.where(fin, mi, 0.0)).sum(axis=1)
                    with np.errstate(divide="ignore"):
                        lse_img_out[h, r0:r0 + len(rr)] = np.where(fin[:, 0] & (si > 0), mi[:, 0] + np.log(np.where(si > 0, si, 1.0)), -np.inf)
    if want_emission:
        return o, lse, x_out, lse_img_out
    return o, lse


def dense_step(state: np.ndarray, *args, **kw) -> np.ndarray:
    """Anchor step: every image token's row of the cached state is recomputed."""
    o, _ = attention(*args, rows=None, **kw)
    return o


def rows_step(state: np.ndarray, rows: np.ndarray, *args, **kw) -> np.ndarray:
    """Sensitive-row step: rows S are recomputed against the global keys; every other row keeps its value."""
    out = np.array(state, dtype=np.float64, copy=True)
    if len(rows) == 0:
        return out
    o, _ = attention(*args, rows=rows, **kw)
    out[:, :, np.asarray(rows, dtype=np.int64)] = o
    return out


def gather_rows(state: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """packed[b,h,r,:] = state[b,h,rows[r],:]."""
    return np.asarray(state)[:, :, np.asarray(rows, dtype=np.int64)]


def scatter_rows(state: np.ndarray, packed: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """state[b,h,rows[r],:] = packed[b,h,r,:]; other rows unchanged."""
    out = np.array(state, copy=True)
    out[:, :, np.asarray(rows, dtype=np.int64)] = packed
    return out
