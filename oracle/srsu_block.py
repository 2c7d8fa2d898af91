"""The rest of a sensitive-row update: QKV projection and FFN on the gathered S token rows, with the FFN
output of the context rows cached.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the SAFE-DiT technical summary (gist.science), Methodology 3 (in a non-anchor step only the
sensitive rows S are recomputed; the context rows keep cached values) and the AccelAes technical
summary, 2. Methodology B.2 SkipSparse (queries of the focus tokens only, keys and values global; the
FFN of background tokens skipped and its most recent cached output reused).

Readings taken where the pages are silent or ambiguous:
- hidden states are token-major [B, N, D] with D = H * d; a linear layer stores its weight as
  [out_features, in_features] and computes y = x W^T + b;
- the FFN is Linear(D -> F) -> GELU (tanh form) -> Linear(F -> D), the DiT block's FFN; its output for
  the rows of S replaces those rows of the cache, the other rows stay as they are;
- the QKV projection of the rows of S writes those rows of the head-major Q, K and V tensors
  [B, H, N, d] (feature j of the projection: tensor j // D, head (j % D) // d, channel j % d); K and V of
  the context rows stay cached.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    return y if b is None else y + np.asarray(b, dtype=np.float64)


def rows_ffn(x: np.ndarray, rows: np.ndarray, w1, b1, w2, b2, cache: np.ndarray) -> np.ndarray:
    """cache [B,N,D] with rows S replaced by FFN(x[:, S])."""
    out = np.array(cache, dtype=np.float64)
    xs = np.asarray(x, dtype=np.float64)[:, rows, :]
    out[:, rows, :] = linear(gelu_tanh(linear(xs, w1, b1)), w2, b2)
    return out


def rows_qkv(x: np.ndarray, rows: np.ndarray, wqkv, bqkv, q, k, v, H: int, d: int):
    """(q, k, v) [B,H,N,d] with rows S replaced by the projection of x[:, S]."""
    B, N, D = x.shape
    y = linear(np.asarray(x, dtype=np.float64)[:, rows, :], wqkv, bqkv)  # [B, k, 3D]
    outs = []
    for which, t in enumerate((q, k, v)):
        o = np.array(t, dtype=np.float64)
        part = y[:, :, which * D:(which + 1) * D].reshape(B, len(rows), H, d).transpose(0, 2, 1, 3)
        o[:, :, rows, :] = part
        outs.append(o)
    return tuple(outs)
