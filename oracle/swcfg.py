"""Sensitivity-weighted classifier-free guidance (SW-CFG) on the model's prediction.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline leg use this.

Follows the SAFE-DiT technical summary (gist.science, Korean and Italian pages), Methodology 4: the
guidance scale is set per token, gamma_i = gamma_ctx + (gamma_sens - gamma_ctx) * s_i, and is applied
to the prediction after the forward pass.  The AccelAes summary (Method B.2, spatial CFG) is the
binary-s special case.

Readings taken where the pages are silent or ambiguous: the guided prediction is eps_u + gamma_i (eps_c - eps_u) with
eps[0] the conditional and eps[1] the unconditional prediction; a latent pixel (y, x) belongs to the
token (y // ph) * side + x // pw of the side x side grid, ph = Hl / side, pw = Wl / side.
"""
from __future__ import annotations

import numpy as np


def gamma(s: np.ndarray, g_ctx: float, g_sens: float) -> np.ndarray:
    return g_ctx + (g_sens - g_ctx) * np.asarray(s, dtype=np.float64)


def token_map(Hl: int, Wl: int, side: int) -> np.ndarray:
    ph, pw = Hl // side, Wl // side
    yy, xx = np.meshgrid(np.arange(Hl), np.arange(Wl), indexing="ij")
    return (yy // ph) * side + xx // pw


def combine(eps: np.ndarray, s: np.ndarray, side: int, g_ctx: float, g_sens: float) -> np.ndarray:
    """out [C,Hl,Wl] (fp64) from eps [2,C,Hl,Wl] and per-token s [side*side]."""
    eps = np.asarray(eps, dtype=np.float64)
    _, C, Hl, Wl = eps.shape
    g = gamma(s, g_ctx, g_sens)[token_map(Hl, Wl, side)]
    ec, eu = eps[0], eps[1]
    return eu + g[None] * (ec - eu)
