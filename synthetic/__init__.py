"""Seeded synthetic inputs shared by the oracle-side tests, the GPU parity tests and the benchmark.

This module holds input recipes only: random draws, bf16 rounding of the draws, the Gaussian-blob
bias placed on the synthetic image-to-text logits and the constant image-block log-sum-exp that
stands in for a real backbone.  It contains none of the method's arithmetic (no softmax, no
aggregation, no selection, no guidance) and imports nothing from the oracle or the HIP package.

Workloads follow the DiT shapes of the SAFE-DiT summary pages (1024^2, 2560^2 and 3072^2 latents
with 2x2 patches, 24 heads of width 64, a cond/uncond pair and a padded 256-slot text sequence).
No backbone weights, prompts or datasets are involved: every tensor is drawn from a seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

# One independent stream per tensor role, spawned from the workload seed.
_STREAMS = {
    "q": 0, "k_img": 1, "v_img": 2, "k_txt": 3, "v_txt": 4,
    "x": 5, "blobs": 6, "eps": 7, "mask": 8, "state": 9, "scores": 10, "aes_sel": 11, "stepcache": 12,
    "hidden": 13, "w_ffn1": 14, "w_ffn2": 15, "w_qkv": 16, "cache": 17,
}


def rng_for(seed: int, role: str, step: int = 0) -> np.random.Generator:
    """PCG64 stream for (seed, role, step); independent across roles and steps."""
    ss = np.random.SeedSequence([int(seed), int(step)])
    child = ss.spawn(len(_STREAMS))[_STREAMS[role]]
    return np.random.Generator(np.random.PCG64(child))


# ----------------------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # non-NaN patterns are at most 0xFF800000, so adding up to 0x8000 cannot wrap in uint32
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values that are exactly representable in bf16 (RNE of x)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": storage type of Q/K/V/state
    B: int
    H: int
    N: int
    side: int             # N = side * side, row-major token grid
    T: int
    tv: tuple             # valid text length per batch entry (trailing padding)
    d: int
    k: int                # |S|
    seed: int
    std: float            # Q/K/V ~ N(0,1) * std
    n_blobs: int = 0      # Gaussian blobs on the synthetic image->text logits
    blob_amp: float = 2.0
    blob_sigma: float = 8.0
    latent: Optional[tuple] = None   # (C, Hl, Wl) of the guidance latent
    g_ctx: float = 1.0
    g_sens: float = 1.0
    warmup_steps: int = 1
    steps: int = 1
    anchor_every: int = 4

    @property
    def flops_dense(self) -> float:
        """Algorithmic attention flops of one dense pass: 4*rows*(N+Tv)*d per (b,h)."""
        return float(sum(4.0 * self.H * self.N * (self.N + t) * self.d for t in self.tv))

    @property
    def flops_rows(self) -> float:
        return float(sum(4.0 * self.H * self.k * (self.N + t) * self.d for t in self.tv))


def _tv(B: int, v: int) -> tuple:
    return tuple([v] * B)


WORKLOADS: Dict[str, Workload] = {
    # 16x16 grid, fp32, 2 heads, text 32 slots with 20 valid; |S| = 64.
    "tiny_srsu_f32": Workload("tiny_srsu_f32", "f32", 1, 2, 256, 16, 32, _tv(1, 20), 64, 64, 1, 0.125),
    # 1024^2 latent, 64x64 tokens, dense anchor step.
    "dense_1024": Workload("dense_1024", "bf16", 2, 24, 4096, 64, 256, _tv(2, 77), 64, 1229, 2, 0.125),
    # 1024^2 SRSU step with PCSP blobs and SW-CFG on a 2x16x128x128 latent.
    "srsu_1024": Workload("srsu_1024", "bf16", 2, 24, 4096, 64, 256, _tv(2, 77), 64, 1229, 3, 0.125,
                          n_blobs=3, latent=(16, 128, 128), g_ctx=3.0, g_sens=6.0),
    # 2560^2 latent, 160x160 tokens, |S| = 20%.
    "srsu_2560": Workload("srsu_2560", "bf16", 2, 24, 25600, 160, 256, _tv(2, 120), 64, 5120, 4, 0.125,
                          n_blobs=5),
    # 1024^2 latent at head dim 128 (24 heads x 128, the width of the d = 128 DiT backbones), dense anchor step.
    "dense_1024_d128": Workload("dense_1024_d128", "bf16", 2, 24, 4096, 64, 256, _tv(2, 77), 128, 1229, 6, 0.125),
    # 3072^2 latent, 192x192 tokens, 10-step trajectory after a 2-step warmup.
    "traj_3072": Workload("traj_3072", "bf16", 2, 24, 36864, 192, 256, _tv(2, 200), 64, 7373, 5, 0.125,
                          n_blobs=5, latent=(16, 384, 384), g_ctx=2.5, g_sens=7.0,
                          warmup_steps=2, steps=10, anchor_every=4),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity shapes)."""
    return dataclasses.replace(w, **kw)


# ----------------------------------------------------------------------------- tensors
def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def attention_inputs(w: Workload, step: int = 0, roles: Sequence[str] = ("q", "k_img", "v_img", "k_txt", "v_txt")
                     ) -> Dict[str, np.ndarray]:
    """Q [B,H,N,d], K/V_img [B,H,N,d], K/V_txt [B,H,T,d] as fp32 arrays.

    For bf16 workloads each value is RNE-rounded to bf16 first, so the fp32 array holds exactly what
    the device sees; `<role>_bits` holds the uint16 patterns to upload.
    """
    shapes = {"q": (w.B, w.H, w.N, w.d), "k_img": (w.B, w.H, w.N, w.d), "v_img": (w.B, w.H, w.N, w.d),
              "k_txt": (w.B, w.H, w.T, w.d), "v_txt": (w.B, w.H, w.T, w.d)}
    out: Dict[str, np.ndarray] = {}
    for r in roles:
        x = _normal(rng_for(w.seed, r, step), shapes[r], w.std)
        if w.dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            out[r + "_bits"] = bits
            x = bf16_bits_to_f32(bits)
        out[r] = x
    return out


# ----------------------------------------------------------------------------- fp8 (OCP E4M3) inputs
def _e4m3_values() -> np.ndarray:
    """The real value of each of the 256 OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (2^-6 * m/8); exponent 15 with mantissa 7 is NaN; there are no infinities
    (largest finite 0x7E = 448)."""
    v = np.empty(256, dtype=np.float64)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
        elif e == 0:
            v[c] = sgn * 2.0 ** -6 * (m / 8.0)
        else:
            v[c] = sgn * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return v


E4M3_VALUES = _e4m3_values()
E4M3_MAX = 448.0


def fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32/fp64 -> E4M3 codes (uint8), saturating at +-448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    pos = E4M3_VALUES[:127]                    # codes 0..126: the non-negative finite values, increasing
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = a - pos[lo], pos[hi] - a
    # nearer neighbour; on a tie the even code (mantissa lsb 0)
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == pos[hi], hi, code).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def fp8_quantize_heads(x: np.ndarray) -> tuple:
    """Per-(b,h) scaled E4M3 codes of x [B,H,...]: scale = amax/448 (1 for an all-zero head) as fp32, codes of
    x / scale.  Returns (codes uint8, scale fp32 [B,H], dequantised value codes * scale in fp64)."""
    B, H = x.shape[:2]
    amax = np.abs(x.reshape(B, H, -1)).max(axis=2)
    scale = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
    sc = scale.astype(np.float64).reshape((B, H) + (1,) * (x.ndim - 2))
    codes = fp8_e4m3_bits(x.astype(np.float64) / sc)
    return codes, scale, E4M3_VALUES[codes] * sc


def attention_inputs_fp8(w: Workload, step: int = 0) -> Dict[str, np.ndarray]:
    """fp8 Q and K with bf16 V: the workload's N(0,1)*std draws, Q quantised per (b,h), K_img and K_txt
    together per (b,h) (one factor per head), V as bf16.  `q`, `k_img`, `k_txt` hold the dequantised values
    (fp64: code value times the fp32 factor, exactly what the device's operands mean); `*_fp8` the codes."""
    base = attention_inputs(dataclasses.replace(w, dtype="f32"), step)
    out: Dict[str, np.ndarray] = {}
    out["q_fp8"], out["q_descale"], out["q"] = fp8_quantize_heads(base["q"])
    N = w.N
    kcat = np.concatenate([base["k_img"], base["k_txt"]], axis=2)
    codes, out["k_descale"], deq = fp8_quantize_heads(kcat)
    out["k_img_fp8"], out["k_txt_fp8"] = codes[:, :, :N], codes[:, :, N:]
    out["k_img"], out["k_txt"] = deq[:, :, :N], deq[:, :, N:]
    for r in ("v_img", "v_txt"):
        out[r + "_bits"] = f32_to_bf16_bits(base[r])
        out[r] = bf16_bits_to_f32(out[r + "_bits"])
    return out


def blob_centres(w: Workload) -> np.ndarray:
    """Integer grid points (y, x) drawn uniformly from the token grid, one row per blob."""
    rng = rng_for(w.seed, "blobs")
    return rng.integers(0, w.side, size=(w.n_blobs, 2)).astype(np.int64)


def blob_bias(w: Workload) -> np.ndarray:
    """Per-token bias amp * sum_c exp(-dist^2 / (2 sigma^2)) on the row-major token grid, fp32 [N]."""
    if w.n_blobs == 0:
        return np.zeros(w.N, dtype=np.float32)
    yy, xx = np.divmod(np.arange(w.N), w.side)
    b = np.zeros(w.N, dtype=np.float64)
    for cy, cx in blob_centres(w):
        b += np.exp(-((yy - cy) ** 2 + (xx - cx) ** 2) / (2.0 * w.blob_sigma ** 2))
    return (w.blob_amp * b).astype(np.float32)


def pcsp_logits(w: Workload, step: int = 0) -> Dict[str, np.ndarray]:
    """Synthetic image->text logits of the cond branch.

    x [H,N,T] fp32 = N(0,1) + blob bias (same bias for every head and valid text slot; padded slots
    hold plain noise and must be ignored).  lse_img [H,N] fp32 = ln N + 1/2, the image-block
    log-sum-exp of N logits drawn from the same N(0,1) law (a modelling stand-in, not measured).
    """
    rng = rng_for(w.seed, "x", step)
    x = rng.standard_normal(size=(w.H, w.N, w.T), dtype=np.float32)
    x[:, :, : w.tv[0]] += blob_bias(w)[None, :, None]
    lse_img = np.full((w.H, w.N), math.log(w.N) + 0.5, dtype=np.float32)
    return {"x": x, "lse_img": lse_img}


def latent_eps(w: Workload) -> np.ndarray:
    """Guidance input [2, C, Hl, Wl] fp32, [0] = cond prediction, [1] = uncond prediction."""
    C, Hl, Wl = w.latent
    return rng_for(w.seed, "eps").standard_normal(size=(2, C, Hl, Wl), dtype=np.float32)


def initial_state(w: Workload) -> np.ndarray:
    """A stale cached state [B,H,N,d] (values a previous step would have left), as stored."""
    x = _normal(rng_for(w.seed, "state"), (w.B, w.H, w.N, w.d), 0.05)
    return round_to_bf16(x) if w.dtype == "bf16" else x


def random_rows(w: Workload, k: Optional[int] = None, seed_step: int = 0) -> np.ndarray:
    """k distinct ascending token indices drawn uniformly (a stand-in partition)."""
    k = w.k if k is None else k
    rng = rng_for(w.seed, "scores", seed_step)
    return np.sort(rng.choice(w.N, size=k, replace=False)).astype(np.int32)


# ----------------------------------------------------------------------------- masks
def mask_all_valid_bool(n_rows: int, n_cols: int) -> np.ndarray:
    """Redundant all-True image self-attention mask [1,1,n_rows,n_cols] (bool)."""
    return np.ones((1, 1, n_rows, n_cols), dtype=np.bool_)


def mask_zeros_f32(n_rows: int, n_cols: int) -> np.ndarray:
    return np.zeros((1, 1, n_rows, n_cols), dtype=np.float32)


def mask_row_constant_f32(w: Workload, n_cols: int, lo: float = -5.0, hi: float = 5.0) -> np.ndarray:
    """Additive mask whose row i is the constant c_i ~ U(lo, hi) over all n_cols columns."""
    c = rng_for(w.seed, "mask").uniform(lo, hi, size=w.N).astype(np.float32)
    return np.broadcast_to(c[None, None, :, None], (1, 1, w.N, n_cols)).copy()


def aesthetic_selection(w: Workload, count: int = 8) -> np.ndarray:
    """u8 [T]: `count` distinct text slots among the first valid ones marked 1 (a stand-in for the
    aesthetic prompt tokens a text-encoder match would pick)."""
    tv = min(w.tv)
    sel = np.zeros(w.T, dtype=np.uint8)
    if tv > 0:
        sel[rng_for(w.seed, "aes_sel").choice(tv, size=min(count, tv), replace=False)] = 1
    return sel


def stepcache_predictions(w: Workload, steps: int) -> np.ndarray:
    """fp32 [steps, C, Hl, Wl]: a smooth per-pixel trajectory (a random start plus a random drift per step
    and a small random curvature) standing in for a model's noise predictions across steps."""
    C, Hl, Wl = w.latent
    rng = rng_for(w.seed, "stepcache")
    e0 = rng.standard_normal((C, Hl, Wl)).astype(np.float32)
    d1 = (0.1 * rng.standard_normal((C, Hl, Wl))).astype(np.float32)
    d2 = (0.01 * rng.standard_normal((C, Hl, Wl))).astype(np.float32)
    s = np.arange(steps, dtype=np.float32)[:, None, None, None]
    return (e0[None] + s * d1[None] + s * s * d2[None]).astype(np.float32)


def hidden_states(w: Workload) -> np.ndarray:
    """bf16-representable fp32 [B, N, D] token-major hidden states, N(0,1), D = H * d."""
    return round_to_bf16(rng_for(w.seed, "hidden").standard_normal((w.B, w.N, w.H * w.d), dtype=np.float32))


def block_weights(w: Workload, ffn_mult: int = 4) -> Dict[str, np.ndarray]:
    """Random-init linear layers of one block in nn.Linear layout [out, in] (bf16-representable fp32,
    N(0, 1/in) weights, N(0, 0.02^2) biases): w1/b1 D->F, w2/b2 F->D, wqkv/bqkv D->3D; F = ffn_mult * D."""
    D = w.H * w.d
    F = ffn_mult * D
    out = {}
    for role, name, o, i in (("w_ffn1", "1", F, D), ("w_ffn2", "2", D, F), ("w_qkv", "qkv", 3 * D, D)):
        rng = rng_for(w.seed, role)
        out["w" + name] = round_to_bf16((rng.standard_normal((o, i), dtype=np.float32) / np.sqrt(i)).astype(np.float32))
        out["b" + name] = (0.02 * rng.standard_normal(o)).astype(np.float32)
    return out


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """Ascending sample of query rows used when a full-size result is checked row by row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(n, size=min(count, n), replace=False))


__all__ = [
    "Workload", "WORKLOADS", "scaled", "rng_for", "aesthetic_selection", "stepcache_predictions", "hidden_states", "block_weights", "f32_to_bf16_bits", "bf16_bits_to_f32", "round_to_bf16",
    "attention_inputs", "blob_centres", "blob_bias", "pcsp_logits", "latent_eps", "initial_state",
    "random_rows", "mask_all_valid_bool", "mask_zeros_f32", "mask_row_constant_f32", "sample_rows",
    "E4M3_VALUES", "E4M3_MAX", "fp8_e4m3_bits", "fp8_quantize_heads", "attention_inputs_fp8",
]
