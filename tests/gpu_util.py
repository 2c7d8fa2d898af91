"""Helpers for the GPU parity tests: upload seeded numpy inputs, read results back, tolerances."""
import numpy as np

# bf16 attention outputs: both bounds must hold.
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
# fp32 attention outputs (no tolerance is fixed for fp32; derived from fp32 accumulation over
# <= a few hundred keys: each output is within ~1e-6 relative, so 1e-5 leaves a 10x margin).
F32_MAX_ABS = 1e-5
F32_REL_L2 = 1e-5
# fp32 CFG: |g - o| <= 1e-5 * (|eps_u| + |gamma| |eps_c - eps_u|), and relative L2 <= 1e-5.
CFG_REL = 1e-5


def torch():
    import torch as t
    return t


def dev(x: np.ndarray, bf16_bits: np.ndarray = None):
    """numpy -> contiguous device tensor; bf16 when bit patterns are given."""
    t = torch()
    if bf16_bits is not None:
        return t.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(x)).cuda()


def host(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.bfloat16:
        return x.float().cpu().numpy().astype(np.float64)
    return x.cpu().numpy()


def err(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str = ""):
    max_abs, rel = err(got, ref)
    if dtype == "bf16":
        ok = max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2
    else:
        ok = max_abs <= F32_MAX_ABS and rel <= F32_REL_L2
    assert ok, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} ({dtype})"
    return max_abs, rel


def attn_tensors(inp: dict, dtype: str):
    """Device Q, K_img, V_img, K_txt, V_txt from a synthetic.attention_inputs() dict."""
    names = ("q", "k_img", "v_img", "k_txt", "v_txt")
    if dtype == "bf16":
        return [dev(None, inp[n + "_bits"]) for n in names]
    return [dev(inp[n]) for n in names]
