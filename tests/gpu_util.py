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
# Worst single output row (one query row of one (b, h)): ||o_row - ref_row|| / ||ref_row|| over the head
# dimension.  The whole-tensor bounds above average over tens of thousands of rows, so on their own they
# would let a few wholly wrong rows through (at the N(0,1)*0.125 workloads |o| stays below 1e-2, so the
# max-abs bound cannot fail, and one zeroed row-head among 59k adds only ~4e-3 to the relative L2).
# Bounds from the measured distribution of the worst row over every parity case on MI355X (bf16: 121
# assertions, worst 5.2e-3 on the logit-std-3 stress rows, 2.8-3.3e-3 on the full-size 1024^2 / 2560^2 /
# 3072^2 launches, 2.5-2.6e-3 on the block products), about twice the worst case.  fp32 rows take the fp32
# figure above (about 1e-6 per output from fp32 accumulation, with the 10x margin): a wider seeded sweep put a
# row with about 1000 keys, logits four times the workload's and an fp32 mask at 2.2e-6.
# A row with a missing key tile, a wrong row index or a zero output lands between 1e-1 and 1.
BF16_ROW_REL = 1e-2
F32_ROW_REL = 1e-5
ROW_STATS = []  # (what, dtype, worst row, rel-L2) of every assert_close call, for the run's summary


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


def worst_row(got, ref) -> float:
    """Largest relative L2 error of one row (last axis) of got against ref; a row whose reference is all
    zero counts its absolute error (so it must come out exactly zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    d = np.linalg.norm((got - ref).reshape(-1, ref.shape[-1]), axis=1)
    r = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    return float(np.max(np.where(r > 0, d / np.where(r > 0, r, 1.0), d / 1e-300)))


def assert_close(got, ref, dtype: str, what: str = ""):
    """Both whole-tensor bounds and the worst-row bound (rows along the last axis)."""
    max_abs, rel = err(got, ref)
    wr = worst_row(got, ref)
    ROW_STATS.append((what, dtype, wr, rel))
    if dtype == "bf16":
        ok = max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2 and wr <= BF16_ROW_REL
    else:
        ok = max_abs <= F32_MAX_ABS and rel <= F32_REL_L2 and wr <= F32_ROW_REL
    assert ok, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst_row={wr:.3e} ({dtype})"
    return max_abs, rel


def attn_tensors(inp: dict, dtype: str):
    """Device Q, K_img, V_img, K_txt, V_txt from a synthetic.attention_inputs() dict."""
    names = ("q", "k_img", "v_img", "k_txt", "v_txt")
    if dtype == "bf16":
        return [dev(None, inp[n + "_bits"]) for n in names]
    return [dev(inp[n]) for n in names]
