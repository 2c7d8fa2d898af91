"""Python binding of libsafe_attn (the spatially-adaptive DiT attention step on MI355X / gfx950).

Argument marshalling only: torch tensors supply device pointers, shapes and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  Each function has the name and
meaning of the C entry point it calls (see include/safe_attn.h).  There is no CPU fallback: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsafe_attn.so")

SAFE_DTYPE_BF16, SAFE_DTYPE_F32, SAFE_DTYPE_BOOL, SAFE_DTYPE_FP8_E4M3 = 0, 1, 2, 3
SAFE_MAX_BATCH = 64
SAFE_STEP_DENSE, SAFE_STEP_ROWS = 0, 1
EXPORTS = ("safe_attn_dense", "safe_attn_rows", "safe_mask_is_row_constant", "safe_mask_check_launch",
           "safe_pcsp_accumulate",
           "safe_pcsp_partition", "safe_swcfg_combine", "safe_gather_rows", "safe_scatter_rows",
           "safe_affinity_accumulate", "safe_percentile_count", "safe_stepcache_extrapolate",
           "safe_stepcache_plan", "safe_trajectory_plan", "safe_rows_ffn", "safe_rows_ffn_workspace_bytes",
           "safe_rows_qkv", "safe_rows_ffn_noalloc", "safe_rows_ffn_noalloc_max_bytes",
           "safe_status_string", "safe_version")


class SafeAttnError(RuntimeError):
    def __init__(self, code: int, name: str, call: str):
        super().__init__(f"{call} failed: {name} ({code})")
        self.code = code
        self.name = name


class safe_attn_desc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("T", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k_img", ctypes.c_void_p), ("v_img", ctypes.c_void_p),
        ("k_txt", ctypes.c_void_p), ("v_txt", ctypes.c_void_p),
        ("text_valid_len", ctypes.POINTER(ctypes.c_int32)),
        ("scale", ctypes.c_float),
        ("mask", ctypes.c_void_p), ("mask_dtype", ctypes.c_int32), ("mask_B", ctypes.c_int32),
        ("mask_H", ctypes.c_int32), ("mask_cols", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("xattn_out", ctypes.c_void_p),
        ("lse_img_out", ctypes.c_void_p), ("q_descale", ctypes.c_void_p), ("k_descale", ctypes.c_void_p),
    ]


_lib = None


def load(path: Optional[str] = None):
    """Load the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with python diffusion_transformer_spatially_amd/build.py")
    lib = ctypes.CDLL(p)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    P = ctypes.POINTER
    lib.safe_attn_dense.argtypes = [P(safe_attn_desc), vp]
    lib.safe_attn_rows.argtypes = [P(safe_attn_desc), vp, i32, vp]
    lib.safe_mask_is_row_constant.argtypes = [vp, i32, i32, i32, i32, i32, i32, P(i32), i32, vp, P(i32), vp, vp]
    lib.safe_mask_check_launch.argtypes = [vp, i32, i32, i32, i32, i32, i32, P(i32), i32, vp, vp, vp]
    lib.safe_pcsp_accumulate.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, i32, vp]
    lib.safe_pcsp_partition.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
    lib.safe_swcfg_combine.argtypes = [vp, vp, i32, i32, i32, i32, f32, f32, vp, vp]
    lib.safe_gather_rows.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.safe_scatter_rows.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.safe_affinity_accumulate.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, i32, vp]
    lib.safe_percentile_count.argtypes = [i32, i32, P(i32)]
    lib.safe_stepcache_extrapolate.argtypes = [vp, vp, ctypes.c_int64, f32, vp, vp]
    lib.safe_stepcache_plan.argtypes = [i32, i32, P(i32), P(i32), P(f32)]
    lib.safe_trajectory_plan.argtypes = [i32, i32, P(i32)]
    lib.safe_rows_ffn.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.safe_rows_ffn_workspace_bytes.argtypes = [i32, i32, i32]
    lib.safe_rows_qkv.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.safe_rows_ffn_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.safe_rows_ffn_noalloc_max_bytes.argtypes = []
    for name in EXPORTS[:-2]:
        getattr(lib, name).restype = i32
    lib.safe_rows_ffn_workspace_bytes.restype = ctypes.c_size_t
    lib.safe_rows_ffn_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.safe_status_string.argtypes = [i32]
    lib.safe_status_string.restype = ctypes.c_char_p
    lib.safe_version.argtypes = []
    lib.safe_version.restype = i32
    _lib = lib
    return lib


def _check(code: int, call: str):
    if code != 0:
        raise SafeAttnError(code, load().safe_status_string(code).decode(), call)


# ----------------------------------------------------------------------------- marshalling helpers
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t, shape, dtype, name: str, optional: bool = True, at_least: bool = False):
    """Shape / dtype check of a tensor handed to the library (the C ABI sees only its address, so a tensor of
    the wrong size would be read or written past its end).  shape: a tuple, or an int for a number of
    elements (at_least: that many or more); dtype: a torch dtype or a tuple of them."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if isinstance(shape, int):
        ok_shape = t.numel() >= shape if at_least else t.numel() == shape
    else:
        ok_shape = tuple(t.shape) == tuple(shape)
    if not ok_shape:
        want = f"at least {shape} elements" if at_least else f"shape {shape}"
        raise ValueError(f"{name} must have {want}, got {tuple(t.shape)}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise ValueError(f"{name} must be {' or '.join(str(x) for x in dts)}, got {t.dtype}")


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SAFE_DTYPE_BF16
    if t.dtype == torch.float32:
        return SAFE_DTYPE_F32
    if t.dtype == torch.bool:
        return SAFE_DTYPE_BOOL
    if t.dtype == torch.float8_e4m3fn:
        return SAFE_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _desc(q, k_img, v_img, k_txt, v_txt, text_valid_len: Sequence[int], out, scale, mask, lse, xattn_out,
          lse_img_out, q_descale=None, k_descale=None):
    torch = _torch()
    B, H, N, d = q.shape
    T = k_txt.shape[2] if k_txt is not None else 0
    tv = (ctypes.c_int32 * max(1, len(text_valid_len)))(*[int(x) for x in text_valid_len])
    if len(text_valid_len) != B:
        raise ValueError("text_valid_len needs one entry per batch element")
    fp8 = q.dtype == torch.float8_e4m3fn
    vdt = torch.bfloat16 if fp8 else q.dtype  # fp8 Q / K come with bf16 V and output
    for t, dt in ((k_img, q.dtype), (v_img, vdt), (out, vdt)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != dt:
            raise ValueError("q, k_img, v_img and out must share shape [B,H,N,d]; k_img the dtype of q; v_img and "
                             "out the dtype of q, or bf16 when q is fp8")
    if k_txt is not None and (k_txt.dtype != q.dtype or v_txt.dtype != vdt):
        raise ValueError("k_txt / v_txt must have the dtypes of k_img / v_img")
    for f in (q_descale, k_descale):
        if f is not None and (f.dtype != torch.float32 or f.numel() != B * H):
            raise ValueError("q_descale / k_descale must be fp32 with B*H entries")
    if k_txt is not None and (tuple(k_txt.shape) != (B, H, T, d) or tuple(v_txt.shape) != (B, H, T, d)):
        raise ValueError("k_txt and v_txt must be [B,H,T,d]")
    _need(lse, (B, H, N), torch.float32, "lse")
    _need(xattn_out, (H, N, T), torch.float32, "xattn_out")
    _need(lse_img_out, (H, N), torch.float32, "lse_img_out")
    if mask is not None:
        if mask.dim() != 4 or mask.shape[2] != N:
            raise ValueError("mask must be [mask_B, mask_H, N, mask_cols]")
        _need(mask, tuple(mask.shape), (torch.bool, torch.float32), "mask")
    D = safe_attn_desc()
    D.dtype = _dtype_code(q)
    D.B, D.H, D.N, D.T, D.d = B, H, N, T, d
    D.q, D.k_img, D.v_img = _ptr(q), _ptr(k_img), _ptr(v_img)
    D.k_txt, D.v_txt = _ptr(k_txt), _ptr(v_txt)
    D.text_valid_len = ctypes.cast(tv, ctypes.POINTER(ctypes.c_int32))
    D.scale = float(scale)
    if mask is not None:
        D.mask = _ptr(mask)
        D.mask_dtype = _dtype_code(mask)
        D.mask_B, D.mask_H, D.mask_cols = mask.shape[0], mask.shape[1], mask.shape[3]
    D.out = _ptr(out)
    D.lse = _ptr(lse)
    D.xattn_out = _ptr(xattn_out)
    D.lse_img_out = _ptr(lse_img_out)
    D.q_descale = _ptr(q_descale)
    D.k_descale = _ptr(k_descale)
    return D, tv


# ----------------------------------------------------------------------------- entry points
def safe_attn_dense(q, k_img, v_img, k_txt, v_txt, text_valid_len, out, scale=0.0, mask=None, lse=None,
                    xattn_out=None, lse_img_out=None, stream=None, q_descale=None, k_descale=None):
    """Dense anchor step: all N image rows of `out` (safe_attn_dense).  fp8 (float8_e4m3fn) q / k take
    bf16 v / out and optional fp32 [B, H] dequantisation factors q_descale / k_descale."""
    D, _keep = _desc(q, k_img, v_img, k_txt, v_txt, text_valid_len, out, scale, mask, lse, xattn_out, lse_img_out,
                     q_descale, k_descale)
    _check(load().safe_attn_dense(ctypes.byref(D), _stream(stream)), "safe_attn_dense")
    return out


def safe_attn_rows(q, k_img, v_img, k_txt, v_txt, text_valid_len, rows, out, scale=0.0, mask=None, lse=None,
                   xattn_out=None, lse_img_out=None, stream=None, q_descale=None, k_descale=None):
    """Sensitive-row step: rows[] of `out` only, against the global keys (safe_attn_rows)."""
    torch = _torch()
    if rows.dtype != torch.int32 or rows.dim() != 1:
        raise ValueError("rows must be a 1-D int32 tensor")
    D, _keep = _desc(q, k_img, v_img, k_txt, v_txt, text_valid_len, out, scale, mask, lse, xattn_out, lse_img_out,
                     q_descale, k_descale)
    _check(load().safe_attn_rows(ctypes.byref(D), _ptr(rows), rows.numel(), _stream(stream)), "safe_attn_rows")
    return out


def _mask_check_args(mask, N, flag_ws, c_out):
    torch = _torch()
    if mask.dim() != 4 or mask.shape[2] != N:
        raise ValueError("mask must be [mask_B, mask_H, N, mask_cols]")
    _need(mask, tuple(mask.shape), (torch.bool, torch.float32), "mask")
    _need(flag_ws, 1, torch.int32, "flag_ws", optional=False)
    _need(c_out, mask.shape[0] * mask.shape[1] * N, torch.float32, "c_out")


def safe_mask_is_row_constant(mask, N: int, T: int, text_valid_len, flag_ws, c_out=None, stream=None) -> bool:
    """Exact elision check; synchronous (safe_mask_is_row_constant)."""
    _mask_check_args(mask, N, flag_ws, c_out)
    B = len(text_valid_len)
    tv = (ctypes.c_int32 * B)(*[int(x) for x in text_valid_len])
    res = ctypes.c_int32(0)
    _check(load().safe_mask_is_row_constant(
        _ptr(mask), _dtype_code(mask), mask.shape[0], mask.shape[1], N, mask.shape[3], T,
        ctypes.cast(tv, ctypes.POINTER(ctypes.c_int32)), B, _ptr(flag_ws), ctypes.byref(res), _ptr(c_out),
        _stream(stream)), "safe_mask_is_row_constant")
    return bool(res.value)


def safe_mask_check_launch(mask, N: int, T: int, text_valid_len, flag_ws, c_out=None, stream=None):
    """Exact elision check, launched only: flag_ws (device int32[1]) holds the verdict once the stream
    reaches this point (safe_mask_check_launch)."""
    _mask_check_args(mask, N, flag_ws, c_out)
    B = len(text_valid_len)
    tv = (ctypes.c_int32 * B)(*[int(x) for x in text_valid_len])
    _check(load().safe_mask_check_launch(
        _ptr(mask), _dtype_code(mask), mask.shape[0], mask.shape[1], N, mask.shape[3], T,
        ctypes.cast(tv, ctypes.POINTER(ctypes.c_int32)), B, _ptr(flag_ws), _ptr(c_out), _stream(stream)),
        "safe_mask_check_launch")
    return flag_ws


def safe_pcsp_accumulate(x, lse_img, Tv: int, c0: int, c1: int, scores, accumulate: bool, stream=None):
    """scores (+)= per-token text-content attention mass summed over heads (safe_pcsp_accumulate)."""
    torch = _torch()
    H, N, T = x.shape
    _need(x, (H, N, T), torch.float32, "x")
    _need(lse_img, (H, N), torch.float32, "lse_img")
    _need(scores, N, torch.float32, "scores", optional=False)
    _check(load().safe_pcsp_accumulate(_ptr(x), _ptr(lse_img), H, N, T, Tv, c0, c1, _ptr(scores),
                                       1 if accumulate else 0, _stream(stream)), "safe_pcsp_accumulate")
    return scores


def safe_pcsp_partition(scores, k: int, S, C, is_sens, s01=None, stream=None):
    """Exact top-k partition of the scores (safe_pcsp_partition)."""
    torch = _torch()
    N = scores.numel()
    _need(scores, N, torch.float32, "scores")
    if not 0 <= k <= N:
        raise ValueError("k must lie in [0, N]")
    _need(S, k, torch.int32, "S", optional=(k == 0), at_least=True)
    _need(C, N - k, torch.int32, "C", optional=(k == N), at_least=True)
    _need(is_sens, N, torch.uint8, "is_sens", optional=False)
    _need(s01, N, torch.float32, "s01")
    _check(load().safe_pcsp_partition(_ptr(scores), N, k, _ptr(S), _ptr(C), _ptr(is_sens), _ptr(s01),
                                      _stream(stream)), "safe_pcsp_partition")


def safe_swcfg_combine(eps, s, side: int, g_ctx: float, g_sens: float, out, stream=None):
    """Per-token guidance combine (safe_swcfg_combine)."""
    torch = _torch()
    _, C, Hl, Wl = eps.shape
    _need(eps, (2, C, Hl, Wl), torch.float32, "eps")
    _need(s, side * side, torch.float32, "s", optional=False)
    _need(out, (C, Hl, Wl), torch.float32, "out", optional=False)
    _check(load().safe_swcfg_combine(_ptr(eps), _ptr(s), C, Hl, Wl, side, float(g_ctx), float(g_sens), _ptr(out),
                                     _stream(stream)), "safe_swcfg_combine")
    return out


def _rows_arg(rows):
    torch = _torch()
    if rows.dtype != torch.int32 or rows.dim() != 1:
        raise ValueError("rows must be a 1-D int32 tensor")


def safe_gather_rows(state, rows, packed, stream=None):
    B, H, N, d = state.shape
    _rows_arg(rows)
    _need(packed, (B, H, rows.numel(), d), state.dtype, "packed", optional=False)
    _check(load().safe_gather_rows(_ptr(state), _ptr(rows), rows.numel(), B, H, N, d, _dtype_code(state),
                                   _ptr(packed), _stream(stream)), "safe_gather_rows")
    return packed


def safe_scatter_rows(packed, rows, state, stream=None):
    B, H, N, d = state.shape
    _rows_arg(rows)
    _need(packed, (B, H, rows.numel(), d), state.dtype, "packed", optional=False)
    _check(load().safe_scatter_rows(_ptr(packed), _ptr(rows), rows.numel(), B, H, N, d, _dtype_code(state),
                                    _ptr(state), _stream(stream)), "safe_scatter_rows")
    return state


def safe_affinity_accumulate(x, lse_img, Tv: int, sel, scores, accumulate: bool, stream=None):
    """scores (+)= per-token attention mass on the selected text slots, summed over heads
    (safe_affinity_accumulate).  sel: device u8 [T]."""
    torch = _torch()
    H, N, T = x.shape
    _need(x, (H, N, T), torch.float32, "x")
    _need(lse_img, (H, N), torch.float32, "lse_img")
    _need(sel, T, torch.uint8, "sel", optional=False)
    _need(scores, N, torch.float32, "scores", optional=False)
    _check(load().safe_affinity_accumulate(_ptr(x), _ptr(lse_img), H, N, T, Tv, _ptr(sel), _ptr(scores),
                                           1 if accumulate else 0, _stream(stream)), "safe_affinity_accumulate")
    return scores


def safe_percentile_count(N: int, pct_bp: int) -> int:
    """Tokens kept at the (pct_bp / 100)-th percentile (safe_percentile_count; host only)."""
    k = ctypes.c_int32(0)
    _check(load().safe_percentile_count(int(N), int(pct_bp), ctypes.byref(k)), "safe_percentile_count")
    return int(k.value)


def safe_stepcache_extrapolate(eps_a, eps_b, w: float, out, stream=None):
    """out = eps_b + w (eps_b - eps_a), elementwise over fp32 tensors (safe_stepcache_extrapolate)."""
    torch = _torch()
    n = out.numel()
    for t, name in ((eps_a, "eps_a"), (eps_b, "eps_b"), (out, "out")):
        _need(t, n, torch.float32, name, optional=False)
    _check(load().safe_stepcache_extrapolate(_ptr(eps_a), _ptr(eps_b), n, float(w), _ptr(out), _stream(stream)),
           "safe_stepcache_extrapolate")
    return out


def safe_stepcache_plan(steps: int, delta: int):
    """[(full, src_a, src_b, w)] per step (safe_stepcache_plan; host only)."""
    a, b, w = (ctypes.c_int32 * max(steps, 1))(), (ctypes.c_int32 * max(steps, 1))(), (ctypes.c_float * max(steps, 1))()
    _check(load().safe_stepcache_plan(int(steps), int(delta), a, b, w), "safe_stepcache_plan")
    return [(a[s] < 0, int(a[s]), int(b[s]), float(w[s])) for s in range(steps)]


def safe_trajectory_plan(steps: int, anchor_every: int):
    """Per step SAFE_STEP_DENSE or SAFE_STEP_ROWS (safe_trajectory_plan; host only)."""
    k = (ctypes.c_int32 * max(steps, 1))()
    _check(load().safe_trajectory_plan(int(steps), int(anchor_every), k), "safe_trajectory_plan")
    return [int(k[t]) for t in range(steps)]


def safe_rows_ffn_workspace_bytes(B: int, k: int, F: int) -> int:
    return int(load().safe_rows_ffn_workspace_bytes(int(B), int(k), int(F)))


def _ffn_args(x, rows, w1, b1, w2, b2, cache):
    torch = _torch()
    B, N, D = x.shape
    F = w1.shape[0]
    _rows_arg(rows)
    _need(x, (B, N, D), torch.bfloat16, "x")
    _need(w1, (F, D), torch.bfloat16, "w1")
    _need(w2, (D, F), torch.bfloat16, "w2", optional=False)
    _need(b1, F, torch.float32, "b1")
    _need(b2, D, torch.float32, "b2")
    _need(cache, (B, N, D), torch.bfloat16, "cache", optional=False)


def safe_rows_ffn(x, rows, w1, b1, w2, b2, cache, ws, stream=None):
    """cache[:, rows] = FFN(x[:, rows]) (safe_rows_ffn).  x, cache: bf16 [B, N, D]; w1 [F, D], w2 [D, F]
    bf16; b1 / b2 fp32 or None; ws: device workspace tensor of at least safe_rows_ffn_workspace_bytes."""
    B, N, D = x.shape
    F = w1.shape[0]
    _ffn_args(x, rows, w1, b1, w2, b2, cache)
    _check(load().safe_rows_ffn(_ptr(x), _ptr(rows), rows.numel(), B, N, D, F, _ptr(w1), _ptr(b1), _ptr(w2),
                                _ptr(b2), _ptr(cache), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "safe_rows_ffn")
    return cache


def safe_rows_ffn_noalloc(x, rows, w1, b1, w2, b2, cache, stream=None):
    """safe_rows_ffn without a workspace: the hidden activation lives in the library's fixed per-GPU array
    (safe_rows_ffn_noalloc; at most safe_rows_ffn_noalloc_max_bytes() bytes)."""
    B, N, D = x.shape
    F = w1.shape[0]
    _ffn_args(x, rows, w1, b1, w2, b2, cache)
    _check(load().safe_rows_ffn_noalloc(_ptr(x), _ptr(rows), rows.numel(), B, N, D, F, _ptr(w1), _ptr(b1), _ptr(w2),
                                        _ptr(b2), _ptr(cache), _stream(stream)), "safe_rows_ffn_noalloc")
    return cache


def safe_rows_ffn_noalloc_max_bytes() -> int:
    return int(load().safe_rows_ffn_noalloc_max_bytes())


def safe_rows_qkv(x, rows, wqkv, bqkv, q, k_cache, v_cache, stream=None):
    """Rows S of q / k_cache / v_cache [B, H, N, d] from the projection of x[:, rows] (safe_rows_qkv)."""
    torch = _torch()
    B, N, D = x.shape
    _, H, _, d = q.shape
    _rows_arg(rows)
    _need(x, (B, N, D), torch.bfloat16, "x")
    if H * d != D:
        raise ValueError("q must be [B, H, N, d] with H * d equal to the hidden width of x")
    _need(wqkv, (3 * D, D), torch.bfloat16, "wqkv", optional=False)
    _need(bqkv, 3 * D, torch.float32, "bqkv")
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, (B, H, N, d), torch.bfloat16, name, optional=False)
    _check(load().safe_rows_qkv(_ptr(x), _ptr(rows), rows.numel(), B, N, H, d, _ptr(wqkv), _ptr(bqkv), _ptr(q),
                                _ptr(k_cache), _ptr(v_cache), _stream(stream)), "safe_rows_qkv")
    return q, k_cache, v_cache


def safe_version() -> int:
    return load().safe_version()


# ----------------------------------------------------------------------------- elide-or-keep helper
class MaskPolicy:
    """Checks a supplied mask once (per tensor version) and drops it when it is provably redundant.

    Mirrors the exact fast-path rewrite: a removable mask goes to the mask-free kernels, any other mask
    is kept and applied exactly.  A cached verdict belongs to one live tensor: each entry holds a weak
    reference to the mask it was computed for and is used only while that very tensor is alive and still
    at the same version, storage address, shape and dtype (a freed mask's address is routinely handed to
    the next allocation of the same size, whose version count starts again at zero).  Entries are dropped
    when their tensor is garbage-collected, so the cache holds at most one entry per live mask and
    argument set.
    """

    def __init__(self):
        self._cache = {}
        self._flag = None

    def _evict(self, ident):
        for key in [k for k in self._cache if k[0] == ident]:
            del self._cache[key]

    def elide(self, mask, N: int, T: int, text_valid_len):
        if mask is None:
            return None
        import weakref
        torch = _torch()
        key = (id(mask), int(N), int(T), tuple(int(t) for t in text_valid_len))
        stamp = (mask.data_ptr(), mask._version, tuple(mask.shape), mask.dtype)
        hit = self._cache.get(key)
        if hit is None or hit[0]() is not mask or hit[1] != stamp:
            if self._flag is None or self._flag.device != mask.device:
                self._flag = torch.empty(1, dtype=torch.int32, device=mask.device)
            verdict = safe_mask_is_row_constant(mask, N, T, text_valid_len, self._flag)
            ident = id(mask)
            this = weakref.ref(self)
            ref = weakref.ref(mask, lambda _r, ident=ident, this=this: this() is not None and this()._evict(ident))
            self._cache[key] = (ref, stamp, verdict)
            hit = self._cache[key]
        return None if hit[2] else mask
