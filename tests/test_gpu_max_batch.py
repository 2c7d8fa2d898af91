"""GPU parity at the largest batch the attention entry points take (64): dense and sensitive rows on the bf16,
fp32 and fp8 paths and at head dim 128, every batch entry with its own text length (0 to T, so the per-entry
text masking is indexed by the right entry on every one), against the fp64 oracle."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as OA
from tests.gpu_util import assert_close, attn_tensors, dev, host, torch

pytestmark = pytest.mark.gpu

B = 64
# text lengths 0..64, each entry its own: 7*i mod 65 visits 0 and 64 among the 64 entries
TV = tuple((7 * i) % 65 for i in range(B))


def _w(dtype="bf16", d=64, N=70, H=2):
    return syn.scaled(syn.WORKLOADS["dense_1024"], side=1, B=B, H=H, N=N, T=64, tv=TV, dtype=dtype, d=d)


def _oracle(w, inp, rows=None):
    return OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], w.tv, rows=rows)


def _fp8(codes):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(codes)).view(t.float8_e4m3fn).cuda()


def _tensors(w, inp):
    if w.dtype == "fp8":
        return ([_fp8(inp["q_fp8"]), _fp8(inp["k_img_fp8"]), dev(None, inp["v_img_bits"]),
                 _fp8(inp["k_txt_fp8"]), dev(None, inp["v_txt_bits"])],
                dict(q_descale=dev(inp["q_descale"].reshape(-1)), k_descale=dev(inp["k_descale"].reshape(-1))))
    return attn_tensors(inp, w.dtype), {}


def _inputs(w):
    return syn.attention_inputs_fp8(w) if w.dtype == "fp8" else syn.attention_inputs(w)


CASES = [("bf16", 64), ("f32", 64), ("fp8", 64), ("bf16", 128), ("fp8", 128)]


@pytest.mark.parametrize("dtype,d", CASES, ids=lambda c: str(c))
def test_max_batch_dense_and_rows(lib, dtype, d):
    t = torch()
    w = _w(dtype=dtype, d=d)
    inp = _inputs(w)
    (q, ki, vi, kt, vt), extra = _tensors(w, inp)
    odt = t.float32 if dtype == "f32" else t.bfloat16
    tol = "f32" if dtype == "f32" else "bf16"
    # dense with lse (the exact row-sum form), rows without it (the fast form)
    lse = t.full((w.B, w.H, w.N), float("nan"), dtype=t.float32, device="cuda")
    out = t.zeros(q.shape, dtype=odt, device="cuda")
    lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, out, lse=lse, **extra)
    t.cuda.synchronize()
    ro, rlse = _oracle(w, inp)
    assert_close(host(out), ro, tol, f"B=64 dense {dtype} d={d}")
    assert np.max(np.abs(host(lse) - rlse)) < (1e-5 if dtype == "f32" else 1e-4)
    # sensitive rows into a stale state: the other rows stay as they were, the chosen ones match the oracle
    rows = syn.random_rows(w, k=23)
    st = syn.initial_state(syn.scaled(w, dtype="f32" if dtype == "f32" else "bf16"))
    state = t.from_numpy(st.astype(np.float32)).to(odt).cuda()
    lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, dev(rows), state, **extra)
    t.cuda.synchronize()
    o = host(state)
    C = np.setdiff1d(np.arange(w.N), rows)
    assert np.array_equal(o[:, :, C], st[:, :, C].astype(np.float64))
    assert_close(o[:, :, rows], _oracle(w, inp, rows)[0], tol, f"B=64 rows {dtype} d={d}")
