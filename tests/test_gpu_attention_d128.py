"""GPU parity of the attention entry points at head dim 128 against the fp64 oracle: the bf16 MFMA kernel
(dense, gathered rows, every work shape, kept bool masks, the exact-sum path with its outputs) and the
generic kernel (fp32, and the bf16 masks the MFMA kernel does not take)."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as OA
from tests.gpu_util import assert_close, attn_tensors, dev, err, host, torch
from tests.test_gpu_attention import _kept_mask, _oracle, _run

pytestmark = pytest.mark.gpu


def _w(base="dense_1024", **kw):
    return syn.scaled(syn.WORKLOADS[base], d=128, side=1, **kw)


SHAPES = [
    (1, 1, 1, 0, (0,)),
    (1, 2, 64, 64, (64,)),
    (2, 3, 65, 40, (17, 0)),
    (2, 2, 127, 256, (77, 1)),
    (1, 2, 300, 256, (65,)),
    (2, 2, 1000, 256, (200, 63)),
]


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dT%d" % s[:4])
def test_d128_dense_parity(lib, shape, want_lse):
    B, H, N, T, tv = shape
    w = _w(B=B, H=H, N=N, T=T, tv=tv)
    inp = syn.attention_inputs(w)
    o, lse, _, _ = _run(lib, w, inp, want_lse=want_lse)
    ro, rlse = _oracle(w, inp)
    assert_close(o, ro, "bf16", f"d128 dense {shape}")
    if want_lse:
        assert np.max(np.abs(lse - rlse)) < 1e-4


@pytest.mark.parametrize("k", [0, 1, 63, 65, 300])
def test_d128_rows_parity_and_untouched_context(lib, k):
    w = _w("srsu_1024", B=2, H=3, N=300, T=256, tv=(77, 5))
    inp = syn.attention_inputs(w)
    rows = syn.random_rows(w, k=k)
    state = syn.initial_state(w)
    o, _, _, _ = _run(lib, w, inp, rows=rows, state=state, want_lse=(k % 2 == 1))
    C = np.setdiff1d(np.arange(w.N), rows)
    assert np.array_equal(o[:, :, C], state[:, :, C].astype(np.float64))
    if k:
        ro, _ = _oracle(w, inp, rows=rows)
        assert_close(o[:, :, rows], ro, "bf16", f"d128 rows k={k}")
    if k == w.N:
        od, _, _, _ = _run(lib, w, inp, want_lse=False)
        assert np.array_equal(o, od)


@pytest.mark.parametrize("B,H,N,T,tv,k", [
    (1, 8, 2000, 256, (77,), None),         # 504 one-block waves: key range in two halves
    (2, 8, 4160, 256, (77, 0), None),       # 2080 one-block waves: no split
    (2, 24, 4096, 256, (77, 77), 1229),     # the 1024^2 rows launch (1872 waves): halves, gathered rows
    (1, 3, 193, 0, (0,), None),             # 4 key tiles: halves of 2 and 2 (ragged tail in the second)
    (1, 3, 130, 0, (0,), None),             # 3 key tiles: halves of 2 and 1
    (1, 3, 40, 0, (0,), None),              # 1 key tile: the second half has none
    (2, 2, 64, 256, (70, 3), None),         # 3 and 2 key tiles by batch entry (text tiles in both halves)
])
def test_d128_work_shapes(lib, B, H, N, T, tv, k):
    w = _w("srsu_1024", B=B, H=H, N=N, T=T, tv=tv)
    inp = syn.attention_inputs(w)
    if k is None:
        o, _, _, _ = _run(lib, w, inp, want_lse=False)
        ro, _ = _oracle(w, inp)
        assert_close(o, ro, "bf16", f"d128 dense B{B}H{H}N{N}")
    else:
        rows = syn.random_rows(w, k=k)
        state = syn.initial_state(w)
        o, _, _, _ = _run(lib, w, inp, rows=rows, state=state, want_lse=False)
        ro, _ = _oracle(w, inp, rows=rows)
        assert_close(o[:, :, rows], ro, "bf16", f"d128 rows B{B}H{H}N{N}k{k}")
        C = np.setdiff1d(np.arange(w.N), rows)
        assert np.array_equal(o[:, :, C], state[:, :, C].astype(np.float64))


def test_d128_closed_forms_and_rescaling(lib):
    w = _w(B=2, H=2, N=257, T=256, tv=(77, 0))
    inp = syn.attention_inputs(w)
    ones = dict(inp, v_img_bits=np.full_like(inp["v_img_bits"], 0x3F80),
                v_txt_bits=np.full_like(inp["v_txt_bits"], 0x3F80))
    o, _, _, _ = _run(lib, w, ones, want_lse=False)
    assert np.max(np.abs(o - 1.0)) <= 1e-6
    zq = dict(inp, q_bits=np.zeros_like(inp["q_bits"]))
    o, lse, _, _ = _run(lib, w, zq)
    for b in range(2):
        vals = np.concatenate([inp["v_img"][b], inp["v_txt"][b, :, : w.tv[b]]], axis=1).astype(np.float64)
        assert_close(o[b], np.broadcast_to(vals.mean(axis=1)[:, None, :], o[b].shape), "bf16", "Q = 0: mean of the valid V rows")
        assert np.max(np.abs(lse[b] - np.log(w.N + w.tv[b]))) < 1e-3
    # large logits: the running max grows often, so the lazy-max exact path runs
    w3 = _w(B=1, H=2, N=513, T=256, tv=(100,), std=3.0)
    inp3 = dict(syn.attention_inputs(w3))
    for r in ("v_img", "v_txt"):
        v = (inp3[r] * np.float32(0.125 / 3.0)).astype(np.float32)
        inp3[r], inp3[r + "_bits"] = syn.round_to_bf16(v), syn.f32_to_bf16_bits(v)
    for want_lse in (False, True):
        o, _, _, _ = _run(lib, w3, inp3, want_lse=want_lse)
        ro, _ = _oracle(w3, inp3)
        assert_close(o, ro, "bf16", f"d128 std=3 lse={want_lse}")


def test_d128_emission_and_determinism(lib):
    w = _w(B=2, H=3, N=333, T=256, tv=(77, 20))
    inp = syn.attention_inputs(w)
    o1, l1, x, li = _run(lib, w, inp, emission=True)
    _, _, rx, rli = _oracle(w, inp, emission=True)
    assert np.max(np.abs(x[:, :, :77] - rx)) < 1e-5
    assert np.max(np.abs(li - rli)) < 1e-4
    o2, l2, _, _ = _run(lib, w, inp, emission=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("N,T,tv,kind,text_cols,mB,mH,want_lse", [
    (256, 64, (30, 64), "bool", True, 1, 1, False),    # MFMA kernel
    (320, 32, (0, 32), "bool", False, 2, 3, True),     # MFMA kernel, image-only mask, exact-sum path
    (448, 256, (77, 20), "f32", True, 2, 1, False),    # fp32 mask at d = 128: generic kernel
    (150, 64, (30, 64), "bool", True, 1, 1, True),     # N not a multiple of 16: generic kernel
])
def test_d128_kept_masks(lib, N, T, tv, kind, text_cols, mB, mH, want_lse):
    w = _w(B=2, H=3, N=N, T=T, tv=tv)
    inp = syn.attention_inputs(w)
    r = np.random.default_rng(N + T + mB + mH)
    cols = N + T if text_cols else N
    full = (5, N - 1) if text_cols else ()
    m = _kept_mask(r, kind, (mB, mH, N, cols), N, max(tv), full_rows=full)
    o, lse, _, _ = _run(lib, w, inp, mask=dev(m), want_lse=want_lse)
    ro, rlse = _oracle(w, inp, mask=m)
    assert_close(o, ro, "bf16", "d128 kept mask")
    if want_lse:
        fin = np.isfinite(rlse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-4
    rows = np.array([0, 5, N // 2, N - 1], dtype=np.int32)
    state = syn.initial_state(w)
    o, _, _, _ = _run(lib, w, inp, mask=dev(m), rows=rows, state=state, want_lse=False)
    ro, _ = _oracle(w, inp, mask=m, rows=rows)
    assert_close(o[:, :, rows], ro, "bf16", "d128 kept mask rows")


def test_d128_f32_generic(lib):
    w = syn.scaled(syn.WORKLOADS["tiny_srsu_f32"], d=128)
    inp = syn.attention_inputs(w)
    o, lse, x, li = _run(lib, w, inp, emission=True)
    ro, rlse, rx, rli = _oracle(w, inp, emission=True)
    assert_close(o, ro, "f32", "d128 fp32 dense")
    assert np.max(np.abs(lse - rlse)) < 1e-5
    assert np.max(np.abs(x[:, :, : w.tv[0]] - rx)) < 1e-5
    assert np.max(np.abs(li - rli)) < 1e-5
    rows = syn.random_rows(w, k=77)
    state = syn.initial_state(w)
    o2, _, _, _ = _run(lib, w, inp, rows=rows, state=state)
    assert_close(o2[:, :, rows], ro[:, :, rows], "f32", "d128 fp32 rows")


def test_d128_full_size_sampled(lib):
    """The 1024^2 dense launch at head dim 128 (the benchmark's d = 128 line) and its rows launch, on
    sampled rows."""
    w = syn.WORKLOADS["dense_1024_d128"]
    t = torch()
    inp = syn.attention_inputs(w)
    q, ki, vi, kt, vt = attn_tensors(inp, w.dtype)
    out = t.zeros_like(q)
    lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, out)
    sample = syn.sample_rows(w.N, 24, seed=w.seed)
    t.cuda.synchronize()
    got = host(out[:, :, t.as_tensor(sample, device="cuda")])
    ro, _ = OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], w.tv, rows=sample)
    assert_close(got, ro, "bf16", "dense_1024_d128")
    rows = syn.random_rows(w)
    out2 = t.zeros_like(q)
    lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, dev(rows), out2)
    t.cuda.synchronize()
    checked = rows[syn.sample_rows(len(rows), 24, seed=w.seed)]
    got = host(out2[:, :, t.as_tensor(checked, device="cuda")])
    ro, _ = OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], w.tv, rows=checked)
    assert_close(got, ro, "bf16", "rows d128")
