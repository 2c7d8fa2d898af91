"""GPU parity of the attention entry points against the fp64 oracle (dense anchor, sensitive rows)."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as OA
from oracle import pcsp as OP
from tests.gpu_util import assert_close, attn_tensors, dev, err, host, torch

pytestmark = pytest.mark.gpu


def _run(lib, w, inp, rows=None, state=None, emission=False, mask=None, want_lse=True):
    t = torch()
    q, ki, vi, kt, vt = attn_tensors(inp, w.dtype)
    out = t.from_numpy(state).to(q.dtype).cuda() if state is not None else t.zeros_like(q)
    lse = t.full((w.B, w.H, w.N), float("nan"), dtype=t.float32, device="cuda") if want_lse else None
    xo = t.full((w.H, w.N, w.T), float("nan"), dtype=t.float32, device="cuda") if emission else None
    li = t.full((w.H, w.N), float("nan"), dtype=t.float32, device="cuda") if emission else None
    if rows is None:
        lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, out, mask=mask, lse=lse, xattn_out=xo, lse_img_out=li)
    else:
        lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, dev(rows.astype(np.int32)), out, mask=mask, lse=lse,
                           xattn_out=xo, lse_img_out=li)
    t.cuda.synchronize()
    return host(out), (host(lse) if want_lse else None), (host(xo) if emission else None), (host(li) if emission else None)


def _oracle(w, inp, rows=None, mask=None, emission=False):
    return OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], w.tv, rows=rows,
                        mask=mask, want_emission=emission)


# ---------------------------------------------------------------- tiny fp32 SRSU workload (16x16 grid)
def test_tiny_f32_dense_rows_and_pcsp(lib):
    w = syn.WORKLOADS["tiny_srsu_f32"]
    inp = syn.attention_inputs(w)
    o, lse, x, lse_img = _run(lib, w, inp, emission=True)
    ro, rlse, rx, rli = _oracle(w, inp, emission=True)
    assert_close(o, ro, "f32", "dense")
    assert np.max(np.abs(lse - rlse)) < 1e-5
    assert np.max(np.abs(x[:, :, : w.tv[0]] - rx)) < 1e-5
    assert np.max(np.abs(lse_img - rli)) < 1e-5
    # PCSP on the real warmup logits, content = the valid text slots, |S| = 64
    t = torch()
    scores = t.zeros(w.N, dtype=t.float32, device="cuda")
    lib.safe_pcsp_accumulate(dev(x.astype(np.float32)), dev(lse_img.astype(np.float32)), w.tv[0], 0, w.tv[0],
                             scores, False)
    S_d = t.zeros(w.k, dtype=t.int32, device="cuda")
    C_d = t.zeros(w.N - w.k, dtype=t.int32, device="cuda")
    is_d = t.zeros(w.N, dtype=t.uint8, device="cuda")
    lib.safe_pcsp_partition(scores, w.k, S_d, C_d, is_d)
    a_gpu = host(scores).astype(np.float64)
    a_ref = OP.scores(rx, rli, w.tv[0], 0, w.tv[0])
    assert np.max(np.abs(a_gpu - a_ref) / a_ref) < 1e-5
    S_ref = OP.partition(a_ref, w.k)[0]
    o_ = OP.order(a_ref)
    margin = (a_ref[o_[w.k - 1]] - a_ref[o_[w.k]]) / a_ref[o_[w.k - 1]]
    rel_err = float(np.max(np.abs(a_gpu - a_ref) / a_ref))
    S = host(S_d)
    assert np.array_equal(S, OP.partition(a_gpu, w.k)[0])  # exact on the GPU's own scores
    # The end-to-end partition equals the fp64 one when the fp64 boundary margin exceeds 10x the measured fp32
    # score error; a seed below that is ill-conditioned at the boundary and is reported as such, never passed
    # silently (this workload's seed is screened on the CPU: margin 3.6e-5 against errors of a few 1e-7).
    assert margin > 10 * rel_err, f"ill-conditioned boundary: margin {margin:.2e}, fp32 score error {rel_err:.2e}"
    assert np.array_equal(S, S_ref)
    # sensitive rows into a stale state; |S| = N equals dense
    state = syn.initial_state(w)
    o2, _, _, _ = _run(lib, w, inp, rows=S, state=state)
    C = np.setdiff1d(np.arange(w.N), S)
    assert np.array_equal(o2[:, :, C], state[:, :, C].astype(np.float64))
    assert_close(o2[:, :, S], ro[:, :, S], "f32", "rows")
    o3, _, _, _ = _run(lib, w, inp, rows=np.arange(w.N, dtype=np.int32), state=state)
    assert np.array_equal(o3, o)


def test_tiny_f32_masks_are_elided_and_kept_path_agrees(lib):
    w = syn.WORKLOADS["tiny_srsu_f32"]
    inp = syn.attention_inputs(w)
    t = torch()
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    zeros = dev(syn.mask_zeros_f32(w.N, w.N))
    rc = syn.mask_row_constant_f32(w, w.N + w.T)
    assert lib.safe_mask_is_row_constant(zeros, w.N, w.T, w.tv, flag)
    assert lib.safe_mask_is_row_constant(dev(rc), w.N, w.T, w.tv, flag)
    # the kept path applies the row-constant mask exactly and agrees with the mask-free result
    o_free, _, _, _ = _run(lib, w, inp)
    o_kept, lse_kept, _, _ = _run(lib, w, inp, mask=dev(rc))
    ro, rlse = _oracle(w, inp, mask=rc)
    assert_close(o_kept, ro, "f32", "kept row-constant")
    assert_close(o_free, ro, "f32", "elided row-constant")
    assert np.max(np.abs(lse_kept - rlse)) < 1e-4


# ---------------------------------------------------------------- bf16 MFMA path, shapes spanning tiles
SHAPES = [
    # (B, H, N, T, tv)
    (1, 1, 1, 0, (0,)),
    (1, 2, 64, 64, (64,)),
    (2, 3, 65, 40, (17, 0)),
    (2, 2, 127, 256, (77, 1)),
    (1, 2, 300, 256, (65,)),
    (2, 2, 1000, 256, (200, 63)),
]


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dT%d" % s[:4])
def test_bf16_dense_parity(lib, shape, want_lse):
    """Both row-sum forms: fp32 sum when lse is requested, bf16-probability sum otherwise."""
    B, H, N, T, tv = shape
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=B, H=H, N=N, T=T, tv=tv, side=1)
    inp = syn.attention_inputs(w)
    o, lse, _, _ = _run(lib, w, inp, want_lse=want_lse)
    ro, rlse = _oracle(w, inp)
    assert_close(o, ro, "bf16", f"dense {shape}")
    if want_lse:
        assert np.max(np.abs(lse - rlse)) < 1e-4


@pytest.mark.parametrize("k", [0, 1, 63, 64, 65, 129, 300])
def test_bf16_rows_parity_and_untouched_context(lib, k):
    w = syn.scaled(syn.WORKLOADS["srsu_1024"], B=2, H=3, N=300, T=256, tv=(77, 5), side=1)
    inp = syn.attention_inputs(w)
    rows = syn.random_rows(w, k=k)
    state = syn.initial_state(w)
    o, _, _, _ = _run(lib, w, inp, rows=rows, state=state, want_lse=(k % 2 == 1))
    C = np.setdiff1d(np.arange(w.N), rows)
    assert np.array_equal(o[:, :, C], state[:, :, C].astype(np.float64))
    if k:
        ro, _ = _oracle(w, inp, rows=rows)
        assert_close(o[:, :, rows], ro, "bf16", f"rows k={k}")
    if k == w.N:
        od, _, _, _ = _run(lib, w, inp, want_lse=False)
        assert np.array_equal(o, od)


@pytest.mark.parametrize("B,H,N,T,tv,k", [
    (1, 8, 2000, 256, (77,), None),         # few two-block waves: one block per wave, key range in two halves
    (2, 8, 2304, 256, (120, 3), None),      # 576 two-block waves: two blocks per wave, key halves
    (2, 8, 4096, 64, (64, 64), None),       # 1024 two-block waves: the largest split case
    (2, 8, 4160, 256, (77, 0), None),       # 1040: one block per wave, no split
    (2, 24, 4096, 256, (77, 77), 1229),     # the 1024^2 rows launch: two blocks per wave, key halves, gathered
    (1, 3, 193, 0, (0,), None),             # 4 key tiles: halves of 2 and 2 (ragged tail in the second)
    (1, 3, 130, 0, (0,), None),             # 3 key tiles: the second half passes one extra barrier
])
def test_bf16_key_split_dispatch_parity(lib, B, H, N, T, tv, k):
    """Every work shape of the mask-free fast path (one or two query blocks per wave, with or without the
    key range split across two halves of a workgroup) against the oracle, element by element."""
    w = syn.scaled(syn.WORKLOADS["srsu_1024"], B=B, H=H, N=N, T=T, tv=tv, side=1)
    inp = syn.attention_inputs(w)
    if k is None:
        o, _, _, _ = _run(lib, w, inp, want_lse=False)
        ro, _ = _oracle(w, inp)
        assert_close(o, ro, "bf16", f"dense B{B}H{H}N{N}")
    else:
        rows = syn.random_rows(w, k=k)
        state = syn.initial_state(w)
        o, _, _, _ = _run(lib, w, inp, rows=rows, state=state, want_lse=False)
        ro, _ = _oracle(w, inp, rows=rows)
        assert_close(o[:, :, rows], ro, "bf16", f"rows B{B}H{H}N{N}k{k}")
        C = np.setdiff1d(np.arange(w.N), rows)
        assert np.array_equal(o[:, :, C], state[:, :, C].astype(np.float64))


def test_bf16_padding_contents_never_leak(lib):
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=2, N=200, T=256, tv=(77, 3), side=1)
    inp = syn.attention_inputs(w)
    o1, _, _, _ = _run(lib, w, inp)
    poisoned = dict(inp)
    for r in ("k_txt", "v_txt"):
        bits = inp[r + "_bits"].copy()
        bits[0, :, 77:] = 0x7FC0  # NaN
        bits[1, :, 3:] = 0x7F80   # +inf
        poisoned[r + "_bits"] = bits
    o2, _, _, _ = _run(lib, w, poisoned)
    assert np.array_equal(o1, o2)


def test_bf16_closed_forms(lib):
    t = torch()
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=2, N=257, T=256, tv=(77, 0), side=1)
    inp = syn.attention_inputs(w)
    one = np.full_like(inp["v_img_bits"], 0x3F80)  # 1.0
    ones = dict(inp, v_img_bits=one, v_txt_bits=np.full_like(inp["v_txt_bits"], 0x3F80))
    o, _, _, _ = _run(lib, w, ones, want_lse=False)
    assert np.max(np.abs(o - 1.0)) <= 1e-6  # the row sum uses the same bf16 probabilities as P V
    o, _, _, _ = _run(lib, w, ones)
    assert np.max(np.abs(o - 1.0)) <= 2e-2
    zq = dict(inp, q_bits=np.zeros_like(inp["q_bits"]))
    o, lse, _, _ = _run(lib, w, zq)
    for b in range(2):
        vals = np.concatenate([inp["v_img"][b], inp["v_txt"][b, :, : w.tv[b]]], axis=1).astype(np.float64)
        mean = vals.mean(axis=1)
        assert_close(o[b], np.broadcast_to(mean[:, None, :], o[b].shape), "bf16", "Q = 0: mean of the valid V rows")
        assert np.max(np.abs(lse[b] - np.log(w.N + w.tv[b]))) < 1e-3


@pytest.mark.parametrize("std", [1.0, 3.0])
def test_bf16_large_logits_exercise_rescaling(lib, std):
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=1, H=2, N=513, T=256, tv=(100,), side=1, std=std)
    inp = dict(syn.attention_inputs(w))
    for r in ("v_img", "v_txt"):  # values back at the workloads' scale (0.125); logits std = 8 * std^2 / 8
        v = (inp[r] * np.float32(0.125 / std)).astype(np.float32)
        inp[r], inp[r + "_bits"] = syn.round_to_bf16(v), syn.f32_to_bf16_bits(v)
    o, lse, _, _ = _run(lib, w, inp)
    ro, rlse = _oracle(w, inp)
    assert_close(o, ro, "bf16", f"std={std}")
    assert np.max(np.abs(lse - rlse)) < 2e-2 * max(1.0, std * std)


def test_bf16_late_spike_key(lib):
    """The last valid text key dominates every row: the running max jumps in the last tile."""
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=1, H=1, N=640, T=256, tv=(40,), side=1)
    inp = syn.attention_inputs(w)
    q = inp["q"] + np.float32(0.5)  # common component u = 0.5 in every query row
    kt = inp["k_txt"].copy()
    kt[0, 0, 39] = 5.0              # key 10*u: logit ~ 0.125 * 10 * 16 = 20 for every row
    spiked = dict(inp, q=syn.round_to_bf16(q), q_bits=syn.f32_to_bf16_bits(q),
                  k_txt=syn.round_to_bf16(kt), k_txt_bits=syn.f32_to_bf16_bits(kt))
    o, _, _, _ = _run(lib, w, spiked)
    ro, _ = _oracle(w, spiked)
    assert_close(o, ro, "bf16", "spike")


def test_bf16_deterministic(lib):
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=2, N=700, T=256, tv=(77, 77), side=1)
    inp = syn.attention_inputs(w)
    a, la, _, _ = _run(lib, w, inp)
    b, lb, _, _ = _run(lib, w, inp)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_bf16_emission_matches_oracle(lib):
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=3, N=333, T=256, tv=(77, 20), side=1)
    inp = syn.attention_inputs(w)
    _, _, x, li = _run(lib, w, inp, emission=True)
    _, _, rx, rli = _oracle(w, inp, emission=True)
    assert np.max(np.abs(x[:, :, :77] - rx)) < 1e-5
    assert np.max(np.abs(li - rli)) < 1e-4


def test_bf16_kept_masks(lib):
    """Non-removable masks (bool image mask, fp32 bias over image+text) are applied exactly."""
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=2, N=150, T=64, tv=(30, 64), side=1)
    inp = syn.attention_inputs(w)
    r = np.random.default_rng(0)
    bm = r.random((1, 2, w.N, w.N)) < 0.7
    bm[..., 0] = True
    o, _, _, _ = _run(lib, w, inp, mask=dev(bm))
    ro, _ = _oracle(w, inp, mask=bm)
    assert_close(o, ro, "bf16", "bool mask")
    fm = (r.standard_normal((2, 1, w.N, w.N + w.T)) * 2).astype(np.float32)
    o, _, _, _ = _run(lib, w, inp, mask=dev(fm), rows=np.array([0, 5, 149], dtype=np.int32),
                      state=np.zeros((2, 2, w.N, 64), np.float32))
    ro, _ = _oracle(w, inp, mask=fm, rows=np.array([0, 5, 149]))
    assert_close(o[:, :, [0, 5, 149]], ro, "bf16", "fp32 mask rows")
    # a fully masked row gives zeros
    bm2 = np.ones((1, 1, w.N, w.N), dtype=bool)
    bm2[0, 0, 7] = False
    w0 = syn.scaled(w, tv=(0, 0))
    o, lse, _, _ = _run(lib, w0, inp, mask=dev(bm2))
    assert np.all(o[:, :, 7] == 0) and np.all(np.isneginf(lse[:, :, 7]))


# ---------------------------------------------------------------- full-size workloads, sampled rows
@pytest.mark.parametrize("name", ["dense_1024", "srsu_1024", "srsu_2560", "traj_3072"])
def test_full_size_sampled(lib, name):
    """The launch configuration the benchmark times, checked on sampled rows against the oracle."""
    w = syn.WORKLOADS[name]
    t = torch()
    inp = syn.attention_inputs(w)
    q, ki, vi, kt, vt = attn_tensors(inp, w.dtype)
    sample = syn.sample_rows(w.N, 24, seed=w.seed)
    out = t.zeros_like(q)
    if name == "dense_1024":
        lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, out)
        rows_checked = sample
    else:
        rows = syn.random_rows(w)
        lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, dev(rows), out)
        rows_checked = rows[syn.sample_rows(len(rows), 24, seed=w.seed)]
        # untouched context rows stay zero
        C = np.setdiff1d(np.arange(w.N), rows)[:64]
        assert t.count_nonzero(out[:, :, t.as_tensor(C, device="cuda")]).item() == 0
    t.cuda.synchronize()
    got = host(out[:, :, t.as_tensor(rows_checked, device="cuda")])
    ro, _ = OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], w.tv, rows=rows_checked)
    assert_close(got, ro, "bf16", name)


# ---------------------------------------------------------------- kept masks on the MFMA kernel
def _kept_mask(r, kind, shape, n_img, tv_max, full_rows=()):
    """A non-removable mask: bool with ~40% False, or fp32 N(0, 2) with ~10% -inf; the listed rows are
    fully masked over every column (image and text)."""
    if kind == "bool":
        m = r.random(shape) < 0.6
        m[..., 0] = True
        for i in full_rows:
            m[..., i, :] = False
    else:
        m = (r.standard_normal(shape) * 2).astype(np.float32)
        m[r.random(shape) < 0.1] = -np.inf
        m[..., 0] = 0.0
        for i in full_rows:
            m[..., i, :] = -np.inf
    return m


@pytest.mark.parametrize("N,T,tv,kind,text_cols,mB,mH,want_lse", [
    (256, 64, (30, 64), "bool", True, 1, 1, False),
    (256, 64, (30, 64), "bool", False, 2, 3, True),
    (448, 256, (77, 20), "f32", True, 2, 1, False),
    (448, 256, (77, 20), "f32", False, 1, 3, True),
    (320, 32, (0, 32), "bool", True, 2, 3, True),
])
def test_bf16_kept_mask_on_mfma_kernel(lib, N, T, tv, kind, text_cols, mB, mH, want_lse):
    """Masks with N and the row length multiples of 16 run on the MFMA kernel: dense and gathered rows
    match the oracle, fully masked rows give 0 and lse = -inf, an image-only mask leaves text unmasked."""
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=3, N=N, T=T, tv=tv, side=1)
    inp = syn.attention_inputs(w)
    r = np.random.default_rng(N + T + mB + mH)
    cols = N + T if text_cols else N
    full = (5, N - 1) if text_cols else ()
    m = _kept_mask(r, kind, (mB, mH, N, cols), N, max(tv), full_rows=full)
    o, lse, _, _ = _run(lib, w, inp, mask=dev(m), want_lse=want_lse)
    ro, rlse = _oracle(w, inp, mask=m)
    assert_close(o, ro, "bf16", "dense kept mask")
    if want_lse:
        fin = np.isfinite(rlse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-4
    for i in full:
        assert np.all(o[:, :, i] == 0)
    rows = np.array(sorted({0, 1, 5, 17, N // 2, N - 1}), dtype=np.int32)
    state = np.full((w.B, w.H, N, 64), 0.25, np.float32)
    o, _, _, _ = _run(lib, w, inp, mask=dev(m), rows=rows, state=state, want_lse=False)
    ro, _ = _oracle(w, inp, mask=m, rows=rows)
    assert_close(o[:, :, rows], ro, "bf16", "rows kept mask")
    untouched = np.setdiff1d(np.arange(N), rows)
    assert np.all(o[:, :, untouched] == 0.25)


def test_bf16_kept_mask_late_first_valid_key(lib):
    """Rows whose first unmasked key comes after several fully masked tiles (the running max stays -inf
    over those tiles) and rows that are masked except for one text key."""
    w = syn.scaled(syn.WORKLOADS["dense_1024"], B=2, H=2, N=512, T=64, tv=(64, 10), side=1)
    inp = syn.attention_inputs(w)
    m = np.zeros((1, 1, w.N, w.N + w.T), dtype=bool)
    m[0, 0, :, 300:] = True          # first 4 image tiles masked for every row, rest attends
    m[0, 0, 7, :] = False
    m[0, 0, 7, w.N + 3] = True       # row 7: only text key 3
    for want_lse in (False, True):
        o, lse, _, _ = _run(lib, w, inp, mask=dev(m), want_lse=want_lse)
        ro, rlse = _oracle(w, inp, mask=m)
        assert_close(o, ro, "bf16", "late first key")
        if want_lse:
            assert np.max(np.abs(lse - rlse)) < 1e-4


def test_bf16_kept_mask_full_size_sampled(lib):
    """The 1024^2 shape with a random bool image mask: sampled rows against the oracle."""
    w = syn.WORKLOADS["dense_1024"]
    t = torch()
    inp = syn.attention_inputs(w)
    q, ki, vi, kt, vt = attn_tensors(inp, w.dtype)
    r = np.random.default_rng(7)
    m = r.random((1, 1, w.N, w.N)) < 0.8
    out = t.zeros_like(q)
    lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, out, mask=dev(m))
    t.cuda.synchronize()
    sample = syn.sample_rows(w.N, 16, seed=3)
    sl = lambda a: a[:, :2]
    ro, _ = OA.attention(sl(inp["q"]), sl(inp["k_img"]), sl(inp["v_img"]), sl(inp["k_txt"]), sl(inp["v_txt"]), w.tv,
                         rows=sample, mask=m)
    got = host(out)[:, :2][:, :, sample]
    assert_close(got, ro, "bf16", "1024^2 kept bool mask")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,k", [(3, 6), (24, 1229)])
def test_rows_entries_outside_range_are_skipped(lib, d, H, k):
    """Row entries outside [0, N) write nothing and every valid entry is computed (the contract of
    safe_attn_rows), on the few-row and the many-row work shapes."""
    w = syn.scaled(syn.WORKLOADS["srsu_1024"], B=2, H=H, N=1000 if H == 3 else 4096, T=256, tv=(77, 9), side=1,
                   d=d)
    inp = syn.attention_inputs(w)
    r = np.random.default_rng(k + d)
    valid = np.sort(r.choice(w.N, size=k - 4, replace=False)).astype(np.int32)
    rows = np.concatenate([[-5, -1], valid, [w.N, w.N + 1000]]).astype(np.int32)
    state = syn.initial_state(w)
    o, _, _, _ = _run(lib, w, inp, rows=rows, state=state, want_lse=False)
    C = np.setdiff1d(np.arange(w.N), valid)
    assert np.array_equal(o[:, :, C], state[:, :, C].astype(np.float64))
    pick = valid if len(valid) <= 64 else valid[syn.sample_rows(len(valid), 64, seed=d)]
    ro, _ = _oracle(w, inp, rows=pick)
    assert_close(o[:, :, pick], ro, "bf16", f"rows with out-of-range entries d={d} H={H}")
