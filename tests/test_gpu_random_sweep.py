"""Seeded random sweep of the attention entry points against the fp64 oracle: each case draws the dtype (bf16,
fp32, fp8 Q / K), head dim, B, H, N, T, a text length per batch entry, dense or sensitive rows (with entries outside
[0, N) mixed in), a kept mask of any accepted layout (bool or fp32, per batch / per head or shared, image-only or
image + text columns, with fully masked rows), lse, the warmup emission, the logit scale and the logit magnitude.
The cases land on every kernel and work shape the dispatch chooses among; each is compared element by element."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as OA
from tests.gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

N_CASES = 96


def _case(i):
    r = np.random.default_rng(9000 + i)
    c = {}
    c["dtype"] = ["bf16", "f32", "fp8"][r.choice(3, p=[0.5, 0.2, 0.3])]
    c["d"] = int(r.choice([64, 128]))
    c["B"] = int(r.integers(1, 4))
    c["H"] = int(r.integers(1, 4))
    c["N"] = int([r.integers(1, 700), 16 * r.integers(1, 40), 64 * r.integers(1, 9)][r.integers(0, 3)])
    c["T"] = int(r.choice([0, 8, 77, 128, 256, 300, 1000]))
    c["tv"] = tuple(int(x) for x in r.integers(0, c["T"] + 1, size=c["B"]))
    c["rows"] = bool(r.random() < 0.5)
    c["k"] = int(r.integers(0, c["N"] + 1)) if c["rows"] else 0
    c["outside"] = bool(c["rows"] and r.random() < 0.3)
    c["mask"] = [None, "bool", "f32"][r.choice(3, p=[0.5, 0.25, 0.25])]
    c["mB"] = int(r.choice([1, c["B"]]))
    c["mH"] = int(r.choice([1, c["H"]]))
    c["text_cols"] = bool(r.random() < 0.5)
    c["lse"] = bool(r.random() < 0.5)
    c["emission"] = bool(r.random() < 0.3)
    c["scale"] = float(r.choice([0.0, 0.07, 0.3]))
    c["amp"] = float(r.choice([1.0, 4.0, 16.0]))
    c["seed"] = 9000 + i
    return c


def _mask(c, r):
    N, T = c["N"], c["T"]
    cols = N + T if c["text_cols"] else N
    shape = (c["mB"], c["mH"], N, cols)
    full = [i for i in (0, N // 3, N - 1) if r.random() < 0.5]
    if c["mask"] == "bool":
        m = r.random(shape) < 0.65
        m[..., min(1, N - 1)] = True
        for i in full:
            m[..., i, :] = False
    else:
        m = (r.standard_normal(shape) * 2).astype(np.float32)
        m[r.random(shape) < 0.1] = -np.inf
        m[..., min(1, N - 1)] = 0.0
        for i in full:
            m[..., i, :] = -np.inf
    return m


def _fp8(codes):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(codes)).view(t.float8_e4m3fn).cuda()


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_case_matches_oracle(lib, i):
    c = _case(i)
    t = torch()
    r = np.random.default_rng(c["seed"] + 1)
    wdt = "f32" if c["dtype"] == "f32" else "bf16"
    w = syn.scaled(syn.WORKLOADS["dense_1024"], side=1, B=c["B"], H=c["H"], N=c["N"], T=c["T"], tv=c["tv"],
                   d=c["d"], dtype=wdt, seed=c["seed"])
    extra = {}
    if c["dtype"] == "fp8":
        inp = syn.attention_inputs_fp8(w)
        # the logit magnitude through the Q factors (the codes stay the same)
        qd = (inp["q_descale"] * np.float32(c["amp"])).astype(np.float32)
        inp["q"] = inp["q"] / inp["q_descale"][:, :, None, None].astype(np.float64) * qd[:, :, None, None]
        q, ki, kt = _fp8(inp["q_fp8"]), _fp8(inp["k_img_fp8"]), _fp8(inp["k_txt_fp8"])
        vi, vt = dev(None, inp["v_img_bits"]), dev(None, inp["v_txt_bits"])
        extra = dict(q_descale=dev(qd.reshape(-1)), k_descale=dev(inp["k_descale"].reshape(-1)))
    else:
        inp = syn.attention_inputs(w)
        qa = inp["q"] * np.float32(c["amp"])
        if wdt == "bf16":
            inp["q"], inp["q_bits"] = syn.round_to_bf16(qa), syn.f32_to_bf16_bits(qa)
            q, ki, vi, kt, vt = (dev(None, inp[n + "_bits"]) for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
        else:
            inp["q"] = qa
            q, ki, vi, kt, vt = (dev(inp[n]) for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
    m = _mask(c, r) if c["mask"] else None
    N, T, B, H, d = c["N"], c["T"], c["B"], c["H"], c["d"]
    odt = t.float32 if wdt == "f32" else t.bfloat16
    state = syn.initial_state(w)
    out = t.from_numpy(state.astype(np.float32)).to(odt).cuda()
    lse = t.full((B, H, N), float("nan"), dtype=t.float32, device="cuda") if c["lse"] else None
    xo = t.full((H, N, T), float("nan"), dtype=t.float32, device="cuda") if c["emission"] else None
    li = t.full((H, N), float("nan"), dtype=t.float32, device="cuda") if c["emission"] else None
    kw = dict(scale=c["scale"], mask=dev(m) if m is not None else None, lse=lse, xattn_out=xo, lse_img_out=li, **extra)
    if c["rows"]:
        rows = np.sort(r.choice(N, size=c["k"], replace=False)).astype(np.int32)
        call_rows = rows
        if c["outside"]:  # entries outside [0, N) at both ends, keeping the call's k <= N
            room = N - len(rows)
            lo, hi = [-3, -1][: (room + 1) // 2], [N, N + 7][: room // 2]
            call_rows = np.concatenate([lo, rows, hi]).astype(np.int32)
        lib.safe_attn_rows(q, ki, vi, kt, vt, c["tv"], dev(call_rows), out, **kw)
    else:
        rows = np.arange(N, dtype=np.int32)
        lib.safe_attn_dense(q, ki, vi, kt, vt, c["tv"], out, **kw)
    t.cuda.synchronize()
    o = host(out)
    what = f"case{i} {c}"
    untouched = np.setdiff1d(np.arange(N), rows)
    assert np.array_equal(o[:, :, untouched], state[:, :, untouched].astype(np.float64)), what
    if len(rows) == 0:
        return
    ro, rlse, *em = OA.attention(inp["q"], inp["k_img"], inp["v_img"], inp["k_txt"], inp["v_txt"], c["tv"],
                                 rows=rows, scale=c["scale"], mask=m, want_emission=c["emission"])
    tol = "f32" if wdt == "f32" else "bf16"
    assert_close(o[:, :, rows], ro, tol, what)
    # fp8: the matrix instruction sums the products of a code dot product below fp32 precision (a measured
    # property of the instruction), so the logits it yields carry up to 2^-13 of scale * sum_i |q_i k_i|
    sc = c["scale"] if c["scale"] != 0.0 else 1.0 / np.sqrt(d)
    f8 = (lambda a, b: sc * 2.0 ** -13 * np.abs(a) @ np.abs(b).swapaxes(-1, -2)) if c["dtype"] == "fp8" else None
    dead = np.isneginf(rlse)
    assert np.all(o[:, :, rows][dead] == 0), what
    if c["lse"]:
        g = host(lse)[:, :, rows]
        assert np.array_equal(np.isneginf(g), dead), what
        live = ~dead
        bound = (1e-5 if tol == "f32" else 1e-4) * np.maximum(1.0, np.abs(rlse))
        if f8 is not None:  # the lse moves by at most the largest logit error of its row
            keys = [np.concatenate([inp["k_img"][b, h], inp["k_txt"][b, h, : c["tv"][b]]]) for b in range(B) for h in range(H)]
            kmax = np.stack([f8(inp["q"][b, h, rows], keys[b * H + h]).max(axis=1, initial=0.0)
                             for b in range(B) for h in range(H)]).reshape(B, H, len(rows))
            bound = bound + kmax
        assert np.all(np.abs(g[live] - rlse[live]) < bound[live]), what
    if c["emission"]:
        rx, rli = em
        gx = host(xo)[:, rows, : c["tv"][0]]
        fin = np.isfinite(rx)
        assert np.array_equal(np.isfinite(gx), fin) and np.array_equal(gx[~fin], rx[~fin]), what
        bound = 2e-5 * np.maximum(1.0, np.abs(rx))
        if f8 is not None:
            bound = bound + np.stack([f8(inp["q"][0, h, rows], inp["k_txt"][0, h, : c["tv"][0]]) for h in range(H)])
        assert np.all(np.abs(gx[fin] - rx[fin]) < bound[fin]), what
        gl = host(li)[:, rows]
        lfin = np.isfinite(rli)
        assert np.array_equal(np.isfinite(gl), lfin), what
        assert np.max(np.abs(gl[lfin] - rli[lfin]) / np.maximum(1.0, np.abs(rli[lfin])), initial=0.0) < 1e-4, what
