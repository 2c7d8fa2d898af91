"""Seeded random sweep of the HBM-bound stages against the fp64 oracle: the exact top-|S| partition (random N on
both sides of the register-resident path's limit, random k, continuous, tied, signed and NaN scores; bit-exact), PCSP
aggregation and the AesMask affinity (random H, N, T, valid text length, content range or slot selection, with and
without the image lse and accumulation), SW-CFG (random scales, latent and token grids), the elision check (random
mask shapes, near-constant rows), the row gather / scatter (random shapes and row sets; bit-exact) and the StepCache
extrapolation (random lengths, offsets and weights)."""
import numpy as np
import pytest

from oracle import aesmask as OAM
from oracle import attention as OA
from oracle import elision as OE
from oracle import pcsp as OP
from oracle import stepcache as OSC
from tests.gpu_util import dev, host, torch
from tests.test_gpu_aesmask_stepcache import _affinity
from tests.test_gpu_misc import _cfg, _cfg_check, _check, _same
from tests.test_gpu_pcsp import _accumulate, _check_exact

pytestmark = pytest.mark.gpu

N_CASES = 12


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_partition_is_exact(lib, i):
    r = np.random.default_rng(5000 + i)
    N = int(r.choice([int(r.integers(1, 5000)), int(r.integers(5000, 40960)), int(r.integers(40961, 90000))]))
    kind = i % 4
    if kind == 0:
        a = r.random(N).astype(np.float32)
    elif kind == 1:
        a = (r.integers(0, int(r.integers(1, 50)), N) / 8.0).astype(np.float32)  # many ties
    elif kind == 2:
        a = (r.standard_normal(N) * 10).astype(np.float32)
        a[r.random(N) < 0.02] = np.nan
    else:
        a = (r.standard_normal(N) * 1e-3 + 7.0).astype(np.float32)  # a narrow range: many shared high bits
    for k in sorted({0, 1, int(r.integers(0, N + 1)), N // 5, N}):
        _check_exact(lib, a, k)


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_pcsp_accumulate(lib, i):
    r = np.random.default_rng(6000 + i)
    H = int(r.integers(1, 30))
    N = int(r.integers(1, 3000))
    T = int(r.choice([1, 8, 37, 77, 128, 256, 300]))
    tv = int(r.integers(0, T + 1))
    c0 = int(r.integers(0, tv + 1))
    c1 = int(r.integers(c0, tv + 1))
    x = (r.standard_normal((H, N, T)) * float(r.choice([0.5, 2.0, 6.0]))).astype(np.float32)
    li = (r.standard_normal((H, N)) + 4).astype(np.float32)
    for lse_img in (li, None):
        got = _accumulate(lib, x, lse_img, tv, c0, c1)
        ref = OP.scores(x, lse_img, tv, c0, c1)
        assert np.all(np.abs(got - ref) <= 5e-6 * np.abs(ref) + 1e-37), (i, H, N, T, tv, c0, c1, lse_img is None)
    prev = r.random(N).astype(np.float32)
    got = _accumulate(lib, x, li, tv, c0, c1, prev=prev)
    ref = prev.astype(np.float64) + OP.scores(x, li, tv, c0, c1)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-30)) < 5e-6, i


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_swcfg(lib, i):
    r = np.random.default_rng(7500 + i)
    side = int(r.integers(1, 80))
    C = int(r.integers(1, 17))
    Hl, Wl = side * int(r.integers(1, 4)), side * int(r.integers(1, 4))
    eps = r.standard_normal((2, C, Hl, Wl)).astype(np.float32)
    s = r.random(side * side).astype(np.float32)
    gc, gs = float(r.uniform(0, 8)), float(r.uniform(0, 8))
    _cfg_check(_cfg(lib, eps, s, side, gc, gs), eps, s.astype(np.float64), side, gc, gs)


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_mask_check(lib, i):
    r = np.random.default_rng(8500 + i)
    N = int(r.integers(1, 400))
    T = int(r.integers(0, 80))
    B = int(r.integers(1, 4))
    tv = tuple(int(x) for x in r.integers(0, T + 1, size=B))
    mB, mH = int(r.choice([1, B])), int(r.integers(1, 4))
    cols = int(r.choice([N, N + T]))
    if i % 2 == 0:
        m = r.random((mB, mH, N, cols)) < float(r.choice([0.999, 1.0]))
    else:
        m = np.broadcast_to(r.integers(-2, 3, size=(mB, mH, N, 1)).astype(np.float32), (mB, mH, N, cols)).copy()
        if cols == N and max(tv) > 0:
            m[:, :, : N // 2] = 0.0  # rows that stay removable beside the implicit zero text block
        for _ in range(int(r.integers(0, 3))):
            m[tuple(int(r.integers(0, s)) for s in m.shape)] = r.choice([np.nan, np.inf, -np.inf, 0.5, -0.0])
    ok, c = _check(lib, m, N, T, tv)
    rok, rc = OE.is_row_constant(m, N, T, tv)
    assert ok == rok and _same(c, rc), (i, m.shape, tv)
    ok2, _ = _check(lib, m, N, T, tv, want_c=False)
    assert ok2 == rok, i


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_affinity(lib, i):
    r = np.random.default_rng(9500 + i)
    H, N = int(r.integers(1, 30)), int(r.integers(1, 3000))
    T = int(r.choice([1, 8, 37, 77, 128, 256, 300]))
    tv = int(r.integers(0, T + 1))
    x = (r.standard_normal((H, N, T)) * 2).astype(np.float32)
    x[:, :, tv:] = 1e30  # padded slots must never count
    li = (r.standard_normal((H, N)) + 4).astype(np.float32)
    sel = (r.random(T) < float(r.uniform(0, 1))).astype(np.uint8)
    off = int(r.choice([0, 0, 1, 3]))
    for lse_img in (li, None):
        got = _affinity(lib, x, lse_img, tv, sel, sel_offset=off)
        ref = OAM.affinity(x, lse_img, tv, sel)
        assert np.all(np.abs(got - ref) <= 5e-6 * np.abs(ref) + 1e-37), (i, H, N, T, tv, off, lse_img is None)


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_gather_scatter(lib, i):
    t = torch()
    r = np.random.default_rng(10500 + i)
    dtype = ["bf16", "f32"][i % 2]
    unit = 8 if dtype == "bf16" else 4  # 16-byte rows
    B, H, N = int(r.integers(1, 4)), int(r.integers(1, 30)), int(r.integers(1, 2000))
    d = unit * int(r.integers(1, 33))
    k = int(r.integers(0, N + 1))
    tdt = t.bfloat16 if dtype == "bf16" else t.float32
    state = t.from_numpy(r.standard_normal((B, H, N, d)).astype(np.float32)).to(tdt).cuda()
    rows = np.sort(r.choice(N, size=k, replace=False)).astype(np.int32)
    rows_d = dev(rows)
    packed = t.zeros((B, H, k, d), dtype=tdt, device="cuda")
    lib.safe_gather_rows(state, rows_d, packed)
    ref = state.float().cpu().numpy()
    canvas = t.full_like(state, 7.0)
    lib.safe_scatter_rows(packed, rows_d, canvas)
    t.cuda.synchronize()
    assert np.array_equal(packed.float().cpu().numpy(), OA.gather_rows(ref, rows)), (i, B, H, N, d, k)
    expect = OA.scatter_rows(np.full(ref.shape, 7.0, dtype=np.float32), OA.gather_rows(ref, rows), rows)
    assert np.array_equal(canvas.float().cpu().numpy(), expect), (i, B, H, N, d, k)


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_stepcache(lib, i):
    t = torch()
    r = np.random.default_rng(11500 + i)
    n = int(r.integers(0, 300000))
    offset = int(r.choice([0, 0, 1, 2, 3]))
    w = float(np.float32(r.uniform(-2, 3)))
    a = r.standard_normal(n + offset).astype(np.float32)
    b = (a + 0.1 * r.standard_normal(n + offset)).astype(np.float32)
    out = t.full((n + offset,), np.nan, dtype=t.float32, device="cuda")[offset:]
    lib.safe_stepcache_extrapolate(dev(a)[offset:], dev(b)[offset:], w, out)
    t.cuda.synchronize()
    got = host(out).astype(np.float64)
    ref = OSC.extrapolate(a[offset:], b[offset:], np.float32(w))
    scale = np.abs(b[offset:]) + abs(w) * np.abs(b[offset:].astype(np.float64) - a[offset:])
    assert np.all(np.abs(got - ref) <= 1e-6 * scale + 1e-37), (i, n, offset, w)
