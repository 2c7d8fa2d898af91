"""Seeded random sweep of the HBM-bound stages against the fp64 oracle: the exact top-|S| partition (random N on
both sides of the register-resident path's limit, random k, continuous, tied, signed and NaN scores; bit-exact), PCSP
aggregation (random H, N, T, valid text length and content range, with and without the image lse and accumulation),
SW-CFG (random latent and token grids) and the elision check (random mask shapes, near-constant rows)."""
import numpy as np
import pytest

from oracle import elision as OE
from oracle import pcsp as OP
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
