"""GPU parity of PCSP aggregation and the exact top-|S| partition."""
import numpy as np
import pytest

import synthetic as syn
from oracle import pcsp as OP
from tests.gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu


def _partition(lib, a: np.ndarray, k: int, s01=True):
    t = torch()
    N = a.shape[0]
    sc = dev(a.astype(np.float32))
    S = t.full((max(k, 1),), -7, dtype=t.int32, device="cuda")
    C = t.full((max(N - k, 1),), -7, dtype=t.int32, device="cuda")
    isn = t.full((N,), 9, dtype=t.uint8, device="cuda")
    s = t.full((N,), 7.0, dtype=t.float32, device="cuda") if s01 else None
    lib.safe_pcsp_partition(sc, k, S, C, isn, s)
    t.cuda.synchronize()
    return host(S)[:k], host(C)[: N - k], host(isn), (host(s) if s01 else None)


def _check_exact(lib, a32: np.ndarray, k: int):
    S, C, isn, s01 = _partition(lib, a32, k)
    rS, rC, risn, rs = OP.partition(a32.astype(np.float64), k)
    assert np.array_equal(S, rS), "S differs"
    assert np.array_equal(C, rC), "C differs"
    assert np.array_equal(isn, risn)
    fin = ~np.isnan(rs)
    assert np.array_equal(np.isnan(s01), ~fin)
    assert np.max(np.abs(s01[fin] - rs[fin]), initial=0.0) <= 2e-7


@pytest.mark.parametrize("N,k", [(1, 0), (1, 1), (7, 3), (1000, 1), (1000, 999), (4096, 1229), (16384, 8000),
                                 (16385, 16385), (25600, 5120), (36864, 7373), (70000, 12345)])
def test_partition_exact_random(lib, N, k):
    a = np.random.default_rng(N + k).random(N).astype(np.float32)
    _check_exact(lib, a, k)


@pytest.mark.parametrize("N", [3000, 20000])
def test_partition_exact_mixed_signs_and_all_nan(lib, N):
    r = np.random.default_rng(N)
    a = (r.standard_normal(N) * 3).astype(np.float32)
    a[r.integers(0, N, N // 50)] = np.nan
    for k in (1, N // 3, N - 1):
        _check_exact(lib, a, k)
    allnan = np.full(N, np.nan, dtype=np.float32)
    S, C, isn, s = _partition(lib, allnan, 10)
    rS, rC, _, _ = OP.partition(allnan.astype(np.float64), 10)
    assert np.array_equal(S, rS) and np.array_equal(C, rC) and np.all(np.isnan(s))


@pytest.mark.parametrize("levels", [1, 2, 5, 300])
def test_partition_exact_with_ties(lib, levels):
    r = np.random.default_rng(levels)
    N = 5000
    a = (r.integers(0, levels, N) / 4.0).astype(np.float32)
    for k in (0, 1, 17, 2500, 4999, 5000):
        _check_exact(lib, a, k)


def test_partition_nan_signed_zero_and_infinities(lib):
    a = np.array([np.nan, -0.0, 0.0, -np.inf, 1.0, np.nan, -1.0, np.inf, 3.5, -0.0], dtype=np.float32)
    for k in range(len(a) + 1):
        S, C, isn, _ = _partition(lib, a, k, s01=False)
        rS, rC, _, _ = OP.partition(a.astype(np.float64), k)
        assert np.array_equal(S, rS) and np.array_equal(C, rC), k


def test_partition_constant_scores_give_lowest_indices_and_zero_s(lib):
    a = np.full(333, 2.5, dtype=np.float32)
    S, C, _, s = _partition(lib, a, 100)
    assert np.array_equal(S, np.arange(100)) and np.array_equal(C, np.arange(100, 333))
    assert np.all(s == 0.0)


def _accumulate(lib, x, lse_img, tv, c0, c1, prev=None):
    t = torch()
    sc = dev(prev.astype(np.float32)) if prev is not None else t.full((x.shape[1],), np.nan, dtype=t.float32, device="cuda")
    lib.safe_pcsp_accumulate(dev(x), dev(lse_img) if lse_img is not None else None, tv, c0, c1, sc, prev is not None)
    t.cuda.synchronize()
    return host(sc).astype(np.float64)


@pytest.mark.parametrize("T,tv,c0,c1", [(256, 77, 0, 77), (256, 77, 5, 60), (64, 64, 0, 64), (37, 20, 0, 20),
                                        (8, 0, 0, 0), (300, 255, 1, 255)])
def test_accumulate_parity(lib, T, tv, c0, c1):
    r = np.random.default_rng(T + tv)
    H, N = 5, 333
    x = (r.standard_normal((H, N, T)) * 2).astype(np.float32)
    li = (r.standard_normal((H, N)) + 4).astype(np.float32)
    for lse_img in (li, None):
        got = _accumulate(lib, x, lse_img, tv, c0, c1)
        ref = OP.scores(x, lse_img, tv, c0, c1)
        assert np.all(np.abs(got - ref) <= 5e-6 * np.abs(ref) + 1e-37), (lse_img is None)
    # accumulation adds
    prev = r.random(N).astype(np.float32)
    got = _accumulate(lib, x, li, tv, c0, c1, prev=prev)
    ref = prev.astype(np.float64) + OP.scores(x, li, tv, c0, c1)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-30)) < 5e-6


def test_accumulate_text_only_closed_form(lib):
    x = (np.random.default_rng(3).standard_normal((24, 1000, 256)) * 3).astype(np.float32)
    got = _accumulate(lib, x, None, 77, 0, 77)
    assert np.max(np.abs(got - 24.0)) < 24 * 2e-6


@pytest.mark.parametrize("name", ["srsu_1024", "srsu_2560", "traj_3072"])
def test_end_to_end_partition_matches_fp64(lib, name):
    """GPU scores (fp32) -> GPU partition equals the fp64 oracle's partition; margin is reported."""
    w = syn.WORKLOADS[name]
    t = torch()
    sc = t.zeros(w.N, dtype=t.float32, device="cuda")
    a_ref = None
    for step in range(w.warmup_steps):
        inp = syn.pcsp_logits(w, step)
        lib.safe_pcsp_accumulate(dev(inp["x"]), dev(inp["lse_img"]), w.tv[0], 0, w.tv[0], sc, step > 0)
        a_ref = OP.accumulate(a_ref, inp["x"], inp["lse_img"], w.tv[0], 0, w.tv[0])
        del inp
    a_gpu = host(sc).astype(np.float64)
    rel_err = float(np.max(np.abs(a_gpu - a_ref) / a_ref))
    o = OP.order(a_ref)
    margin = float((a_ref[o[w.k - 1]] - a_ref[o[w.k]]) / a_ref[o[w.k - 1]])
    print(f"{name}: boundary margin {margin:.3e}, max rel fp32 score error {rel_err:.3e}")
    assert rel_err < 2e-6
    assert margin > 10 * rel_err, "boundary ill-conditioned for this seed"
    S, C, isn, s01 = _partition(lib, a_gpu.astype(np.float32), w.k)
    rS, rC, _, rs = OP.partition(a_ref, w.k)
    assert np.array_equal(S, rS) and np.array_equal(C, rC)
    assert np.max(np.abs(s01 - rs)) < 1e-5
