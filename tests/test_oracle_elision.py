"""Pins of the mask-elision oracle: accepted masks leave attention unchanged, rejected ones change it."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import elision as E

N, T, d = 13, 5, 8


def _qkv(B=2, H=2, seed=0):
    r = np.random.default_rng(seed)
    f = lambda *s: r.standard_normal(s)
    return f(B, H, N, d), f(B, H, N, d), f(B, H, N, d), f(B, H, T, d), f(B, H, T, d)


def _equal_attention(mask, tv, seed=0):
    """Does the mask leave the attention output unchanged on generic random inputs?"""
    args = _qkv(B=len(tv), seed=seed)
    o0, _ = A.attention(*args, tv, mask=None)
    with np.errstate(invalid="ignore"):
        o1, _ = A.attention(*args, tv, mask=mask)
    return bool(np.all(np.abs(o0 - o1) < 1e-9))


def test_accepts_redundant_masks():
    tv = (3, 5)
    assert E.is_row_constant(np.ones((1, 1, N, N), dtype=np.bool_), N, T, tv)[0]
    assert E.is_row_constant(np.zeros((1, 1, N, N), dtype=np.float32), N, T, tv)[0]
    assert E.is_row_constant(np.ones((1, 1, N, N + T), dtype=np.bool_), N, T, tv)[0]
    c = np.random.default_rng(1).uniform(-5, 5, N)
    m = np.broadcast_to(c[None, None, :, None], (1, 1, N, N + T)).copy()
    ok, cc = E.is_row_constant(m, N, T, tv)
    assert ok and np.array_equal(cc, c)
    # negative zero equals zero
    m0 = np.zeros((1, 1, N, N)); m0[0, 0, 2, 3] = -0.0
    assert E.is_row_constant(m0, N, T, tv)[0]
    # image-only row-constant block is removable only without valid text
    mi = np.broadcast_to(c[None, None, :, None], (2, 1, N, N)).copy()
    assert E.is_row_constant(mi, N, T, (0, 0))[0]
    assert not E.is_row_constant(mi, N, T, (0, 2))[0]
    mi[1] = 0.0  # the slice used by the batch entry with text is zero
    assert E.is_row_constant(mi, N, T, (0, 2))[0]


def test_padded_columns_are_ignored():
    m = np.zeros((1, 1, N, N + T))
    m[0, 0, 4, N + 4] = 7.0  # beyond the largest valid length (3)
    m[0, 0, 5, N + 3] = np.nan
    assert E.is_row_constant(m, N, T, (3, 2))[0]
    assert not E.is_row_constant(m, N, T, (5, 2))[0]


@pytest.mark.parametrize("col,val", [(0, 1e-7), (N - 1, -1.0), (N, 0.5), (N + 2, -np.inf), (3, np.nan), (4, np.inf), (5, -np.inf)])
def test_rejects_single_perturbation(col, val):
    m = np.zeros((1, 2, N, N + T))
    m[0, 1, 6, col] = val
    ok, c = E.is_row_constant(m, N, T, (3, 3))
    assert not ok
    assert np.isnan(c[N + 6]) and np.sum(np.isnan(c)) == 1


def test_rejects_all_minus_infinity_and_false_rows():
    m = np.ones((1, 1, N, N), dtype=np.bool_)
    m[0, 0, 3] = False
    assert not E.is_row_constant(m, N, T, (2, 2))[0]
    f = np.zeros((1, 1, N, N)); f[0, 0, 3] = -np.inf
    assert not E.is_row_constant(f, N, T, (0, 0))[0]


def test_criterion_agrees_with_attention_invariance():
    """Random small masks: removable by the criterion <=> attention unchanged when it is removed."""
    r = np.random.default_rng(7)
    seen = {True: 0, False: 0}
    for trial in range(120):
        tv = tuple(int(x) for x in r.integers(0, T + 1, size=2))
        cols = N if trial % 2 else N + T
        mB, mH = int(r.integers(1, 3)), int(r.integers(1, 3))
        if r.random() < 0.5:
            base = r.integers(-2, 3, size=(mB, mH, N, 1)).astype(np.float64)
            m = np.broadcast_to(base, (mB, mH, N, cols)).copy()
            if r.random() < 0.5:  # perturb one entry somewhere (maybe in padding)
                m[tuple(int(r.integers(0, s)) for s in m.shape)] += float(r.choice([1.0, -np.inf, np.nan]))
        else:
            m = r.random((mB, mH, N, cols)) < 0.97
            if r.random() < 0.5:
                m[:] = True
        ok, _ = E.is_row_constant(m, N, T, tv)
        assert ok == _equal_attention(m, tv, seed=trial), (trial, tv, cols, mB, mH)
        seen[ok] += 1
    assert seen[True] > 20 and seen[False] > 20
