"""Pins of the AesMask oracle: the affinity is joint-softmax attention mass over the selected text slots,
and the percentile mask keeps the tokens numpy's percentile keeps."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import aesmask as A


def _joint(r, H, N, T, d, tv):
    q, ki, kt = r.standard_normal((H, N, d)), r.standard_normal((H, N, d)), r.standard_normal((H, T, d))
    scale = 1 / math.sqrt(d)
    logits = torch.cat([torch.from_numpy(q) @ torch.from_numpy(ki).transpose(1, 2),
                        torch.from_numpy(q) @ torch.from_numpy(kt[:, :tv]).transpose(1, 2)], dim=2) * scale
    prob = torch.softmax(logits, dim=2).numpy()  # [H, N, N + tv]
    x = np.zeros((H, N, T))
    x[:, :, :tv] = scale * np.einsum("hnd,htd->hnt", q, kt[:, :tv])
    x[:, :, tv:] = 1e30  # padded slots must never be read
    lse_img = np.log(np.exp(scale * np.einsum("hnd,hmd->hnm", q, ki)).sum(axis=2))
    return prob, x, lse_img


def test_affinity_is_the_joint_attention_mass_of_the_selected_slots():
    r = np.random.default_rng(11)
    H, N, T, d, tv = 3, 12, 10, 8, 7
    prob, x, lse_img = _joint(r, H, N, T, d, tv)
    sel = np.zeros(T, dtype=np.uint8)
    sel[[0, 2, 5, 8, 9]] = 1  # slots 8 and 9 are padding: ignored
    ref = prob[:, :, N + np.array([0, 2, 5])].sum(axis=2).sum(axis=0)
    assert np.max(np.abs(A.affinity(x, lse_img, tv, sel) - ref)) < 1e-12


def test_all_valid_text_only_gives_head_count_and_empty_selection_gives_zero():
    x = np.random.default_rng(12).standard_normal((6, 30, 16)) * 4
    assert np.max(np.abs(A.affinity(x, None, 13, np.ones(16, dtype=np.uint8)) - 6.0)) < 1e-12
    assert np.all(A.affinity(x, None, 13, np.zeros(16, dtype=np.uint8)) == 0)


def test_disjoint_selections_add_and_rows_shift_invariant():
    r = np.random.default_rng(13)
    x, li = r.standard_normal((4, 25, 20)), r.standard_normal((4, 25)) + 2
    s1 = (r.random(20) < 0.3).astype(np.uint8)
    s2 = ((r.random(20) < 0.4) & (s1 == 0)).astype(np.uint8)
    a12 = A.affinity(x, li, 17, s1 | s2)
    assert np.max(np.abs(a12 - A.affinity(x, li, 17, s1) - A.affinity(x, li, 17, s2))) < 1e-12
    sh = r.uniform(-20, 20, size=(4, 25))
    assert np.max(np.abs(A.affinity(x + sh[:, :, None], li + sh, 17, s1) - A.affinity(x, li, 17, s1))) < 1e-12


@pytest.mark.parametrize("N", [1, 2, 3, 10, 97, 1000, 4096])
@pytest.mark.parametrize("pct_bp", [0, 1, 777, 2500, 3333, 5000, 7500, 8000, 9000, 9999, 10000])
def test_percentile_count_matches_numpy_percentile(N, pct_bp):
    """For distinct scores, the kept tokens are those at or above numpy's (linearly interpolated)
    percentile.  Where p (N - 1) / 100 is an integer numpy's own float rounding of the interpolation
    index decides between two order statistics, so there the threshold is that order statistic."""
    a = np.random.default_rng(N * 7 + pct_bp).permutation(N).astype(np.float64) + 0.5
    k, S, is_focus = A.mask(a, pct_bp)
    exact = Fraction(pct_bp * (N - 1), 10000)
    if exact.denominator == 1:
        thr = np.sort(a)[int(exact)]
    else:
        thr = np.percentile(a, pct_bp / 100.0)
    want = np.flatnonzero(a >= thr)
    assert k == len(want)
    assert np.array_equal(S, want) and np.array_equal(np.flatnonzero(is_focus), want)


def test_percentile_count_edges_and_ties():
    assert A.percentile_count(0, 5000) == 0
    assert [A.percentile_count(5, p) for p in (0, 2500, 5000, 7500, 10000)] == [5, 4, 3, 2, 1]
    with pytest.raises(ValueError):
        A.percentile_count(5, 10001)
    # equal scores: the count stays, the lower index wins
    k, S, _ = A.mask(np.array([1.0, 3.0, 3.0, 3.0, 0.0, 3.0]), 5000)
    assert k == 3 and list(S) == [1, 2, 3]
