"""Pins of the PCSP oracle: scores as attention mass, exact top-k, invariants."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import pcsp as P
import synthetic as syn


def test_text_only_softmax_over_all_valid_gives_head_count():
    x = np.random.default_rng(0).standard_normal((5, 40, 16)) * 3
    a = P.scores(x, None, 11, 0, 11)
    assert np.max(np.abs(a - 5.0)) < 1e-12


def test_scores_are_the_joint_attention_text_content_mass():
    """The score is the attention weight a joint softmax gives the text content slots, summed over heads."""
    r = np.random.default_rng(1)
    H, N, T, d, tv, c0, c1 = 3, 10, 6, 8, 5, 1, 4
    q, ki, kt = r.standard_normal((H, N, d)), r.standard_normal((H, N, d)), r.standard_normal((H, T, d))
    scale = 1 / math.sqrt(d)
    logits = torch.cat([torch.from_numpy(q) @ torch.from_numpy(ki).transpose(1, 2),
                        torch.from_numpy(q) @ torch.from_numpy(kt[:, :tv]).transpose(1, 2)], dim=2) * scale
    prob = torch.softmax(logits, dim=2).numpy()
    ref = prob[:, :, N + c0:N + c1].sum(axis=2).sum(axis=0)
    x = np.zeros((H, N, T))
    x[:, :, :tv] = scale * np.einsum("hnd,htd->hnt", q, kt[:, :tv])
    x[:, :, tv:] = 123.0  # padding must be ignored
    lse_img = np.log(np.exp(scale * np.einsum("hnd,hmd->hnm", q, ki)).sum(axis=2))
    a = P.scores(x, lse_img, tv, c0, c1)
    assert np.max(np.abs(a - ref)) < 1e-12


def test_row_shift_invariance_and_accumulation():
    r = np.random.default_rng(2)
    x = r.standard_normal((4, 30, 12))
    li = r.standard_normal((4, 30)) + 3
    a = P.scores(x, li, 9, 0, 9)
    sh = r.uniform(-10, 10, size=(4, 30))
    a2 = P.scores(x + sh[:, :, None], li + sh, 9, 0, 9)
    assert np.max(np.abs(a - a2)) < 1e-12
    x2 = r.standard_normal((4, 30, 12))
    acc = P.accumulate(P.accumulate(None, x, li, 9, 2, 7), x2, li, 9, 2, 7)
    assert np.max(np.abs(acc - (P.scores(x, li, 9, 2, 7) + P.scores(x2, li, 9, 2, 7)))) < 1e-12
    assert np.all(P.scores(x, li, 9, 3, 3) == 0)


def test_order_matches_stable_library_sort():
    r = np.random.default_rng(3)
    a = r.integers(0, 6, size=500).astype(np.float64)  # many exact ties
    ref = np.argsort(-a, kind="stable")
    assert np.array_equal(P.order(a), ref)


def test_brute_force_subsets():
    r = np.random.default_rng(4)
    for trial in range(40):
        n = int(r.integers(1, 11))
        k = int(r.integers(0, n + 1))
        a = r.integers(0, 4, size=n).astype(np.float64)
        best = None
        for sub in itertools.combinations(range(n), k):  # lexicographic order
            s = a[list(sub)].sum() if sub else 0.0
            if best is None or s > best[0]:
                best = (s, sub)
        S, C, is_sens, _ = P.partition(a, k)
        assert tuple(S) == best[1]
        assert np.array_equal(np.sort(np.concatenate([S, C])), np.arange(n))
        assert np.array_equal(np.flatnonzero(is_sens), S)


def test_nan_ranks_lowest_and_signed_zero_ties():
    a = np.array([np.nan, -0.0, 0.0, -np.inf, 1.0, np.nan, -1.0])
    S, C, _, _ = P.partition(a, 4)
    assert list(S) == [1, 2, 4, 6]
    S, _, _, _ = P.partition(a, 6)
    assert list(S) == [0, 1, 2, 3, 4, 6]


def test_normalise():
    assert np.array_equal(P.normalise(np.array([2.0, 4.0, 3.0])), np.array([0.0, 1.0, 0.5]))
    assert np.array_equal(P.normalise(np.array([5.0, 5.0])), np.array([0.0, 0.0]))


def test_blob_workload_selects_tokens_near_blob_centres():
    w = syn.WORKLOADS["srsu_1024"]
    inp = syn.pcsp_logits(w)
    a = P.scores(inp["x"], inp["lse_img"], w.tv[0], 0, w.tv[0])
    S, _, _, s01 = P.partition(a, w.k)
    cen = syn.blob_centres(w)
    yy, xx = np.divmod(S, w.side)
    dist = np.min(np.hypot(yy[:, None] - cen[None, :, 0], xx[:, None] - cen[None, :, 1]), axis=1)
    assert np.quantile(dist, 0.99) < 20.0
    assert s01.min() == 0.0 and s01.max() == 1.0
    o = P.order(a)
    margin = (a[o[w.k - 1]] - a[o[w.k]]) / a[o[w.k - 1]]
    assert margin > 1e-5  # wide enough for fp32 scores to reproduce the partition
