"""Pins of the fp64 attention oracle against things other than itself (CPU only)."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as A


def _inputs(B=2, H=3, N=37, T=11, d=16, seed=0, std=0.5):
    r = np.random.default_rng(seed)
    f = lambda *s: (r.standard_normal(s) * std)
    return f(B, H, N, d), f(B, H, N, d), f(B, H, N, d), f(B, H, T, d), f(B, H, T, d)


def _sdpa(q, ki, vi, kt, vt, tv, mask=None, scale=None):
    """torch's fp64 CPU scaled_dot_product_attention over [image | all T text] keys, padding as -inf."""
    B, H, N, d = q.shape
    T = kt.shape[2]
    K = torch.from_numpy(np.concatenate([ki, kt], axis=2))
    V = torch.from_numpy(np.concatenate([vi, vt], axis=2))
    m = torch.zeros(B, H, N, N + T, dtype=torch.float64)
    for b in range(B):
        m[b, :, :, N + tv[b]:] = -math.inf
    if mask is not None:
        mm = torch.from_numpy(np.where(mask, 0.0, -np.inf) if mask.dtype == np.bool_ else mask.astype(np.float64))
        if mm.shape[-1] == N:
            mm = torch.cat([mm, torch.zeros(*mm.shape[:-1], T, dtype=torch.float64)], dim=-1)
        m = m + mm
    return torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), K, V, attn_mask=m, scale=scale).numpy()


@pytest.mark.parametrize("tv", [(11, 11), (4, 7), (0, 3)])
def test_matches_torch_sdpa(tv):
    q, ki, vi, kt, vt = _inputs()
    o, _ = A.attention(q, ki, vi, kt, vt, tv)
    ref = _sdpa(q, ki, vi, kt, vt, tv)
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_matches_torch_sdpa_at_the_library_head_dims(d):
    """The default scale 1/sqrt(d) and the full-width dot products at both head dims the library takes."""
    q, ki, vi, kt, vt = _inputs(B=1, H=2, N=40, T=9, d=d, seed=d, std=0.3)
    o, lse = A.attention(q, ki, vi, kt, vt, (6,))
    ref = _sdpa(q, ki, vi, kt, vt, (6,))
    assert np.max(np.abs(o - ref)) < 1e-12
    keys = np.concatenate([ki, kt[:, :, :6]], axis=2)
    ref_lse = logsumexp(np.einsum("bhnd,bhmd->bhnm", q, keys) / math.sqrt(d), axis=-1)
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_matches_torch_sdpa_with_per_head_mask():
    q, ki, vi, kt, vt = _inputs()
    r = np.random.default_rng(5)
    mask = r.standard_normal((2, 3, 37, 37 + 11))
    mask[r.random(mask.shape) < 0.2] = -np.inf
    mask[..., 0] = 0.0  # no fully masked row
    o, _ = A.attention(q, ki, vi, kt, vt, (5, 9), mask=mask)
    ref = _sdpa(q, ki, vi, kt, vt, (5, 9), mask=mask)
    assert np.max(np.abs(o - ref)) < 1e-12
    bmask = r.random((1, 3, 37, 37)) < 0.8
    bmask[..., 0] = True
    o, _ = A.attention(q, ki, vi, kt, vt, (5, 9), mask=bmask)
    ref = _sdpa(q, ki, vi, kt, vt, (5, 9), mask=np.broadcast_to(bmask, (2, 3, 37, 37)))
    assert np.max(np.abs(o - ref)) < 1e-12


def test_brute_force_loops():
    """Pure-Python loops with math.exp on a tiny instance."""
    q, ki, vi, kt, vt = _inputs(B=1, H=2, N=5, T=3, d=4, seed=3, std=1.0)
    tv = (2,)
    o, lse = A.attention(q, ki, vi, kt, vt, tv, scale=0.7)
    for h in range(2):
        for i in range(5):
            keys = [ki[0, h, j] for j in range(5)] + [kt[0, h, t] for t in range(2)]
            vals = [vi[0, h, j] for j in range(5)] + [vt[0, h, t] for t in range(2)]
            logits = [0.7 * sum(q[0, h, i, c] * kk[c] for c in range(4)) for kk in keys]
            w = [math.exp(z) for z in logits]
            z = sum(w)
            for c in range(4):
                ref = sum(w[j] * vals[j][c] for j in range(7)) / z
                assert abs(o[0, h, i, c] - ref) < 1e-12
            assert abs(lse[0, h, i] - math.log(z)) < 1e-12


def test_rows_sum_to_one():
    q, ki, vi, kt, vt = _inputs(seed=1, std=2.0)
    o, _ = A.attention(q, ki, np.ones_like(vi), kt, np.ones_like(vt), (3, 11))
    assert np.max(np.abs(o - 1.0)) < 1e-12


def test_zero_query_is_mean_of_valid_values():
    q, ki, vi, kt, vt = _inputs(seed=2)
    tv = (4, 0)
    o, lse = A.attention(np.zeros_like(q), ki, vi, kt, vt, tv)
    for b in range(2):
        mean = np.concatenate([vi[b], vt[b, :, : tv[b]]], axis=1).mean(axis=1)
        assert np.max(np.abs(o[b] - mean[:, None, :])) < 1e-12
        assert np.max(np.abs(lse[b] - math.log(37 + tv[b]))) < 1e-12


def test_dominant_key_selects_its_value():
    q, ki, vi, kt, vt = _inputs(B=1, H=1, N=9, T=4, d=8, seed=4, std=0.1)
    d = 8
    kt = kt.copy()
    kt[0, 0, 2] = q[0, 0, 3] / np.dot(q[0, 0, 3], q[0, 0, 3]) * 40.0 * math.sqrt(d)  # logit +40 for row 3
    o, _ = A.attention(q, ki, vi, kt, vt, (4,), rows=np.array([3]))
    assert np.max(np.abs(o[0, 0, 0] - vt[0, 0, 2])) < 1e-12


def test_key_value_permutation_equivariance():
    q, ki, vi, kt, vt = _inputs(seed=6)
    p = np.random.default_rng(0).permutation(37)
    o1, _ = A.attention(q, ki, vi, kt, vt, (6, 6))
    o2, _ = A.attention(q, ki[:, :, p], vi[:, :, p], kt, vt, (6, 6))
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_row_constant_shift_leaves_output_unchanged():
    q, ki, vi, kt, vt = _inputs(seed=7)
    c = np.random.default_rng(1).uniform(-5, 5, size=37)
    mask = np.broadcast_to(c[None, None, :, None], (1, 1, 37, 48)).copy()
    o1, l1 = A.attention(q, ki, vi, kt, vt, (6, 11))
    o2, l2 = A.attention(q, ki, vi, kt, vt, (6, 11), mask=mask)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs((l2 - l1) - c[None, None, :])) < 1e-12


def test_padding_contents_are_ignored():
    q, ki, vi, kt, vt = _inputs(seed=8)
    tv = (3, 8)
    kt2, vt2 = kt.copy(), vt.copy()
    kt2[0, :, 3:] = np.nan
    vt2[0, :, 3:] = np.nan
    kt2[1, :, 8:] = 1e30
    vt2[1, :, 8:] = -1e30
    o1, _ = A.attention(q, ki, vi, kt, vt, tv)
    o2, _ = A.attention(q, ki, vi, kt2, vt2, tv)
    assert np.array_equal(o1, o2)


def test_no_text_is_plain_image_self_attention():
    q, ki, vi, kt, vt = _inputs(seed=9)
    o, _ = A.attention(q, ki, vi, kt, vt, (0, 0))
    ref = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, ki, vi))).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_fully_masked_row_is_zero():
    q, ki, vi, kt, vt = _inputs(B=1, seed=10)
    mask = np.ones((1, 1, 37, 37), dtype=np.bool_)
    mask[0, 0, 5] = False
    o, lse = A.attention(q, ki, vi, kt, vt, (0,), mask=mask)
    assert np.all(o[0, :, 5] == 0.0) and np.all(np.isneginf(lse[0, :, 5]))
    assert np.all(np.isfinite(lse[0, :, 4]))


def test_lse_and_emission_match_library_logsumexp():
    q, ki, vi, kt, vt = _inputs(seed=11)
    tv = (7, 2)
    scale = 0.25
    o, lse, x, lse_img = A.attention(q, ki, vi, kt, vt, tv, scale=scale, want_emission=True)
    for h in range(3):
        li = scale * torch.from_numpy(q[0, h]) @ torch.from_numpy(ki[0, h]).T
        lt = scale * torch.from_numpy(q[0, h]) @ torch.from_numpy(kt[0, h, :7]).T
        assert np.max(np.abs(x[h] - lt.numpy())) < 1e-12
        assert np.max(np.abs(lse_img[h] - logsumexp(li.numpy(), axis=1))) < 1e-12
        assert np.max(np.abs(lse[0, h] - logsumexp(np.concatenate([li.numpy(), lt.numpy()], 1), axis=1))) < 1e-12


def test_sensitive_rows_step():
    q, ki, vi, kt, vt = _inputs(seed=12)
    tv = (5, 11)
    state = np.random.default_rng(3).standard_normal((2, 3, 37, 16))
    dense = A.dense_step(state, q, ki, vi, kt, vt, tv=tv)
    S = np.array([0, 3, 4, 20, 36])
    new = A.rows_step(state, S, q, ki, vi, kt, vt, tv=tv)
    C = np.setdiff1d(np.arange(37), S)
    assert np.array_equal(new[:, :, C], state[:, :, C])
    assert np.max(np.abs(new[:, :, S] - dense[:, :, S])) < 1e-12
    full = A.rows_step(state, np.arange(37), q, ki, vi, kt, vt, tv=tv)
    assert np.max(np.abs(full - dense)) < 1e-12
    assert np.array_equal(A.rows_step(state, np.array([], dtype=np.int32), q, ki, vi, kt, vt, tv=tv), state)


def test_gather_scatter_roundtrip():
    st = np.random.default_rng(4).standard_normal((2, 3, 37, 16))
    S = np.array([1, 2, 30])
    p = A.gather_rows(st, S)
    assert p.shape == (2, 3, 3, 16) and np.array_equal(p[:, :, 2], st[:, :, 30])
    z = np.zeros_like(st)
    back = A.scatter_rows(z, p, S)
    assert np.array_equal(back[:, :, S], st[:, :, S]) and np.all(back[:, :, 0] == 0)


def test_golden_hand_examples():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "attention_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"]).reshape(1, 1, 1, 1)
        ki = np.array(c["k_img"]).reshape(1, 1, 2, 1)
        vi = np.array(c["v_img"]).reshape(1, 1, 2, 1)
        kt = np.array(c["k_txt"]).reshape(1, 1, 1, 1)
        vt = np.array(c["v_txt"]).reshape(1, 1, 1, 1)
        # the query row is image row 0; image row 1 gets a copy of the same query
        q2 = np.concatenate([q, q], axis=2)
        mask = np.full((1, 1, 2, 3), c["row_shift"])
        o, lse = A.attention(q2, ki, vi, kt, vt, (c["tv"],), scale=c["scale"], mask=mask, rows=np.array([0]))
        assert abs(o[0, 0, 0, 0] - c["o"]) < 1e-12, c["why"]
        assert abs(lse[0, 0, 0] - c["lse"]) < 1e-12, c["why"]
