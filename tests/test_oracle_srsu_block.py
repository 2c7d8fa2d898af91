"""Pins of the sensitive-row block oracle: torch's linear and GELU, the cache contract, the head split."""
import numpy as np
import torch

from oracle import srsu_block as SB


def test_gelu_tanh_against_torch_and_closed_forms():
    x = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(SB.gelu_tanh(x) - ref)) < 1e-14
    assert SB.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(SB.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(SB.gelu_tanh(np.array([-30.0]))[0]) < 1e-12


def test_rows_ffn_is_torch_linear_gelu_linear_on_the_rows_and_keeps_the_rest():
    r = np.random.default_rng(1)
    B, N, D, F = 2, 30, 16, 24
    x = r.standard_normal((B, N, D))
    w1, b1 = r.standard_normal((F, D)) * 0.3, r.standard_normal(F)
    w2, b2 = r.standard_normal((D, F)) * 0.3, r.standard_normal(D)
    cache = r.standard_normal((B, N, D))
    rows = np.array([0, 3, 4, 17, 29])
    got = SB.rows_ffn(x, rows, w1, b1, w2, b2, cache)
    t = torch.from_numpy
    full = torch.nn.functional.linear(
        torch.nn.functional.gelu(torch.nn.functional.linear(t(x), t(w1), t(b1)), approximate="tanh"), t(w2), t(b2)).numpy()
    assert np.max(np.abs(got[:, rows] - full[:, rows])) < 1e-12
    other = np.setdiff1d(np.arange(N), rows)
    assert np.array_equal(got[:, other], cache[:, other])
    # all rows: the dense FFN
    assert np.max(np.abs(SB.rows_ffn(x, np.arange(N), w1, b1, w2, b2, cache) - full)) < 1e-12


def test_rows_qkv_head_split():
    r = np.random.default_rng(2)
    B, N, H, d = 2, 12, 3, 4
    D = H * d
    x = r.standard_normal((B, N, D))
    w, b = r.standard_normal((3 * D, D)), r.standard_normal(3 * D)
    q0, k0, v0 = (r.standard_normal((B, H, N, d)) for _ in range(3))
    rows = np.array([1, 5, 11])
    q, k, v = SB.rows_qkv(x, rows, w, b, q0, k0, v0, H, d)
    y = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    for which, (got, orig) in enumerate(((q, q0), (k, k0), (v, v0))):
        for bb in range(B):
            for h in range(H):
                for rr in rows:
                    want = y[bb, rr, which * D + h * d: which * D + (h + 1) * d]
                    assert np.max(np.abs(got[bb, h, rr] - want)) < 1e-12
        other = np.setdiff1d(np.arange(N), rows)
        assert np.array_equal(got[:, :, other], orig[:, :, other])
