"""Seeded random sweep of the sensitive-row block products against the fp64 oracle: each case draws B, N, the
head count and width (D = H d), the FFN width F, the number of rows of S (so token counts land on and off the tile
sizes, and the tile grids on and off the narrow product's groups of five token tiles) and whether biases are given;
sampled rows of S are compared and every context row must be untouched."""
import numpy as np
import pytest

import synthetic as syn
from oracle import srsu_block as SB
from tests.gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu

N_CASES = 24


def _bf(x):
    return dev(None, syn.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)))


def _case(i):
    r = np.random.default_rng(7000 + i)
    d = int(r.choice([64, 128]))
    H = int(r.choice([2, 4, 6, 8, 12, 16])) if d == 64 else int(r.choice([1, 2, 3, 4, 6, 8]))
    D = H * d
    return dict(B=int(r.integers(1, 4)), N=int(r.integers(40, 1600)), H=H, d=d, D=D,
                F=int(r.choice([1, 2, 3, 4, 6])) * D, frac=float(r.uniform(0.02, 1.0)), bias=bool(r.random() < 0.7),
                seed=7000 + i)


@pytest.mark.parametrize("i", range(N_CASES), ids=lambda i: f"case{i}")
def test_random_block_case_matches_oracle(lib, i):
    c = _case(i)
    t = torch()
    r = np.random.default_rng(c["seed"])
    B, N, H, d, D, F = c["B"], c["N"], c["H"], c["d"], c["D"], c["F"]
    k = max(1, int(c["frac"] * N))
    rows = np.sort(r.choice(N, size=k, replace=False)).astype(np.int32)
    x = syn.round_to_bf16(r.standard_normal((B, N, D)).astype(np.float32))
    w1 = syn.round_to_bf16((r.standard_normal((F, D)) / np.sqrt(D)).astype(np.float32))
    w2 = syn.round_to_bf16((r.standard_normal((D, F)) / np.sqrt(F)).astype(np.float32))
    wq = syn.round_to_bf16((r.standard_normal((3 * D, D)) / np.sqrt(D)).astype(np.float32))
    b1 = (0.02 * r.standard_normal(F)).astype(np.float32) if c["bias"] else None
    b2 = (0.02 * r.standard_normal(D)).astype(np.float32) if c["bias"] else None
    bq = (0.02 * r.standard_normal(3 * D)).astype(np.float32) if c["bias"] else None
    cache0 = syn.round_to_bf16(r.standard_normal((B, N, D)).astype(np.float32))
    q0, k0, v0 = (syn.round_to_bf16(r.standard_normal((B, H, N, d)).astype(np.float32)) for _ in range(3))
    xd, rd = _bf(x), dev(rows)
    cache = _bf(cache0)
    ws = t.empty(max(lib.safe_rows_ffn_workspace_bytes(B, k, F) // 2, 1), dtype=t.bfloat16, device="cuda")
    lib.safe_rows_ffn(xd, rd, _bf(w1), dev(b1) if b1 is not None else None, _bf(w2),
                      dev(b2) if b2 is not None else None, cache, ws)
    q, kc, vc = _bf(q0), _bf(k0), _bf(v0)
    lib.safe_rows_qkv(xd, rd, _bf(wq), dev(bq) if bq is not None else None, q, kc, vc)
    t.cuda.synchronize()
    what = f"case{i} {c} k={k}"
    other = np.setdiff1d(np.arange(N), rows)
    got = host(cache)
    assert np.array_equal(got[:, other], cache0[:, other].astype(np.float64)), what
    pick = rows[syn.sample_rows(len(rows), 96, seed=c["seed"])]
    ref = SB.rows_ffn(x, pick, w1, b1, w2, b2, cache0)
    assert_close(got[:, pick], ref[:, pick], "bf16", "FFN " + what)
    ref_qkv = SB.rows_qkv(x, pick, wq, bq, q0, k0, v0, H, d)
    for g, rf, orig in zip((host(q), host(kc), host(vc)), ref_qkv, (q0, k0, v0)):
        assert np.array_equal(g[:, :, other], orig[:, :, other].astype(np.float64)), what
        assert_close(g[:, :, pick], rf[:, :, pick], "bf16", "QKV " + what)
