"""GPU parity of the sensitive-row block products: the FFN with cached context rows and the QKV projection
into the head-major attention tensors, against the fp64 oracle (every row, up to the 1024^2 shapes)."""
import numpy as np
import pytest

import synthetic as syn
from oracle import srsu_block as SB
from tests.gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu


def _bf(x):
    return dev(None, syn.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)))


def _inputs(B, N, H, d, k, seed, ffn_mult=4):
    r = np.random.default_rng(seed)
    D = H * d
    F = ffn_mult * D
    x = syn.round_to_bf16(r.standard_normal((B, N, D)).astype(np.float32))
    w1 = syn.round_to_bf16((r.standard_normal((F, D)) / np.sqrt(D)).astype(np.float32))
    w2 = syn.round_to_bf16((r.standard_normal((D, F)) / np.sqrt(F)).astype(np.float32))
    wqkv = syn.round_to_bf16((r.standard_normal((3 * D, D)) / np.sqrt(D)).astype(np.float32))
    b1 = (0.02 * r.standard_normal(F)).astype(np.float32)
    b2 = (0.02 * r.standard_normal(D)).astype(np.float32)
    bq = (0.02 * r.standard_normal(3 * D)).astype(np.float32)
    rows = np.sort(r.choice(N, size=k, replace=False)).astype(np.int32)
    return dict(x=x, w1=w1, w2=w2, wqkv=wqkv, b1=b1, b2=b2, bqkv=bq, rows=rows, D=D, F=F)


def _ffn(lib, p, cache0, with_bias=True):
    t = torch()
    B, N, D = p["x"].shape
    k = len(p["rows"])
    cache = _bf(cache0)
    ws = t.empty(max(lib.safe_rows_ffn_workspace_bytes(B, k, p["F"]) // 2, 1), dtype=t.bfloat16, device="cuda")
    lib.safe_rows_ffn(_bf(p["x"]), dev(p["rows"]), _bf(p["w1"]), dev(p["b1"]) if with_bias else None, _bf(p["w2"]),
                      dev(p["b2"]) if with_bias else None, cache, ws)
    t.cuda.synchronize()
    return host(cache)


@pytest.mark.parametrize("B,N,H,d,k,mult", [(1, 40, 2, 64, 1, 4), (2, 300, 2, 64, 77, 4), (2, 300, 2, 64, 300, 4),
                                            (2, 500, 4, 64, 129, 2), (3, 257, 2, 64, 200, 1),
                                            (2, 300, 8, 64, 77, 4), (1, 600, 8, 64, 299, 4),  # F = 2048: 256 x 256 tiles
                                            (2, 300, 12, 64, 131, 3),  # F = 2304: 192 x 256 tiles, ragged tokens
                                            # D -> F with K = D = 128 (four 32-element stages: the ring's tail
                                            # alone) on both tile widths, and K = 256 (one pass of the loop)
                                            (1, 100, 2, 64, 37, 16), (1, 100, 2, 64, 37, 18), (2, 100, 4, 64, 50, 8)])
def test_rows_ffn_parity_and_cache_untouched(lib, B, N, H, d, k, mult):
    p = _inputs(B, N, H, d, k, seed=N + k, ffn_mult=mult)
    cache0 = syn.round_to_bf16(np.random.default_rng(k).standard_normal((B, N, p["D"])).astype(np.float32))
    for with_bias in (True, False):
        got = _ffn(lib, p, cache0, with_bias)
        ref = SB.rows_ffn(p["x"], p["rows"], p["w1"], p["b1"] if with_bias else None, p["w2"],
                          p["b2"] if with_bias else None, cache0)
        rows = p["rows"]
        assert_close(got[:, rows], ref[:, rows], "bf16", "block product")
        other = np.setdiff1d(np.arange(N), rows)
        assert np.array_equal(got[:, other], cache0[:, other].astype(np.float64))


def _qkv(lib, p, H, d, q0, k0, v0):
    t = torch()
    q, kc, vc = _bf(q0), _bf(k0), _bf(v0)
    lib.safe_rows_qkv(_bf(p["x"]), dev(p["rows"]), _bf(p["wqkv"]), dev(p["bqkv"]), q, kc, vc)
    t.cuda.synchronize()
    return host(q), host(kc), host(vc)


@pytest.mark.parametrize("B,N,H,d,k", [(1, 40, 2, 64, 1), (2, 300, 2, 64, 77), (2, 200, 6, 64, 200),
                                       (2, 200, 12, 64, 131)])  # 3D = 2304: 192 x 256 tiles
def test_rows_qkv_parity_and_context_untouched(lib, B, N, H, d, k):
    p = _inputs(B, N, H, d, k, seed=3 * N + k)
    r = np.random.default_rng(k)
    q0, k0, v0 = (syn.round_to_bf16(r.standard_normal((B, H, N, d)).astype(np.float32)) for _ in range(3))
    got = _qkv(lib, p, H, d, q0, k0, v0)
    ref = SB.rows_qkv(p["x"], p["rows"], p["wqkv"], p["bqkv"], q0, k0, v0, H, d)
    rows = p["rows"]
    other = np.setdiff1d(np.arange(N), rows)
    for g, rf, orig in zip(got, ref, (q0, k0, v0)):
        assert_close(g[:, :, rows], rf[:, :, rows], "bf16", "block product")
        assert np.array_equal(g[:, :, other], orig[:, :, other].astype(np.float64))


def test_rows_outside_range_are_skipped(lib):
    """Row entries outside [0, N) write nothing (the same contract as the row gather / scatter)."""
    p = _inputs(2, 64, 2, 64, 10, seed=9)
    p["rows"] = np.array([-1, 0, 5, 9, 20, 33, 40, 63, 64, 1000], dtype=np.int32)
    cache0 = np.zeros((2, 64, p["D"]), dtype=np.float32)
    got = _ffn(lib, p, cache0)
    valid = p["rows"][(p["rows"] >= 0) & (p["rows"] < 64)]
    ref = SB.rows_ffn(p["x"], valid, p["w1"], p["b1"], p["w2"], p["b2"], cache0)
    assert_close(got, ref, "bf16", "block product")


@pytest.mark.parametrize("name", ["srsu_1024"])
def test_full_size_block_products(lib, name):
    """The 1024^2 shapes: B = 2, N = 4096, D = 1536 (24 x 64), F = 6144, |S| = 1229, every row compared."""
    w = syn.WORKLOADS[name]
    t = torch()
    x = syn.hidden_states(w)
    bw = syn.block_weights(w)
    rows = syn.random_rows(w)
    cache0 = np.zeros_like(x)
    cache = _bf(cache0)
    ws = t.empty(lib.safe_rows_ffn_workspace_bytes(w.B, w.k, bw["w1"].shape[0]) // 2, dtype=t.bfloat16, device="cuda")
    xd = _bf(x)
    lib.safe_rows_ffn(xd, dev(rows), _bf(bw["w1"]), dev(bw["b1"]), _bf(bw["w2"]), dev(bw["b2"]), cache, ws)
    q = t.zeros((w.B, w.H, w.N, w.d), dtype=t.bfloat16, device="cuda")
    kc, vc = t.zeros_like(q), t.zeros_like(q)
    lib.safe_rows_qkv(xd, dev(rows), _bf(bw["wqkv"]), dev(bw["bqkv"]), q, kc, vc)
    t.cuda.synchronize()
    ref = SB.rows_ffn(x, rows, bw["w1"], bw["b1"], bw["w2"], bw["b2"], cache0)
    mx, rel = assert_close(host(cache)[:, rows], ref[:, rows], "bf16", f"{name} FFN")

    print(f"{name} FFN: max-abs {mx:.3e}, rel-L2 {rel:.3e}")
    z = np.zeros((w.B, w.H, w.N, w.d), dtype=np.float32)
    rq = SB.rows_qkv(x, rows, bw["wqkv"], bw["bqkv"], z, z, z, w.H, w.d)
    for g, rf in zip((q, kc, vc), rq):
        mx, rel = assert_close(host(g)[:, :, rows], rf[:, :, rows], "bf16", f"{name} QKV")

        print(f"{name} QKV: max-abs {mx:.3e}, rel-L2 {rel:.3e}")


def test_rows_ffn_many_tokens(lib):
    """5632 gathered tokens (more token tiles than the GPU has CUs, in both products) with F = 2048: sampled
    rows against the oracle, and every context row untouched."""
    B, N, H, d, k = 2, 3000, 24, 64, 2816
    p = _inputs(B, N, H, d, k, seed=77, ffn_mult=4)
    F = 2048  # D -> F on 256 x 256 tiles, F -> D on 128 x 128 tiles
    r = np.random.default_rng(78)
    D = p["D"]
    p["F"] = F
    p["w1"] = syn.round_to_bf16((r.standard_normal((F, D)) / np.sqrt(D)).astype(np.float32))
    p["w2"] = syn.round_to_bf16((r.standard_normal((D, F)) / np.sqrt(F)).astype(np.float32))
    p["b1"] = (0.02 * r.standard_normal(F)).astype(np.float32)
    cache0 = syn.round_to_bf16(r.standard_normal((B, N, D)).astype(np.float32))
    got = _ffn(lib, p, cache0)
    rows = p["rows"]
    pick = rows[syn.sample_rows(len(rows), 48, seed=5)]
    ref = SB.rows_ffn(p["x"], pick, p["w1"], p["b1"], p["w2"], p["b2"], cache0)
    assert_close(got[:, pick], ref[:, pick], "bf16", "block product")
    other = np.setdiff1d(np.arange(N), rows)
    assert np.array_equal(got[:, other], cache0[:, other].astype(np.float64))
