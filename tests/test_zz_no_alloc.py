"""The allocation-free FFN entry point (safe_rows_ffn_noalloc) against the workspace form (safe_rows_ffn),
through the C ABI: bitwise equal outputs on two calls in a row, the second with fewer rows, and a request
beyond the fixed scratch size rejected without a launch."""
import numpy as np
import pytest

import synthetic as syn
from oracle import srsu_block as SB
from tests.gpu_util import assert_close, dev, host, torch

pytestmark = pytest.mark.gpu


def _bf(x):
    return dev(None, syn.f32_to_bf16_bits(np.ascontiguousarray(x, dtype=np.float32)))


def test_noalloc_ffn_matches_the_workspace_form(lib):
    t = torch()
    w = syn.WORKLOADS["srsu_1024"]
    x = syn.hidden_states(w)
    bw = syn.block_weights(w)
    F = bw["w1"].shape[0]
    xd, w1, w2 = _bf(x), _bf(bw["w1"]), _bf(bw["w2"])
    b1, b2 = dev(bw["b1"]), dev(bw["b2"])
    assert lib.safe_rows_ffn_noalloc_max_bytes() >= lib.safe_rows_ffn_workspace_bytes(w.B, w.k, F)
    cache0 = syn.round_to_bf16(np.random.default_rng(3).standard_normal(x.shape).astype(np.float32))
    # first call: the full 1024^2 block (k = 1229); second: a smaller, different row set (k = 300)
    for k, seed in ((w.k, 0), (300, 1)):
        rows = syn.random_rows(w, k=k, seed_step=seed)
        rd = dev(rows)
        ws = t.empty(lib.safe_rows_ffn_workspace_bytes(w.B, k, F) // 2, dtype=t.bfloat16, device="cuda")
        ref_cache = _bf(cache0)
        lib.safe_rows_ffn(xd, rd, w1, b1, w2, b2, ref_cache, ws)
        got_cache = _bf(cache0)
        lib.safe_rows_ffn_noalloc(xd, rd, w1, b1, w2, b2, got_cache)
        t.cuda.synchronize()
        got, ref = host(got_cache), host(ref_cache)
        assert np.array_equal(got, ref), k  # same kernels, same arithmetic
        other = np.setdiff1d(np.arange(w.N), rows)
        assert np.array_equal(got[:, other], cache0[:, other].astype(np.float64))
        pick = rows[syn.sample_rows(len(rows), 16, seed=k)]
        oracle = SB.rows_ffn(x, pick, bw["w1"], bw["b1"], bw["w2"], bw["b2"], cache0)
        assert_close(got[:, pick], oracle[:, pick], "bf16", f"noalloc FFN k={k}")


def test_noalloc_ffn_rejects_requests_beyond_its_scratch(lib):
    t = torch()
    B, N, D = 2, 8192, 128
    F = 4096
    max_bytes = lib.safe_rows_ffn_noalloc_max_bytes()
    k = N  # 2 * 8192 * 4096 * 2 = 128 MiB > the scratch
    assert lib.safe_rows_ffn_workspace_bytes(B, k, F) > max_bytes
    x = t.zeros((B, N, D), dtype=t.bfloat16, device="cuda")
    w1 = t.zeros((F, D), dtype=t.bfloat16, device="cuda")
    w2 = t.zeros((D, F), dtype=t.bfloat16, device="cuda")
    cache = t.full((B, N, D), 1.5, dtype=t.bfloat16, device="cuda")
    rows = t.arange(N, dtype=t.int32, device="cuda")
    with pytest.raises(lib.SafeAttnError) as e:
        lib.safe_rows_ffn_noalloc(x, rows, w1, None, w2, None, cache)
    assert e.value.code == 5  # SAFE_ERR_WORKSPACE
    t.cuda.synchronize()
    assert bool((cache == 1.5).all())  # nothing was launched
