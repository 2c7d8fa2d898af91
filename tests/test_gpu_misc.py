"""GPU parity of SW-CFG, row gather/scatter and the mask-elision check."""
import numpy as np
import pytest

import synthetic as syn
from oracle import elision as OE
from oracle import swcfg as OG
from oracle import attention as OA
from tests.gpu_util import CFG_REL, dev, host, torch

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------------------ SW-CFG
def _cfg(lib, eps, s, side, gc, gs):
    t = torch()
    out = t.full(eps.shape[1:], np.nan, dtype=t.float32, device="cuda")
    lib.safe_swcfg_combine(dev(eps), dev(s.astype(np.float32)), side, gc, gs, out)
    t.cuda.synchronize()
    return host(out).astype(np.float64)


def _cfg_check(got, eps, s, side, gc, gs):
    ref = OG.combine(eps, s, side, gc, gs)
    e = eps.astype(np.float64)
    g = OG.gamma(s, gc, gs)[OG.token_map(e.shape[2], e.shape[3], side)]
    bound = CFG_REL * (np.abs(e[1]) + np.abs(g)[None] * np.abs(e[0] - e[1]))
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    assert np.linalg.norm(got - ref) <= CFG_REL * np.linalg.norm(ref)


@pytest.mark.parametrize("name", ["srsu_1024", "traj_3072"])
def test_swcfg_workloads(lib, name):
    w = syn.WORKLOADS[name]
    eps = syn.latent_eps(w)
    s = np.random.default_rng(w.seed).random(w.N).astype(np.float32)
    _cfg_check(_cfg(lib, eps, s, w.side, w.g_ctx, w.g_sens), eps, s.astype(np.float64), w.side, w.g_ctx, w.g_sens)


@pytest.mark.parametrize("C,Hl,Wl,side", [(3, 6, 9, 3), (1, 5, 5, 5), (2, 8, 12, 4), (16, 128, 128, 64)])
def test_swcfg_shapes_and_closed_forms(lib, C, Hl, Wl, side):
    r = np.random.default_rng(C * Hl)
    eps = r.standard_normal((2, C, Hl, Wl)).astype(np.float32)
    s = r.random(side * side).astype(np.float32)
    _cfg_check(_cfg(lib, eps, s, side, 3.0, 6.0), eps, s.astype(np.float64), side, 3.0, 6.0)
    # gamma = 0 gives the unconditional branch exactly; equal scales are global CFG
    assert np.array_equal(_cfg(lib, eps, s, side, 0.0, 0.0), eps[1].astype(np.float64))
    got = _cfg(lib, eps, s, side, 4.5, 4.5)
    _cfg_check(got, eps, np.zeros(side * side), side, 4.5, 4.5)
    # the per-token scale is exactly the global one: every pixel matches the s = 0 launch bit for bit
    assert np.array_equal(got, _cfg(lib, eps, np.zeros_like(s), side, 4.5, 4.5))


# ------------------------------------------------------------------------------------ gather/scatter
@pytest.mark.parametrize("d", [64, 24, 8])  # rows of 8 / 16 chunks (shift indexing), 3 / 6 chunks, 1 / 2 chunks
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k", [0, 1, 77, 300])
def test_gather_scatter_bitwise(lib, dtype, k, d):
    t = torch()
    B, H, N = 2, 3, 300
    r = np.random.default_rng(k)
    tdt = t.bfloat16 if dtype == "bf16" else t.float32
    state = t.from_numpy(r.standard_normal((B, H, N, d)).astype(np.float32)).to(tdt).cuda()
    rows = np.sort(r.choice(N, size=k, replace=False)).astype(np.int32)
    rows_d = dev(rows)
    packed = t.zeros((B, H, k, d), dtype=tdt, device="cuda")
    lib.safe_gather_rows(state, rows_d, packed)
    t.cuda.synchronize()
    ref = state.float().cpu().numpy()
    assert np.array_equal(packed.float().cpu().numpy(), OA.gather_rows(ref, rows))
    canvas = t.full_like(state, 7.0)
    lib.safe_scatter_rows(packed, rows_d, canvas)
    t.cuda.synchronize()
    expect = OA.scatter_rows(np.full(ref.shape, 7.0, dtype=np.float32), OA.gather_rows(ref, rows), rows)
    assert np.array_equal(canvas.float().cpu().numpy(), expect)


# ------------------------------------------------------------------------------------ mask check
def _check(lib, mask: np.ndarray, N, T, tv, want_c=True):
    t = torch()
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    c = t.full((mask.shape[0] * mask.shape[1] * N,), 123.0, dtype=t.float32, device="cuda") if want_c else None
    ok = lib.safe_mask_is_row_constant(dev(mask), N, T, tv, flag, c_out=c)
    return ok, (host(c).astype(np.float64) if want_c else None)


def _same(c_gpu, c_ref):
    nan = np.isnan(c_ref)
    return np.array_equal(np.isnan(c_gpu), nan) and np.array_equal(c_gpu[~nan], c_ref[~nan])


def test_mask_check_random_small(lib):
    r = np.random.default_rng(11)
    N, T = 37, 9
    for trial in range(60):
        tv = tuple(int(x) for x in r.integers(0, T + 1, size=2))
        cols = N if trial % 2 else N + T
        mB, mH = int(r.integers(1, 3)), int(r.integers(1, 4))
        if trial % 3 == 0:
            m = r.random((mB, mH, N, cols)) < 0.995
        else:
            m = np.broadcast_to(r.integers(-2, 3, size=(mB, mH, N, 1)).astype(np.float32), (mB, mH, N, cols)).copy()
            if trial % 3 == 1:
                m[tuple(int(r.integers(0, s)) for s in m.shape)] = r.choice([np.nan, np.inf, -np.inf, 0.5, -0.0])
        ok, c = _check(lib, m, N, T, tv)
        rok, rc = OE.is_row_constant(m, N, T, tv)
        assert ok == rok and _same(c, rc), trial
        ok2, _ = _check(lib, m, N, T, tv, want_c=False)
        assert ok2 == rok


def test_mask_check_launch_matches_the_synchronous_verdict(lib):
    """The launch-only form leaves in its device flag exactly the verdict (and per-row constants) the
    synchronous form returns, also with other work queued on the stream behind it."""
    t = torch()
    r = np.random.default_rng(5)
    N, T = 37, 9
    for trial in range(24):
        tv = tuple(int(x) for x in r.integers(0, T + 1, size=2))
        cols = N if trial % 2 else N + T
        if trial % 3 == 0:
            m = r.random((1, 2, N, cols)) < 0.99
        else:
            m = np.broadcast_to(r.integers(-2, 3, size=(2, 1, N, 1)).astype(np.float32), (2, 1, N, cols)).copy()
            if trial % 3 == 1:
                m[tuple(int(r.integers(0, s)) for s in m.shape)] = 0.25
        ok, c = _check(lib, m, N, T, tv)
        flag = t.full((1,), 7, dtype=t.int32, device="cuda")
        c2 = t.full((m.shape[0] * m.shape[1] * N,), 123.0, dtype=t.float32, device="cuda")
        lib.safe_mask_check_launch(dev(m), N, T, tv, flag, c_out=c2)
        t.cuda.synchronize()
        assert int(host(flag)[0]) == (1 if ok else 0), trial
        assert _same(host(c2).astype(np.float64), c), trial
        flag.fill_(7)
        lib.safe_mask_check_launch(dev(m), N, T, tv, flag)
        t.cuda.synchronize()
        assert int(host(flag)[0]) == (1 if ok else 0), trial
    w = syn.WORKLOADS["dense_1024"]
    big = dev(syn.mask_all_valid_bool(w.N, w.N))
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    lib.safe_mask_check_launch(big, w.N, w.T, w.tv, flag)
    t.cuda.synchronize()
    assert int(host(flag)[0]) == 1


def test_mask_check_dense_1024_all_valid(lib):
    w = syn.WORKLOADS["dense_1024"]
    m = syn.mask_all_valid_bool(w.N, w.N)
    assert _check(lib, m, w.N, w.T, w.tv, want_c=False)[0]
    m[0, 0, 4095, 4095] = False
    assert not _check(lib, m, w.N, w.T, w.tv, want_c=False)[0]
    f = np.zeros((1, 1, w.N, w.N), dtype=np.float32)
    f[0, 0, 17, 3] = -0.0
    ok, c = _check(lib, f, w.N, w.T, w.tv)
    assert ok and np.all(c == 0)
    assert _check(lib, f, w.N, w.T, w.tv, want_c=False)[0]
    f[0, 0, 17, 3] = 1e-30
    ok, c = _check(lib, f, w.N, w.T, w.tv)
    assert not ok and np.isnan(c[17]) and np.sum(np.isnan(c)) == 1
    assert not _check(lib, f, w.N, w.T, w.tv, want_c=False)[0]


def test_mask_check_srsu_2560_all_valid(lib):
    w = syn.WORKLOADS["srsu_2560"]
    m = syn.mask_all_valid_bool(w.N, w.N)
    assert _check(lib, m, w.N, w.T, w.tv, want_c=False)[0]
    m[0, 0, 12345, 25599] = False
    assert not _check(lib, m, w.N, w.T, w.tv, want_c=False)[0]


def test_mask_check_unaligned_row_lengths(lib):
    N, T = 29, 3
    for cols in (N, N + T):
        m = np.zeros((1, 2, N, cols), dtype=np.float32)
        ok, c = _check(lib, m, N, T, (3,))
        assert ok
        assert _check(lib, m, N, T, (3,), want_c=False)[0]
        m[0, 1, 28, cols - 1] = 2.0
        ok, c = _check(lib, m, N, T, (3,))
        assert not ok and np.isnan(c[N + 28])
        assert not _check(lib, m, N, T, (3,), want_c=False)[0]
        mb = np.ones((1, 1, N, cols), dtype=np.bool_)
        mb[0, 0, 3, cols - 1] = False
        for want_c in (True, False):
            assert not _check(lib, mb, N, T, (3,), want_c=want_c)[0]
            assert _check(lib, mb, N, T, (0,), want_c=want_c)[0] == (cols == N + T)


def test_mask_policy_checks_once_per_tensor_version(lib):
    """The host side of "check once, then elide or keep": a redundant mask is dropped, a semantic one is
    kept, the verdict is cached per tensor version, and an in-place edit of the mask is re-checked."""
    t = torch()
    N, T = 96, 16
    pol = lib.MaskPolicy()
    m = t.ones((1, 1, N, N), dtype=t.bool, device="cuda")
    assert pol.elide(m, N, T, (5, 9)) is None
    assert pol.elide(m, N, T, (5, 9)) is None and len(pol._cache) == 1
    m[0, 0, 3, 7] = False  # bumps the tensor version
    assert pol.elide(m, N, T, (5, 9)) is m and len(pol._cache) == 1
    f = t.zeros((1, 1, N, N + T), dtype=t.float32, device="cuda")
    assert pol.elide(f, N, T, (T, T)) is None
    f[0, 0, 1, N + T - 1] = -1.0  # a valid text column of row 1 differs
    assert pol.elide(f, N, T, (T, T)) is f
    assert pol.elide(f, N, T, (T - 1, T - 1)) is None  # that column is padding for these lengths
    assert pol.elide(None, N, T, (T, T)) is None


def test_mask_policy_never_reuses_a_freed_masks_verdict(lib):
    """A verdict is tied to the live tensor it was computed for: after a removable mask is freed, a
    semantic mask of the same shape built without in-place edits (version 0 again) that the caching
    allocator places at the freed address must be checked afresh and kept; dead entries are dropped."""
    import gc
    t = torch()
    N, T = 128, 16
    pol = lib.MaskPolicy()
    reused = 0
    for trial in range(4):
        m1 = t.from_numpy(np.ones((1, 1, N, N), dtype=np.bool_)).cuda()
        assert m1._version == 0 and pol.elide(m1, N, T, (7,)) is None
        addr = m1.data_ptr()
        del m1
        gc.collect()
        assert len(pol._cache) == 0  # the entry went with its tensor
        sem = np.ones((1, 1, N, N), dtype=np.bool_)
        sem[0, 0, 5 + trial, 9] = False  # a semantic (non-uniform) mask
        m2 = t.from_numpy(sem).cuda()
        reused += int(m2.data_ptr() == addr)
        assert m2._version == 0
        assert pol.elide(m2, N, T, (7,)) is m2, trial
        del m2
        gc.collect()
    assert reused > 0, "the allocator never reused the address; the stale-entry case was not exercised"


@pytest.mark.parametrize("dtype", ["bool", "f32"])
def test_mask_check_unaligned_buffer(lib, dtype):
    """A mask whose base is not 16-byte aligned (1 byte past an aligned address for bool, 4 for fp32) and
    whose total length is not a multiple of 16 bytes: the verdict and per-row constants equal the oracle's,
    with the first or the last entry of the buffer deciding (the scan reads those edge blocks byte by byte
    and nothing outside the buffer)."""
    t = torch()
    N, T = 29, 4
    es = 1 if dtype == "bool" else 4
    for cols, tv in ((N, (0,)), (N + T, (4,)), (N + T, (1,))):
        for trial in range(3):
            if dtype == "bool":
                m = np.ones((1, 2, N, cols), dtype=np.bool_)
                bad = False
            else:
                m = np.full((1, 2, N, cols), -1.5, dtype=np.float32)
                bad = np.float32(2.0)
            if trial == 1:
                m[0, 0, 0, 0] = bad                 # first byte(s) of the buffer
            elif trial == 2:
                m[0, 1, N - 1, tv[0] + N - 1 if cols > N else N - 1] = bad  # last checked entry of the buffer
            nbytes = m.size * es
            assert nbytes % 16 != 0
            raw = t.zeros(16 + nbytes + 16, dtype=t.uint8, device="cuda")
            assert raw.data_ptr() % 16 == 0
            raw[es:es + nbytes] = t.from_numpy(m.view(np.uint8).ravel()).cuda()
            view = raw[es:es + nbytes].view(t.bool if dtype == "bool" else t.float32).view(m.shape)
            assert view.data_ptr() % 16 == es
            flag = t.zeros(1, dtype=t.int32, device="cuda")
            c = t.full((2 * N,), 123.0, dtype=t.float32, device="cuda")
            ok = lib.safe_mask_is_row_constant(view, N, T, tv, flag, c_out=c)
            rok, rc = OE.is_row_constant(m, N, T, tv)
            assert ok == rok and _same(host(c).astype(np.float64), rc), (cols, tv, trial)
            assert lib.safe_mask_is_row_constant(view, N, T, tv, flag) == rok, (cols, tv, trial)


def test_concurrent_streams_match_sequential(lib):
    """Two streams running different entry points at once (dense attention and the block products on one,
    sensitive-row attention, PCSP, the partition and SW-CFG on the other) give the results of running them one
    after the other, bit for bit: no call keeps state that another call on another stream could disturb."""
    t = torch()
    w = syn.scaled(syn.WORKLOADS["srsu_1024"], N=1024, side=32, k=300, H=4)
    inp = syn.attention_inputs(w)
    bits = lambda n: t.from_numpy(inp[n + "_bits"].view(np.int16)).view(t.bfloat16).cuda()
    q, ki, vi, kt, vt = (bits(n) for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
    rows = dev(syn.random_rows(w))
    x = syn.pcsp_logits(w)
    xd, lid = dev(x["x"]), dev(x["lse_img"])
    eps = dev(syn.latent_eps(syn.scaled(w, latent=(4, 64, 64))))
    r = np.random.default_rng(5)
    D, F = w.H * w.d, 4 * w.H * w.d
    hx = t.from_numpy(r.standard_normal((w.B, w.N, D)).astype(np.float32)).to(t.bfloat16).cuda()
    w1 = t.from_numpy((r.standard_normal((F, D)) / np.sqrt(D)).astype(np.float32)).to(t.bfloat16).cuda()
    w2 = t.from_numpy((r.standard_normal((D, F)) / np.sqrt(F)).astype(np.float32)).to(t.bfloat16).cuda()
    wq = t.from_numpy((r.standard_normal((3 * D, D)) / np.sqrt(D)).astype(np.float32)).to(t.bfloat16).cuda()
    ws = t.empty(lib.safe_rows_ffn_workspace_bytes(w.B, w.k, F) // 2, dtype=t.bfloat16, device="cuda")
    dense_out, rows_out = t.zeros_like(q), t.zeros_like(q)
    lse = t.empty((w.B, w.H, w.N), dtype=t.float32, device="cuda")
    cache = t.zeros_like(hx)
    pq, pk, pv = t.zeros_like(q), t.zeros_like(q), t.zeros_like(q)
    sc = t.empty(w.N, dtype=t.float32, device="cuda")
    S = t.empty(w.k, dtype=t.int32, device="cuda")
    C = t.empty(w.N - w.k, dtype=t.int32, device="cuda")
    isn = t.empty(w.N, dtype=t.uint8, device="cuda")
    s01 = t.empty(w.N, dtype=t.float32, device="cuda")
    cfg = t.empty(eps.shape[1:], dtype=t.float32, device="cuda")
    outs = (dense_out, lse, cache, pq, pk, pv, rows_out, sc, S, C, isn, s01, cfg)

    def first(stream=None):
        lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, dense_out, lse=lse, stream=stream)
        lib.safe_rows_ffn(hx, rows, w1, None, w2, None, cache, ws, stream=stream)
        lib.safe_rows_qkv(hx, rows, wq, None, pq, pk, pv, stream=stream)

    def second(stream=None):
        lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, rows, rows_out, stream=stream)
        lib.safe_pcsp_accumulate(xd, lid, w.tv[0], 0, w.tv[0], sc, False, stream=stream)
        lib.safe_pcsp_partition(sc, w.k, S, C, isn, s01, stream=stream)
        lib.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg, stream=stream)

    first()
    second()
    t.cuda.synchronize()
    ref = [o.clone() for o in outs]
    sa, sb = t.cuda.Stream(), t.cuda.Stream()
    for rep in range(3):
        for o in outs:
            o.zero_()
        t.cuda.synchronize()
        with t.cuda.stream(sa):
            first(sa)
        with t.cuda.stream(sb):
            second(sb)
        t.cuda.synchronize()
        for i, (o, rf) in enumerate(zip(outs, ref)):
            assert t.equal(o, rf), (rep, i)
