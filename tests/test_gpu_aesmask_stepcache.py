"""GPU parity of the AesMask affinity and mask and of the StepCache extrapolation and trajectory."""
import numpy as np
import pytest

import synthetic as syn
from oracle import aesmask as OA
from oracle import pcsp as OP
from oracle import stepcache as OSC
from tests.gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu


def _affinity(lib, x, lse_img, tv, sel, prev=None, sel_offset=0):
    t = torch()
    sc = dev(prev.astype(np.float32)) if prev is not None else t.full((x.shape[1],), np.nan, dtype=t.float32, device="cuda")
    if sel_offset:
        # a selection that starts 1 byte into its allocation (not 4-byte aligned): the per-slot byte path
        buf = t.zeros(sel.shape[0] + sel_offset, dtype=t.uint8, device="cuda")
        buf[sel_offset:] = dev(sel)
        sd = buf[sel_offset:]
    else:
        sd = dev(sel)
    lib.safe_affinity_accumulate(dev(x), dev(lse_img) if lse_img is not None else None, tv, sd, sc, prev is not None)
    t.cuda.synchronize()
    return host(sc).astype(np.float64)


@pytest.mark.parametrize("T,tv,pattern,sel_offset", [
    (256, 77, "sparse", 0), (256, 77, "all", 0), (256, 77, "none", 0), (256, 77, "padding-only", 0),
    (64, 64, "sparse", 0), (256, 200, "sparse", 0), (256, 256, "sparse", 0),
    (256, 77, "sparse", 1),            # unaligned selection: the generic kernel
    (37, 20, "sparse", 0), (300, 255, "sparse", 0), (8, 0, "all", 0)])
def test_affinity_parity(lib, T, tv, pattern, sel_offset):
    r = np.random.default_rng(T * 3 + tv)
    H, N = 5, 333
    x = (r.standard_normal((H, N, T)) * 2).astype(np.float32)
    x[:, :, tv:] = 1e30  # padded slots must never count
    li = (r.standard_normal((H, N)) + 4).astype(np.float32)
    sel = {"sparse": (r.random(T) < 0.2), "all": np.ones(T, bool), "none": np.zeros(T, bool),
           "padding-only": np.arange(T) >= tv}[pattern].astype(np.uint8)
    for lse_img in (li, None):
        got = _affinity(lib, x, lse_img, tv, sel, sel_offset=sel_offset)
        ref = OA.affinity(x, lse_img, tv, sel)
        assert np.all(np.abs(got - ref) <= 5e-6 * np.abs(ref) + 1e-37), (pattern, lse_img is None)
    prev = r.random(N).astype(np.float32)
    got = _affinity(lib, x, li, tv, sel, prev=prev, sel_offset=sel_offset)
    ref = prev.astype(np.float64) + OA.affinity(x, li, tv, sel)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-30)) < 5e-6


def test_affinity_with_range_selection_equals_pcsp_scores(lib):
    """A selection that is a contiguous range gives the PCSP kernel's scores (same kernel family)."""
    r = np.random.default_rng(5)
    x = (r.standard_normal((4, 500, 256)) * 2).astype(np.float32)
    li = (r.standard_normal((4, 500)) + 4).astype(np.float32)
    sel = np.zeros(256, np.uint8)
    sel[10:50] = 1
    t = torch()
    a = t.zeros(500, dtype=t.float32, device="cuda")
    b = t.zeros(500, dtype=t.float32, device="cuda")
    lib.safe_affinity_accumulate(dev(x), dev(li), 77, dev(sel), a, False)
    lib.safe_pcsp_accumulate(dev(x), dev(li), 77, 10, 50, b, False)
    t.cuda.synchronize()
    assert np.array_equal(host(a), host(b))


def _mask(lib, a32, k):
    t = torch()
    N = a32.shape[0]
    S = t.full((max(k, 1),), -7, dtype=t.int32, device="cuda")
    C = t.full((max(N - k, 1),), -7, dtype=t.int32, device="cuda")
    isn = t.full((N,), 9, dtype=t.uint8, device="cuda")
    lib.safe_pcsp_partition(dev(a32), k, S, C, isn)
    t.cuda.synchronize()
    return host(S)[:k], host(isn)


@pytest.mark.parametrize("name,pct_bp", [("srsu_1024", 8000), ("srsu_1024", 5000), ("srsu_2560", 9000)])
def test_aesmask_end_to_end(lib, name, pct_bp):
    """GPU affinity (fp32) -> percentile count -> GPU partition: bit-exact against the oracle's partition
    of the same fp32 scores, and equal to the fp64 oracle's mask except for tokens within the fp32 score
    error of the threshold."""
    w = syn.WORKLOADS[name]
    inp = syn.pcsp_logits(w, 0)
    sel = syn.aesthetic_selection(w)
    t = torch()
    sc = t.zeros(w.N, dtype=t.float32, device="cuda")
    lib.safe_affinity_accumulate(dev(inp["x"]), dev(inp["lse_img"]), w.tv[0], dev(sel), sc, False)
    t.cuda.synchronize()
    a_gpu = host(sc)
    a_ref = OA.affinity(inp["x"], inp["lse_img"], w.tv[0], sel)
    del inp
    rel = float(np.max(np.abs(a_gpu - a_ref) / a_ref))
    assert rel < 2e-6
    k = lib.safe_percentile_count(w.N, pct_bp)
    assert k == OA.percentile_count(w.N, pct_bp)
    S, isn = _mask(lib, a_gpu, k)
    rS, _, risn, _ = OP.partition(a_gpu.astype(np.float64), k)
    assert np.array_equal(S, rS) and np.array_equal(isn, risn)
    k2, fS, fmask = OA.mask(a_ref, pct_bp)
    o = OP.order(a_ref)
    thr = a_ref[o[k - 1]]
    diff = np.flatnonzero(isn != fmask)
    print(f"{name} p={pct_bp / 100}: k={k}, fp32 rel err {rel:.2e}, tokens differing from fp64 {len(diff)}")
    assert np.all(np.abs(a_ref[diff] - thr) <= 4 * rel * thr)


@pytest.mark.parametrize("n,offset", [(0, 0), (1, 0), (3, 0), (4, 0), (5, 0), (1023, 0), (4099, 0),
                                      (100003, 0), (4099, 1), (2 * 16 * 384 * 384, 0)])
def test_stepcache_extrapolate_parity(lib, n, offset):
    t = torch()
    r = np.random.default_rng(n + offset)
    a = r.standard_normal(n + offset).astype(np.float32)
    b = (a + 0.1 * r.standard_normal(n + offset)).astype(np.float32)
    da, db = dev(a)[offset:], dev(b)[offset:]  # offset 1: pointers not 16-byte aligned, the scalar kernel
    out = t.full((n + offset,), np.nan, dtype=t.float32, device="cuda")[offset:]
    for w in (0.0, 1.0 / 3.0, 0.75, -1.0, 2.5):
        lib.safe_stepcache_extrapolate(da, db, w, out)
        t.cuda.synchronize()
        got = host(out).astype(np.float64)
        ref = OSC.extrapolate(a[offset:], b[offset:], np.float32(w))
        scale = np.abs(b[offset:]) + abs(float(np.float32(w))) * np.abs(b[offset:].astype(np.float64) - a[offset:])
        assert np.all(np.abs(got - ref) <= 1e-6 * scale + 1e-37), w
        if w == 0.0:
            assert np.array_equal(host(out), b[offset:])
    # out may alias eps_b
    if n:
        lib.safe_stepcache_extrapolate(da, db, 0.5, db)
        t.cuda.synchronize()
        ref = OSC.extrapolate(a[offset:], b[offset:], 0.5)
        assert np.max(np.abs(host(db) - ref)) <= 1e-6 * (np.max(np.abs(ref)) + 1)


def test_stepcache_plan_and_trajectory(lib):
    """The library's plan equals the oracle's, and a StepCache trajectory of the 3072^2 latent built from
    the plan and the GPU extrapolation matches the oracle's trajectory."""
    w = syn.WORKLOADS["traj_3072"]
    steps, delta = 10, 3
    plan = lib.safe_stepcache_plan(steps, delta)
    ref_plan = OSC.plan(steps, delta)
    for (f, a, b, wt), (rf, ra, rb, rw) in zip(plan, ref_plan):
        assert (f, a, b) == (rf, ra, rb) and wt == np.float32(rw)
    preds = syn.stepcache_predictions(w, steps)
    t = torch()
    full = {}
    out = []
    for s, (f, a, b, wt) in enumerate(plan):
        if f:
            full[s] = dev(preds[s])
            out.append(host(full[s]).astype(np.float64))
        else:
            o = t.empty(preds[s].shape, dtype=t.float32, device="cuda")
            lib.safe_stepcache_extrapolate(full[a], full[b], wt, o)
            t.cuda.synchronize()
            out.append(host(o).astype(np.float64))
    ref = OSC.run(lambda s: preds[s], steps, delta)
    for s in range(steps):
        scale = np.max(np.abs(ref[s])) + 1.0
        assert np.max(np.abs(out[s] - ref[s])) <= 2e-6 * scale, s
