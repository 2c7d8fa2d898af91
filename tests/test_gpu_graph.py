"""The attention step's work after the elision verdict (PCSP aggregation, partition, dense and
sensitive-row attention, gather, scatter, guidance combine) captured once in a HIP graph and replayed:
every replay must equal the eager run bit for bit, both for the sequential capture and for the
two-branch capture the benchmark replays (aggregation, partition and guidance on a second stream beside
the dense attention, joined before the sensitive rows).  Replays are interleaved with eager work and
synchronisations, and every output is poisoned before each replay, so a replay that skipped or reordered a
node would show."""
import numpy as np
import pytest

import synthetic as syn
from tests.gpu_util import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("branched", [False, True], ids=["sequential", "two-branch"])
def test_step_graph_replays_match_eager(lib, branched):
    t = torch()
    w = syn.WORKLOADS["srsu_1024"]
    N, k, Tv = w.N, w.k, w.tv[0]
    inp = syn.attention_inputs(w)
    bf = lambda n: t.from_numpy(inp[n + "_bits"].view(np.int16)).view(t.bfloat16).cuda()
    q, ki, vi, kt, vt = (bf(n) for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
    x = syn.pcsp_logits(w)
    xd, lid = t.from_numpy(x["x"]).cuda(), t.from_numpy(x["lse_img"]).cuda()
    eps = t.from_numpy(syn.latent_eps(w)).cuda()
    state = t.empty_like(q)
    scores = t.empty(N, dtype=t.float32, device="cuda")
    S = t.empty(k, dtype=t.int32, device="cuda")
    C = t.empty(N - k, dtype=t.int32, device="cuda")
    isn = t.empty(N, dtype=t.uint8, device="cuda")
    s01 = t.empty(N, dtype=t.float32, device="cuda")
    packed = t.empty((w.B, w.H, k, w.d), dtype=t.bfloat16, device="cuda")
    cfg = t.empty(eps.shape[1:], dtype=t.float32, device="cuda")
    outs = (scores, S, C, isn, s01, state, packed, cfg)

    def poison():
        for o in outs:
            o.fill_(3 if o.dtype in (t.int32, t.uint8) else -1.5)

    def work():
        lib.safe_pcsp_accumulate(xd, lid, Tv, 0, Tv, scores, False)
        lib.safe_pcsp_partition(scores, k, S, C, isn, s01)
        lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state)
        lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, S, state)
        lib.safe_gather_rows(state, S, packed)
        lib.safe_scatter_rows(packed, S, state)
        lib.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg)

    branch = t.cuda.Stream()

    def work_branched():
        main = t.cuda.current_stream()
        fork = t.cuda.Event()
        fork.record(main)
        lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state)
        branch.wait_event(fork)
        with t.cuda.stream(branch):
            lib.safe_pcsp_accumulate(xd, lid, Tv, 0, Tv, scores, False)
            lib.safe_pcsp_partition(scores, k, S, C, isn, s01)
            lib.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg)
            join = t.cuda.Event()
            join.record(branch)
        main.wait_event(join)
        lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, S, state)
        lib.safe_gather_rows(state, S, packed)
        lib.safe_scatter_rows(packed, S, state)

    poison()
    work()
    t.cuda.synchronize()
    ref = [o.clone() for o in outs]

    g = t.cuda.CUDAGraph()
    poison()
    t.cuda.synchronize()
    with t.cuda.graph(g):
        (work_branched if branched else work)()
    t.cuda.synchronize()
    for rep in range(4):
        poison()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert t.equal(o, r), (rep, i)
        poison()
        work()  # eager work between replays
        t.cuda.synchronize()
        assert t.equal(state, ref[5])


def test_block_products_fp8_and_head_dim_128_replay_match_eager(lib):
    """The other captured entry points: the sensitive-row QKV projection and FFN (workspace and allocation-free
    forms, the latter for callers that capture graphs and cannot allocate), fp8 Q / K attention at head dim 128
    with lse, and bf16 head-dim-128 rows with a kept bool mask; four replays, each equal to the eager run bit for
    bit, with eager work and synchronisations between them."""
    t = torch()
    r = np.random.default_rng(31)
    B, N, H, d, k = 2, 512, 4, 128, 150
    D, F = H * d, 4 * H * d
    bf = lambda a: t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(t.bfloat16).cuda()
    x = bf(r.standard_normal((B, N, D)))
    w1, w2 = bf(r.standard_normal((F, D)) / np.sqrt(D)), bf(r.standard_normal((D, F)) / np.sqrt(F))
    wq = bf(r.standard_normal((3 * D, D)) / np.sqrt(D))
    b1, b2 = t.from_numpy(0.02 * r.standard_normal(F).astype(np.float32)).cuda(), None
    bq = t.from_numpy(0.02 * r.standard_normal(3 * D).astype(np.float32)).cuda()
    rows = t.from_numpy(np.sort(r.choice(N, size=k, replace=False)).astype(np.int32)).cuda()
    ws = t.empty(lib.safe_rows_ffn_workspace_bytes(B, k, F) // 2, dtype=t.bfloat16, device="cuda")
    w8 = syn.scaled(syn.WORKLOADS["dense_1024"], side=1, B=B, H=H, N=N, T=64, tv=(40, 64), d=d)
    inp8 = syn.attention_inputs_fp8(w8)
    f8 = lambda c: t.from_numpy(np.ascontiguousarray(c)).view(t.float8_e4m3fn).cuda()
    q8, k8, kt8 = f8(inp8["q_fp8"]), f8(inp8["k_img_fp8"]), f8(inp8["k_txt_fp8"])
    bits = lambda n: t.from_numpy(inp8[n + "_bits"].view(np.int16)).view(t.bfloat16).cuda()
    vi, vt = bits("v_img"), bits("v_txt")
    qd = t.from_numpy(inp8["q_descale"].reshape(-1).astype(np.float32)).cuda()
    kd = t.from_numpy(inp8["k_descale"].reshape(-1).astype(np.float32)).cuda()
    mask = t.from_numpy(r.random((1, H, N, N + 64)) < 0.8).cuda()
    qb, kb = bf(inp8["q"]), bf(inp8["k_img"])
    ktb = bf(inp8["k_txt"])
    q = t.empty((B, H, N, d), dtype=t.bfloat16, device="cuda")
    kc, vc = t.empty_like(q), t.empty_like(q)
    cache, cache2 = t.empty_like(x), t.empty_like(x)
    o8, ob = t.empty((B, H, N, d), dtype=t.bfloat16, device="cuda"), t.empty((B, H, N, d), dtype=t.bfloat16, device="cuda")
    lse8 = t.empty((B, H, N), dtype=t.float32, device="cuda")
    outs = (q, kc, vc, cache, cache2, o8, ob, lse8)

    def poison():
        for o in outs:
            o.fill_(-1.5)

    def work():
        lib.safe_rows_qkv(x, rows, wq, bq, q, kc, vc)
        lib.safe_rows_ffn(x, rows, w1, b1, w2, b2, cache, ws)
        lib.safe_rows_ffn_noalloc(x, rows, w1, b1, w2, b2, cache2)
        lib.safe_attn_dense(q8, k8, vi, kt8, vt, w8.tv, o8, lse=lse8, q_descale=qd, k_descale=kd)
        lib.safe_attn_rows(qb, kb, vi, ktb, vt, w8.tv, rows, ob, mask=mask)

    poison()
    work()
    t.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert t.equal(cache, cache2)  # the two FFN forms share their kernels

    g = t.cuda.CUDAGraph()
    poison()
    t.cuda.synchronize()
    with t.cuda.graph(g):
        work()
    t.cuda.synchronize()
    for rep in range(4):
        poison()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for i, (o, rf) in enumerate(zip(outs, ref)):
            assert t.equal(o, rf), (rep, i)
        poison()
        work()
        t.cuda.synchronize()
