"""The warmup / anchor / sensitive-row trajectory on the GPU against the oracle's schedule."""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention as OA
from oracle import pcsp as OP
from oracle import schedule as OS
from tests.gpu_util import assert_close, attn_tensors, dev, host, torch

pytestmark = pytest.mark.gpu


def _gpu_trajectory(lib, w, step_inputs, warm, state0, scores_out=None):
    t = torch()
    sc = t.zeros(w.N, dtype=t.float32, device="cuda")
    for i, (x, li) in enumerate(warm):
        lib.safe_pcsp_accumulate(dev(x), dev(li), w.tv[0], 0, w.tv[0], sc, i > 0)
    S = t.zeros(w.k, dtype=t.int32, device="cuda")
    C = t.zeros(w.N - w.k, dtype=t.int32, device="cuda")
    isn = t.zeros(w.N, dtype=t.uint8, device="cuda")
    lib.safe_pcsp_partition(sc, w.k, S, C, isn)
    if scores_out is not None:
        scores_out.append(host(sc))
    state = t.from_numpy(state0).to(t.bfloat16).cuda()
    snaps = []
    # the library's own plan (checked against the oracle's on the CPU) orders the launches
    for step, kind in enumerate(lib.safe_trajectory_plan(w.steps, w.anchor_every)):
        q, ki, vi, kt, vt = step_inputs(step)
        if kind == lib.SAFE_STEP_DENSE:
            lib.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state)
        else:
            lib.safe_attn_rows(q, ki, vi, kt, vt, w.tv, S, state)
        snaps.append(state.clone())
    t.cuda.synchronize()
    return state, host(S), snaps


def test_small_trajectory_matches_oracle(lib):
    w = syn.scaled(syn.WORKLOADS["traj_3072"], N=400, side=20, k=80, H=2, n_blobs=2, blob_sigma=3.0)
    inputs = [syn.attention_inputs(w, step=s) for s in range(w.steps)]
    warm = [(lambda d: (d["x"], d["lse_img"]))(syn.pcsp_logits(w, s)) for s in range(w.warmup_steps)]
    state0 = syn.initial_state(w)
    st, S, _ = _gpu_trajectory(lib, w, lambda s: attn_tensors(inputs[s], "bf16"), warm, state0)
    ref, rS, _, kinds = OS.run(state0, warm, lambda s: tuple(inputs[s][n] for n in ("q", "k_img", "v_img", "k_txt", "v_txt")),
                               w.k, w.steps, w.anchor_every, w.tv, 0, w.tv[0])
    assert np.array_equal(S, rS)
    assert_close(host(st), ref, "bf16", "trajectory")


def test_full_size_trajectory_keeps_context_rows(lib):
    """At 3072^2 (N = 36864): after 10 steps the context rows hold the last anchor's output bitwise."""
    w = syn.WORKLOADS["traj_3072"]
    t = torch()
    g = t.Generator(device="cuda")

    def step_inputs(step):
        g.manual_seed(1000 + step)
        mk = lambda n: (t.randn((w.B, w.H, n, w.d), generator=g, device="cuda") * w.std).to(t.bfloat16)
        return mk(w.N), mk(w.N), mk(w.N), mk(w.T), mk(w.T)

    warm = [(lambda d: (d["x"], d["lse_img"]))(syn.pcsp_logits(w, s)) for s in range(w.warmup_steps)]
    state0 = np.zeros((w.B, w.H, w.N, w.d), dtype=np.float32)
    st, S, snaps = _gpu_trajectory(lib, w, step_inputs, warm, state0)
    C = t.as_tensor(np.setdiff1d(np.arange(w.N), S), device="cuda")
    Sd = t.as_tensor(S.astype(np.int64), device="cuda")
    assert t.equal(st[:, :, C], snaps[8][:, :, C])   # last anchor at step 8
    assert t.equal(st[:, :, Sd], snaps[9][:, :, Sd])
    assert not t.equal(snaps[9][:, :, Sd], snaps[8][:, :, Sd])


@pytest.mark.parametrize("i", range(6), ids=lambda i: f"case{i}")
def test_random_trajectory_matches_oracle_composition(lib, i):
    """Seeded random trajectories (grid size, |S|, heads, step count, anchor period, warmup length, text lengths):
    the partition is bit-exact on the GPU's own fp32 scores, the launch order follows the oracle's plan, and the
    final state equals the oracle's composition of dense and sensitive-row steps with that partition."""
    r = np.random.default_rng(12500 + i)
    side = int(r.integers(6, 25))
    N = side * side
    w = syn.scaled(syn.WORKLOADS["traj_3072"], N=N, side=side, k=int(r.integers(1, N + 1)), H=int(r.integers(1, 4)),
                   T=int(r.choice([16, 77, 128])), steps=int(r.integers(1, 9)), anchor_every=int(r.integers(1, 6)),
                   warmup_steps=int(r.integers(1, 4)), n_blobs=2, blob_sigma=3.0, seed=12500 + i)
    w = syn.scaled(w, tv=tuple(int(x) for x in r.integers(1, w.T + 1, size=w.B)))
    assert [lib.SAFE_STEP_DENSE if kd == "dense" else lib.SAFE_STEP_ROWS for kd in OS.plan(w.steps, w.anchor_every)] \
        == lib.safe_trajectory_plan(w.steps, w.anchor_every)
    inputs = [syn.attention_inputs(w, step=s) for s in range(w.steps)]
    warm = [(lambda d: (d["x"], d["lse_img"]))(syn.pcsp_logits(w, s)) for s in range(w.warmup_steps)]
    state0 = syn.initial_state(w)
    scores = []
    st, S, _ = _gpu_trajectory(lib, w, lambda s: attn_tensors(inputs[s], "bf16"), warm, state0, scores)
    assert np.array_equal(S, OP.partition(scores[0].astype(np.float64), w.k)[0]), (i, w.N, w.k)
    ref = np.asarray(state0, dtype=np.float64)
    for step, kind in enumerate(OS.plan(w.steps, w.anchor_every)):
        args = tuple(inputs[step][n] for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
        ref = OA.dense_step(ref, *args, tv=w.tv) if kind == "dense" else OA.rows_step(ref, S, *args, tv=w.tv)
    assert_close(host(st), ref, "bf16", f"trajectory case{i}")
