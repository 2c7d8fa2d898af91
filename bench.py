#!/usr/bin/env python3
"""Benchmark of one pass of the spatially-adaptive DiT attention step on one MI355X.

A step runs every stage of the hot path once over the 1024^2-latent workload (B = 2 cond/uncond,
H = 24, d = 64, N = 4096 image tokens, T = 256 text slots with 77 valid, |S| = 1229):
  elision check of the redundant all-valid image mask -> PCSP aggregation of the warmup
  cross-attention logits -> exact top-|S| partition -> dense anchor attention (all rows) ->
  sensitive-row attention (rows of S, scattered into the cached state) -> stand-alone gather and
  scatter of the S rows -> SW-CFG on the 2x16x128x128 latent.
Inputs are seeded synthetic tensors already resident in HBM.  The reported value is attention
TFLOP/s over the whole step (dense + sensitive-row algorithmic flops, 4*rows*(N+Tv)*d per head,
divided by the wall time of the whole step).  Each step's elision check runs on a side stream, launched
two steps ahead (the mask is a step input; the host reads the verdict when it launches the step), and the
rest of the step is replayed from a HIP graph of the stages in order; per-kernel durations come from HIP
events in an eager pass of the same steps.

Prints ONE JSON line.  --gpus above 1 exits with a message: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed graph steps before the timed ones (the step time settles over the first ~100-300)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the oracle sample")
    ap.add_argument("--no-large", action="store_true", help="skip the 2560^2 attention lines")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the attention step runs on exactly one GPU; "
              "--gpus above 1 is not supported (no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import diffusion_transformer_spatially_amd as dts
    import synthetic as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dts.load()
    dev = torch.device("cuda:0")
    w = syn.WORKLOADS["srsu_1024"]
    B, H, N, T, d, k = w.B, w.H, w.N, w.T, w.d, w.k
    Tv = w.tv[0]

    # ---------------------------------------------------------------- inputs (seeded, resident in HBM)
    inp = syn.attention_inputs(w)
    bf = lambda n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
    q, ki, vi, kt, vt = (bf(n) for n in ("q", "k_img", "v_img", "k_txt", "v_txt"))
    x = syn.pcsp_logits(w)
    xd = torch.from_numpy(x["x"]).to(dev)
    lid = torch.from_numpy(x["lse_img"]).to(dev)
    eps = torch.from_numpy(syn.latent_eps(w)).to(dev)
    mask = torch.ones((1, 1, N, N), dtype=torch.bool, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    state = torch.zeros_like(q)
    scores = torch.zeros(N, dtype=torch.float32, device=dev)
    S = torch.zeros(k, dtype=torch.int32, device=dev)
    C = torch.zeros(N - k, dtype=torch.int32, device=dev)
    isn = torch.zeros(N, dtype=torch.uint8, device=dev)
    s01 = torch.zeros(N, dtype=torch.float32, device=dev)
    packed = torch.empty((B, H, k, d), dtype=torch.bfloat16, device=dev)
    cfg_out = torch.empty(eps.shape[1:], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    stages = ["mask_check", "pcsp_accumulate", "pcsp_partition", "attn_dense", "attn_rows", "gather_rows",
              "scatter_rows", "swcfg_combine"]
    ev = {s: [] for s in stages}
    # The elision check is synchronous (its verdict decides, on the host, which attention kernel runs),
    # so it runs on a second stream of default priority: it overlaps the previous step's work still
    # queued on the main stream, and its host round trip is hidden behind that work.
    side = torch.cuda.Stream(device=dev)

    def check():
        return dts.safe_mask_is_row_constant(mask, N, T, w.tv, flag, stream=side)

    def work(m, mark):
        """Everything after the verdict, on the current stream."""
        mark("pcsp_accumulate", lambda: dts.safe_pcsp_accumulate(xd, lid, Tv, 0, Tv, scores, False))
        mark("pcsp_partition", lambda: dts.safe_pcsp_partition(scores, k, S, C, isn, s01))
        mark("attn_dense", lambda: dts.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state, mask=m))
        mark("attn_rows", lambda: dts.safe_attn_rows(q, ki, vi, kt, vt, w.tv, S, state, mask=m))
        mark("gather_rows", lambda: dts.safe_gather_rows(state, S, packed))
        mark("scatter_rows", lambda: dts.safe_scatter_rows(packed, S, state))
        mark("swcfg_combine", lambda: dts.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg_out))

    # Headline: the work of a step after the verdict is one HIP graph (captured once per verdict, outside
    # the timed region) replayed after each step's check, which removes the per-kernel launch gaps; its
    # kernels run in stage order on one stream.  A second graph puts PCSP aggregation, the partition and
    # SW-CFG on a branch beside the dense anchor attention (none of them reads the anchor's output; the
    # sensitive rows, gather and scatter wait for both branches); it is timed as a side line.
    graphs = {}
    branch = torch.cuda.Stream(device=dev)

    def work_overlapped(m):
        main = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(main)
        dts.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state, mask=m)
        branch.wait_event(fork)
        with torch.cuda.stream(branch):
            dts.safe_pcsp_accumulate(xd, lid, Tv, 0, Tv, scores, False)
            dts.safe_pcsp_partition(scores, k, S, C, isn, s01)
            dts.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg_out)
            join = torch.cuda.Event()
            join.record(branch)
        main.wait_event(join)
        dts.safe_attn_rows(q, ki, vi, kt, vt, w.tv, S, state, mask=m)
        dts.safe_gather_rows(state, S, packed)
        dts.safe_scatter_rows(packed, S, state)

    # The mask is an input of the step, known before the step starts, so each step's elision check is
    # launched two steps ahead: the launch-only check leaves its verdict in a device flag, an asynchronous
    # copy brings it to pinned host memory, and the host reads it (after the check's event) when it
    # launches the step.  Checks run on the side stream beside the graphs; the host never waits for the
    # GPU to drain before queueing the next step.  Two checks are launched before the warm-up steps.
    ring = 2
    flags = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(ring)]
    verdicts = [torch.zeros(1, dtype=torch.int32, pin_memory=True) for _ in range(ring)]
    checked = [torch.cuda.Event() for _ in range(ring)]
    step_no = [0]

    def launch_check(slot):
        dts.safe_mask_check_launch(mask, N, T, w.tv, flags[slot], stream=side)
        with torch.cuda.stream(side):
            verdicts[slot].copy_(flags[slot], non_blocking=True)
            checked[slot].record(side)

    def graph_step(overlapped=False):
        slot = step_no[0] % ring
        step_no[0] += 1
        checked[slot].synchronize()
        elided = bool(int(verdicts[slot][0]))
        key = (elided, overlapped)
        if key not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                if overlapped:
                    work_overlapped(None if elided else mask)
                else:
                    work(None if elided else mask, lambda name, fn: fn())
            graphs[key] = g
        graphs[key].replay()
        launch_check(slot)  # the check of the step `ring` steps ahead

    def eager_step(record: bool):
        def mark(name, fn, on=None):
            on = on or torch.cuda.current_stream()
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(on)
                fn()
                e1.record(on)
                ev[name].append((e0, e1))
            else:
                fn()
        elided = []
        if record:
            # no overlap in the timed eager pass: each kernel's events see it alone on the GPU; the
            # spin keeps the main-stream launches queued so their events time the kernels themselves
            torch.cuda.current_stream().synchronize()
            gpu_busy(torch, 1.0)
        mark("mask_check", lambda: elided.append(check()), on=side)
        work(None if elided[0] else mask, mark)

    # Per-kernel durations first: HIP events around each launch on its stream, in an eager pass of the
    # same steps (events cannot sit inside the graph), with each step's check started only once the
    # previous step's kernels have finished, so that no kernel shares the GPU with another.  This pass
    # also brings the GPU to its working clock before the timed graph steps (the first few dozen steps
    # after an idle GPU run slower).
    for _ in range(args.warmup):
        eager_step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        eager_step(True)
    torch.cuda.synchronize()
    avg_ms = {s: float(np.median([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}  # median per launch
    kernel_ms_sum = sum(avg_ms[s] for s in stages if s != "mask_check")

    # Headline: W untimed warm-up steps, then exactly K timed steps of the graph path.
    for slot in range(ring):
        launch_check(slot)
    for _ in range(args.warmup):
        graph_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps

    # The same steps from the two-branch graph.
    for _ in range(min(args.warmup, 50)):
        graph_step(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph_step(True)
    torch.cuda.synchronize()
    ms_per_step_branched = 1e3 * (time.perf_counter() - t0) / args.steps

    attn_flops = w.flops_dense + w.flops_rows
    value = attn_flops / (ms_per_step * 1e-3) / 1e12

    # algorithmic work per launch
    dense_tf = w.flops_dense / (avg_ms["attn_dense"] * 1e-3) / 1e12
    rows_tf = w.flops_rows / (avg_ms["attn_rows"] * 1e-3) / 1e12
    pcsp_bytes = 4.0 * H * N * Tv + 4.0 * H * N + 4.0 * N
    C_, Hl, Wl = w.latent
    cfg_bytes = 3 * 4.0 * C_ * Hl * Wl + 4.0 * N
    gs_bytes = 2 * 2.0 * B * H * k * d
    mask_bytes = 1.0 * N * N
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    hbm = lambda b, ms: {"ms": ms, "gbs": gbs(b, ms), "frac_hbm": gbs(b, ms) / HBM_PEAK_GBS, "bytes": b}
    breakdown = {
        "attn_dense": {"ms": avg_ms["attn_dense"], "tflops": dense_tf, "frac_mfma": dense_tf / MFMA_BF16_PEAK_TFLOPS},
        "attn_rows": {"ms": avg_ms["attn_rows"], "tflops": rows_tf, "frac_mfma": rows_tf / MFMA_BF16_PEAK_TFLOPS},
        "pcsp_accumulate": hbm(pcsp_bytes, avg_ms["pcsp_accumulate"]),
        "pcsp_partition": {"ms": avg_ms["pcsp_partition"], "note": "one workgroup: latency-bound, no roofline"},
        "swcfg_combine": hbm(cfg_bytes, avg_ms["swcfg_combine"]),
        "gather_rows": hbm(gs_bytes, avg_ms["gather_rows"]),
        "scatter_rows": hbm(gs_bytes, avg_ms["scatter_rows"]),
        "mask_check": dict(hbm(mask_bytes, avg_ms["mask_check"]),
                           note="synchronous (host verdict), includes the device-to-host copy"),
        "stat": "median over the timed launches",
    }

    # Cold mode: each HBM-bound stage of the step with L2 and MALL swept by a 1 GiB write before the launch
    # (the step's own working set, tens of MB, otherwise stays in the 256 MB MALL from step to step).
    flush = torch.empty(256 << 20, dtype=torch.float32, device=dev)
    cold = {
        "pcsp_accumulate": cold_line(hbm, pcsp_bytes, cold_launch_ms(
            torch, lambda: dts.safe_pcsp_accumulate(xd, lid, Tv, 0, Tv, scores, False), flush)),
        "gather_rows": cold_line(hbm, gs_bytes, cold_launch_ms(
            torch, lambda: dts.safe_gather_rows(state, S, packed), flush)),
        "scatter_rows": cold_line(hbm, gs_bytes, cold_launch_ms(
            torch, lambda: dts.safe_scatter_rows(packed, S, state), flush)),
        "swcfg_combine": cold_line(hbm, cfg_bytes, cold_launch_ms(
            torch, lambda: dts.safe_swcfg_combine(eps, s01, w.side, w.g_ctx, w.g_sens, cfg_out), flush)),
        "mask_scan": cold_line(hbm, mask_bytes, cold_launch_ms(
            torch, lambda: dts.safe_mask_check_launch(mask, N, T, w.tv, flags[0]), flush)),
        "note": "1024^2 step shapes; a 1 GiB write and a 1 GiB read sweep L2 and MALL before each launch; one event "
                "pair per launch, the median of an empty pair after the same sweep subtracted (ms_raw, event_pair_ms)",
    }
    del flush

    sclk = profiled_traffic("sclk_mhz")
    peak_sclk = 256 * 4 * 1024 * sclk / 1e6 if sclk else None  # TFLOP/s
    result = {
        "metric": "attention TFLOP/s + % bf16 MFMA peak (dense & |S|-row) at N=4096/25600",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "kernel_ms_sum": kernel_ms_sum,
        "timing": "wall clock of K whole steps (each step: its elision check, launched two steps ahead on a "
                  "side stream, and a graph replay of the rest, every stage in order on one stream); kernel "
                  "durations and the roofline from HIP events in an eager pass of the same steps, run "
                  "without overlap between steps, each step's launches queued behind a spin so that the "
                  "events time the kernels; kernel_ms_sum adds the main-stream kernels' medians",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.125 Q/K/V, blob-biased cross-attention logits, N(0,1) latents)",
        "config": {"workload": "srsu_1024: 1024^2 latent, B=2, H=24, d=64, N=4096, T=256 (Tv=77), |S|=1229, "
                               "SW-CFG 2x16x128x128", "attention_flops_per_step": attn_flops},
        "roofline": {"bound": "mfma", "achieved": dense_tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": dense_tf / MFMA_BF16_PEAK_TFLOPS, "traffic": profiled_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                     "kernel": "k_attn_mfma<false, 2, false, 0, 1, 64> (dense anchor attention)",
                     "flops_per_launch": w.flops_dense, "avg_launch_ms": avg_ms["attn_dense"],
                     "sclk_mhz": sclk, "peak_at_sclk": peak_sclk,
                     "frac_at_sclk": (dense_tf / peak_sclk) if peak_sclk else None,
                     "sclk_note": "shader clock during this kernel from the profile's GRBM_COUNT pass; "
                                  "peak_at_sclk = 256 CU x 4 SIMD x 1024 flop/clk x sclk"},
        "breakdown": breakdown,
        "hbm_cold": cold,
        "step_branched": {"ms_per_step": ms_per_step_branched,
                          "value": attn_flops / (ms_per_step_branched * 1e-3) / 1e12,
                          "note": "the same steps from a graph that runs PCSP, partition and SW-CFG on a branch beside "
                                  "the dense anchor attention (the headline graph runs every stage in order)"},
    }

    # ---------------------------------------------------------------- the mask tax on this stack
    # The redundant all-valid mask passed through (kept) instead of elided: the dense anchor launch with
    # the mask streamed from HBM into the same MFMA kernel, bool and fp32.
    fmask = torch.zeros((1, 1, N, N), dtype=torch.float32, device=dev)
    tax = {"dense_elided_ms": time_launches(torch, lambda: dts.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state)),
           "dense_kept_bool_ms": time_launches(torch, lambda: dts.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state,
                                                                                  mask=mask)),
           "dense_kept_f32_ms": time_launches(torch, lambda: dts.safe_attn_dense(q, ki, vi, kt, vt, w.tv, state,
                                                                                 mask=fmask))}
    tax["tax_bool"] = tax["dense_kept_bool_ms"] / tax["dense_elided_ms"]
    tax["tax_f32"] = tax["dense_kept_f32_ms"] / tax["dense_elided_ms"]
    tax["workload"] = "srsu_1024 dense anchor; mask [1,1,4096,4096] all valid (16.8 MB bool / 67.1 MB fp32)"
    del fmask

    # ---------------------------------------------------------------- 2560^2 attention (same kernels)
    if not args.no_large:
        wl = syn.WORKLOADS["srsu_2560"]
        lq, lki, lvi, lkt, lvt, lrows, lout, line = attention_large(dts, torch, syn, dev, wl, stream)
        result["attention_2560"] = line
        result["hbm_large"] = hbm_large(dts, torch, np, syn, dev, lout, lrows, hbm)
        lmask = torch.ones((1, 1, wl.N, wl.N), dtype=torch.bool, device=dev)  # 655 MB
        kept = time_launches(torch, lambda: dts.safe_attn_dense(lq, lki, lvi, lkt, lvt, wl.tv, lout, mask=lmask), reps=3)
        tax["dense_2560_elided_ms"] = line["dense_ms"]
        tax["dense_2560_kept_bool_ms"] = kept
        tax["tax_2560_bool"] = kept / line["dense_ms"]
        # the elision check itself on the 655 MB bool mask (verdict only, launch form, device flag)
        lflag = torch.zeros(1, dtype=torch.int32, device=dev)
        chk = {"bool_ms": time_launches(torch, lambda: dts.safe_mask_check_launch(lmask, wl.N, wl.T, wl.tv, lflag),
                                        reps=5)}
        del lmask
        lfmask = torch.zeros((1, 1, wl.N, wl.N), dtype=torch.float32, device=dev)  # 2.6 GB
        chk["f32_ms"] = time_launches(torch, lambda: dts.safe_mask_check_launch(lfmask, wl.N, wl.T, wl.tv, lflag),
                                      reps=5)
        kept32 = time_launches(torch, lambda: dts.safe_attn_dense(lq, lki, lvi, lkt, lvt, wl.tv, lout, mask=lfmask),
                               reps=2)
        tax["dense_2560_kept_f32_ms"] = kept32
        tax["tax_2560_f32"] = kept32 / line["dense_ms"]
        del lfmask
        nb = float(wl.N) * wl.N
        chk.update({"bool_frac_hbm": nb / (chk["bool_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "f32_frac_hbm": 4 * nb / (chk["f32_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "workload": "srsu_2560 all-valid image mask [1,1,25600,25600]: 655 MB bool / 2.62 GB fp32 zeros; "
                                "verdict-only scan, 5 back-to-back launches"})
        result["mask_check_2560"] = chk
        del lq, lki, lvi, lkt, lvt, lout, lrows
        result["attention_3072"] = attention_large(dts, torch, syn, dev, syn.WORKLOADS["traj_3072"], stream,
                                                   reps=3)[-1]

    result["mask_tax"] = tax
    # head dim 128 at the 1024^2 grid (24 heads x 128): the same path at the other head dim the library takes
    result["attention_d128_1024"] = attention_large(dts, torch, syn, dev, syn.WORKLOADS["dense_1024_d128"], stream,
                                                    reps=10)[-1]
    result["aesmask_stepcache"] = next_rows(dts, torch, np, syn, dev, hbm, not args.no_large)
    result["srsu_block"] = srsu_block(dts, torch, np, syn, dev)

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}

    # ---------------------------------------------------------------- oracle on the host cores
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        result["cpu_oracle_other_stages"] = cpu_other_stages(w, x, syn)
    print(json.dumps(result), flush=True)


_SLEEP_CYCLES_PER_MS = []


def gpu_busy(torch, ms=1.0):
    """Queues about `ms` of spinning on the current stream.  Launches enqueued behind it then run back
    to back, so the HIP event pair around each one times the kernel, not the host's launch latency (a
    kernel of a few microseconds is shorter than one Python launch call)."""
    if not _SLEEP_CYCLES_PER_MS:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS.append((1 << 20) / max(e0.elapsed_time(e1), 1e-3))
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS[0]))


def cold_launch_ms(torch, fn, flush, reps=10):
    """Duration (ms) of one launch that finds none of its data in L2 or the 256 MB MALL: before each launch
    a 1 GiB write and then a 1 GiB read sweep both caches (the read leaves them holding clean lines, so the
    timed launch does not pay for writing back the sweep's dirty ones); a HIP event pair brackets the
    launch alone.  The median of an event pair bracketing nothing after the same sweep (the event packets'
    own cost, about 2-4 us) is subtracted.  Returns (corrected, raw, empty-pair) medians."""
    import statistics
    fn()
    torch.cuda.synchronize()
    raw, empty = [], []
    for r in range(2 * reps):
        flush.fill_(float(r))
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if r % 2 == 0:
            fn()
        e1.record()
        torch.cuda.synchronize()
        (raw if r % 2 == 0 else empty).append(e0.elapsed_time(e1))
    raw_ms, empty_ms = statistics.median(raw), statistics.median(empty)
    return max(raw_ms - empty_ms, 1e-6), raw_ms, empty_ms


def cold_line(hbm, bytes_, timed):
    ms, raw, empty = timed
    line = hbm(bytes_, ms)
    line.update({"ms_raw": raw, "event_pair_ms": empty})
    return line


def attention_large(dts, torch, syn, dev, wl, stream, reps=5):
    """Dense and sensitive-row attention on a large workload (same kernels as the step): seeded
    N(0,1)*std bf16 tensors drawn on the device, `reps` back-to-back launches between one event pair."""
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    mk = lambda n: (torch.randn((wl.B, wl.H, n, wl.d), generator=g, device=dev) * wl.std).to(torch.bfloat16)
    q, ki, vi, kt, vt = mk(wl.N), mk(wl.N), mk(wl.N), mk(wl.T), mk(wl.T)
    rows = torch.from_numpy(syn.random_rows(wl)).to(dev)
    out = torch.zeros_like(q)
    timing = {}
    for name, fn in (("dense", lambda: dts.safe_attn_dense(q, ki, vi, kt, vt, wl.tv, out)),
                     ("rows", lambda: dts.safe_attn_rows(q, ki, vi, kt, vt, wl.tv, rows, out))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        timing[name] = e0.elapsed_time(e1) / reps
    tfd = wl.flops_dense / (timing["dense"] * 1e-3) / 1e12
    tfr = wl.flops_rows / (timing["rows"] * 1e-3) / 1e12
    line = {"workload": f"{wl.name}: B={wl.B}, H={wl.H}, d={wl.d}, N={wl.N}, Tv={wl.tv[0]}, |S|={wl.k}",
            "dense_ms": timing["dense"], "dense_tflops": tfd, "dense_frac_mfma": tfd / MFMA_BF16_PEAK_TFLOPS,
            "rows_ms": timing["rows"], "rows_tflops": tfr, "rows_frac_mfma": tfr / MFMA_BF16_PEAK_TFLOPS,
            "reps": reps}
    return q, ki, vi, kt, vt, rows, out, line


def time_launches(torch, fn, reps=20):
    """Average duration (ms) of `reps` back-to-back launches between one pair of HIP events, queued
    behind a spin so that they run back to back (one event pair per launch would add the dispatch of
    each event packet to every kernel, about 2 us, which is a third of a 6 us kernel)."""
    fn()
    torch.cuda.synchronize()
    gpu_busy(torch, 0.05 * reps + 0.5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def hbm_large(dts, torch, np, syn, dev, state, rows, hbm):
    """The HBM-bound stages on the 2560^2 / 3072^2 shapes (working sets of tens to hundreds of MB, far
    beyond the launch-overhead regime of the 1024^2 step), and torch's device copy as a reference point."""
    wl, w5 = syn.WORKLOADS["srsu_2560"], syn.WORKLOADS["traj_3072"]
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed + 100)
    out = {}
    H, N, T, Tv = wl.H, wl.N, wl.T, wl.tv[0]
    x = torch.randn((H, N, T), generator=g, device=dev)
    li = torch.randn((H, N), generator=g, device=dev) + float(np.log(N))
    sc = torch.empty(N, dtype=torch.float32, device=dev)
    out["pcsp_accumulate_2560"] = hbm(4.0 * H * N * Tv + 4.0 * H * N + 4.0 * N,
                                      time_launches(torch, lambda: dts.safe_pcsp_accumulate(x, li, Tv, 0, Tv, sc, False)))
    sweep = torch.empty(256 << 20, dtype=torch.float32, device=dev)  # 1 GiB
    pcsp_cold = cold_line(hbm, 4.0 * H * N * Tv + 4.0 * H * N + 4.0 * N, cold_launch_ms(
        torch, lambda: dts.safe_pcsp_accumulate(x, li, Tv, 0, Tv, sc, False), sweep))
    del x, li, sweep
    S = torch.empty(wl.k, dtype=torch.int32, device=dev)
    C = torch.empty(N - wl.k, dtype=torch.int32, device=dev)
    isn = torch.empty(N, dtype=torch.uint8, device=dev)
    s01 = torch.empty(N, dtype=torch.float32, device=dev)
    out["pcsp_partition_2560"] = {"ms": time_launches(torch, lambda: dts.safe_pcsp_partition(sc, wl.k, S, C, isn, s01)),
                                  "note": "one workgroup over N=25600: latency-bound, no roofline"}
    packed = torch.empty((wl.B, wl.H, wl.k, wl.d), dtype=torch.bfloat16, device=dev)
    gs = 2 * 2.0 * wl.B * wl.H * wl.k * wl.d
    out["gather_rows_2560"] = hbm(gs, time_launches(torch, lambda: dts.safe_gather_rows(state, rows, packed)))
    out["scatter_rows_2560"] = hbm(gs, time_launches(torch, lambda: dts.safe_scatter_rows(packed, rows, state)))
    C5, Hl, Wl = w5.latent
    eps = torch.randn((2, C5, Hl, Wl), generator=g, device=dev)
    s5 = torch.rand(w5.N, generator=g, device=dev)
    cout = torch.empty((C5, Hl, Wl), dtype=torch.float32, device=dev)
    out["swcfg_combine_3072"] = hbm(3 * 4.0 * C5 * Hl * Wl + 4.0 * w5.N,
                                    time_launches(torch, lambda: dts.safe_swcfg_combine(eps, s5, w5.side, w5.g_ctx,
                                                                                         w5.g_sens, cout)))
    src = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)  # 1 GiB
    dst = torch.empty_like(src)
    out["torch_copy_1GiB"] = hbm(2.0 * src.numel() * 4, time_launches(torch, lambda: dst.copy_(src), reps=10))
    # the same stages once more with L2 and MALL swept before each launch (dst is the sweep buffer)
    out["cold"] = {
        "pcsp_accumulate_2560": pcsp_cold,
        "gather_rows_2560": cold_line(hbm, gs, cold_launch_ms(
            torch, lambda: dts.safe_gather_rows(state, rows, packed), dst)),
        "scatter_rows_2560": cold_line(hbm, gs, cold_launch_ms(
            torch, lambda: dts.safe_scatter_rows(packed, rows, state), dst)),
        "swcfg_combine_3072": cold_line(hbm, 3 * 4.0 * C5 * Hl * Wl + 4.0 * w5.N, cold_launch_ms(
            torch, lambda: dts.safe_swcfg_combine(eps, s5, w5.side, w5.g_ctx, w5.g_sens, cout), dst)),
    }
    out["note"] = ("shapes: PCSP x [24,25600,256] fp32 (Tv=120 valid), partition N=25600 k=5120, gather/scatter "
                   "[2,24,25600,64] bf16 k=5120, SW-CFG [2,16,384,384] fp32; torch_copy_1GiB is torch's device copy, a "
                   "reference point rather than the ceiling (a streaming copy with nontemporal loads and stores "
                   "moves about 6.4 TB/s on this part)")
    return out


def next_rows(dts, torch, np, syn, dev, hbm, large: bool):
    """AesMask (affinity over the selected aesthetic text slots -> percentile count -> top-k mask) and
    StepCache (linear extrapolation of the prediction between full steps): warm and cold-cache timings."""
    out = {}
    sweep = torch.empty(256 << 20, dtype=torch.float32, device=dev)  # 1 GiB
    for name in (("srsu_1024", "srsu_2560") if large else ("srsu_1024",)):
        w = syn.WORKLOADS[name]
        H, N, T, Tv = w.H, w.N, w.T, w.tv[0]
        inp = syn.pcsp_logits(w, 0)
        x, li = torch.from_numpy(inp["x"]).to(dev), torch.from_numpy(inp["lse_img"]).to(dev)
        del inp
        sel = torch.from_numpy(syn.aesthetic_selection(w)).to(dev)
        sc = torch.empty(N, dtype=torch.float32, device=dev)
        k = dts.safe_percentile_count(N, 8000)
        S = torch.empty(k, dtype=torch.int32, device=dev)
        C = torch.empty(N - k, dtype=torch.int32, device=dev)
        isn = torch.empty(N, dtype=torch.uint8, device=dev)
        nbytes = 4.0 * H * N * Tv + 4.0 * H * N + 4.0 * N
        aff = lambda: dts.safe_affinity_accumulate(x, li, Tv, sel, sc, False)
        line = {"affinity_warm": hbm(nbytes, time_launches(torch, aff)),
                "affinity_cold": cold_line(hbm, nbytes, cold_launch_ms(torch, aff, sweep)),
                "mask_ms": time_launches(torch, lambda: (aff(), dts.safe_pcsp_partition(sc, k, S, C, isn))),
                "k": k,
                "workload": f"{name}: x [{H},{N},{T}] fp32 (Tv={Tv}), 8 selected slots, 80th percentile (k={k})"}
        out["aesmask_" + name.split("_")[1]] = line
        del x, li
    for name in (("srsu_1024", "traj_3072") if large else ("srsu_1024",)):
        w = syn.WORKLOADS[name]
        preds = torch.from_numpy(syn.stepcache_predictions(w, 2)).to(dev)
        o = torch.empty_like(preds[0])
        n = o.numel()
        ex = lambda: dts.safe_stepcache_extrapolate(preds[0], preds[1], 1.0 / 3.0, o)
        C_, Hl, Wl = w.latent
        out["stepcache_" + name.split("_")[1]] = {
            "warm": hbm(12.0 * n, time_launches(torch, ex)),
            "cold": cold_line(hbm, 12.0 * n, cold_launch_ms(torch, ex, sweep)),
            "workload": f"{name}: prediction [{C_},{Hl},{Wl}] fp32, w = 1/3"}
    out["note"] = ("warm: 20 back-to-back launches between one event pair; cold: each launch after a 1 GiB write "
                   "and a 1 GiB read, its own event pair minus an empty pair; mask_ms: affinity + partition")
    del sweep
    return out


def srsu_block(dts, torch, np, syn, dev):
    """The rest of a sensitive-row update on the 1024^2 shapes (B = 2, N = 4096, D = 1536, F = 6144, |S| = 1229):
    the FFN of the S rows into the cache (two products) and the QKV projection into the attention tensors."""
    w = syn.WORKLOADS["srsu_1024"]
    bf = lambda a: torch.from_numpy(syn.f32_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
    x = bf(syn.hidden_states(w))
    bw = syn.block_weights(w)
    w1, w2, wq = bf(bw["w1"]), bf(bw["w2"]), bf(bw["wqkv"])
    b1, b2, bq = (torch.from_numpy(bw[n]).to(dev) for n in ("b1", "b2", "bqkv"))
    rows = torch.from_numpy(syn.random_rows(w)).to(dev)
    D, F, T = w.H * w.d, bw["w1"].shape[0], w.B * w.k
    cache = torch.zeros_like(x)
    ws = torch.empty(dts.safe_rows_ffn_workspace_bytes(w.B, w.k, F) // 2, dtype=torch.bfloat16, device=dev)
    q = torch.zeros((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    kc, vc = torch.zeros_like(q), torch.zeros_like(q)
    ffn_ms = time_launches(torch, lambda: dts.safe_rows_ffn(x, rows, w1, b1, w2, b2, cache, ws))
    qkv_ms = time_launches(torch, lambda: dts.safe_rows_qkv(x, rows, wq, bq, q, kc, vc))
    ffn_fl, qkv_fl = 4.0 * T * D * F, 2.0 * T * D * 3 * D
    return {"ffn": {"ms": ffn_ms, "tflops": ffn_fl / (ffn_ms * 1e-3) / 1e12,
                    "frac_mfma": ffn_fl / (ffn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "flops": ffn_fl},
            "qkv": {"ms": qkv_ms, "tflops": qkv_fl / (qkv_ms * 1e-3) / 1e12,
                    "frac_mfma": qkv_fl / (qkv_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "flops": qkv_fl},
            "workload": f"srsu_1024: x [2,4096,{D}] bf16, |S|={w.k} rows per batch entry (T={T} tokens), F={F}; "
                        "FFN = gathered D->F + GELU, then F->D scattered into the cache; QKV D->3D into [B,H,N,d]"}


def cpu_other_stages(w, x, syn):
    """The fp64 oracle of the non-attention stages of the step, in full, on the step's own inputs."""
    import numpy as np
    from oracle import pcsp as OP, swcfg as OS
    t0 = time.perf_counter()
    a = OP.scores(x["x"].astype(np.float64), x["lse_img"].astype(np.float64), w.tv[0], 0, w.tv[0])
    t1 = time.perf_counter()
    OP.partition(a, w.k)
    t2 = time.perf_counter()
    s = OP.normalise(a)
    eps = syn.latent_eps(w).astype(np.float64)
    t3 = time.perf_counter()
    OS.combine(eps, s, w.side, w.g_ctx, w.g_sens)
    t4 = time.perf_counter()
    return {"pcsp_accumulate_ms": 1e3 * (t1 - t0), "pcsp_partition_ms": 1e3 * (t2 - t1),
            "swcfg_combine_ms": 1e3 * (t4 - t3), "kind": "oracle", "sample": "srsu_1024 stages in full"}


def profiled_traffic(field: str = "traffic_bytes_per_launch"):
    """A counter-derived figure of the dense attention kernel from the committed profile summary (HBM
    bytes per launch, or the shader clock in MHz), or None when the kernel source has changed since
    those counters were taken."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "attn_dense_1024.md")
    if not os.path.exists(prof):
        return None
    fields = {}
    for line in open(prof):
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch", "sclk_mhz", "kernel_source_sha256"):
            k, v = line.strip().split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in ("attn_mfma.hip", "common.hpp"):
        with open(os.path.join(ROOT, "diffusion_transformer_spatially_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest() or field not in fields:
        return None
    return float(fields[field])


def cpu_baseline(w, inp, budget_s: float):
    """The fp64 oracle as it stands, on a bounded sample of the same step's attention work."""
    import numpy as np
    from oracle import attention as OA

    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    rows = None  # every query row of each (b, h) visited
    flops = 0.0
    done = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.H):
            sl = lambda a: a[b:b + 1, h:h + 1]
            OA.attention(sl(inp["q"]), sl(inp["k_img"]), sl(inp["v_img"]), sl(inp["k_txt"]), sl(inp["v_txt"]),
                         (w.tv[b],), rows=rows)
            flops += 4.0 * w.N * (w.N + w.tv[b]) * w.d
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": min(cores, blas) if blas else cores,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle dense attention (all {w.N} query rows) of {done} of the "
                      f"{w.B * w.H} (b,h) heads of srsu_1024, stopped after a {budget_s:.0f} s budget ({el:.1f} s); "
                      f"host affinity {cores} cores, BLAS threads {blas}"}


if __name__ == "__main__":
    main()
