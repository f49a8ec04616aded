#!/usr/bin/env python3
"""Throughput of the LSSAR causal attention forward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the key-row L2-norm prep kernel, then the fused two-pass attention kernel
(what lssar_attn_fwd_ws launches), with inputs already resident in HBM.

Metric: algorithmic TFLOP/s, counting 4*d flops per unmasked (query, key)
pair (QK^T once plus P.V once; the pass-2 score recompute and all
elementwise work are not counted), i.e. 4*d*B*H*L(L+1)/2 per step.

Default workload: 8x length extrapolation, B=1 H=12 L=8192 d=64 bf16 p=15
with 16 planted keys per head (cosine 0.9 to one query), seed 0.

Prints ONE JSON line.  Extra objects: "roofline" for the attention kernel
(its mean duration from HIP events recorded around each kernel on the
launch stream, over K more steps right after the K timed ones: events
between the two kernels of a step add a gap of several microseconds, so the
timed steps carry none), "cpu_baseline" (the fp64 oracle on a bounded row sample, on
the host's cores), "sweep" (the same path at L = 1K..16K, H=12, d=64,
p=15, B = 16384/L, on device-generated N(0,1) inputs) and "variants" (the
note's two ablation variants on the same resident inputs: the Sigmoid
stage-1 map with re-weighting, and stage 1 alone, each timed as its whole
entry point, prep included) and "decode" (the decode step over a key/value
cache: 16 sequences x 12 heads at 8192 cached tokens, the same with ragged
lengths, and a wide-head case; HBM-bound, reported as GB/s of algorithmic
bytes and tokens/s; caches drawn N(0,1) on the device, lengths from the
input generator) and "backward" (on the bench workload: the training pair's
backward, lssar_attn_bwd_stats_ws with the row statistics of
lssar_attn_fwd_stats_ws, and the recomputing lssar_attn_bwd_ws; algorithmic
TFLOP/s counting 8*d flops per causal pair, the four products dO V^T,
W^T dO, dC K and dC^T Q; the score recompute is not counted; the training
forward's time beside the plain forward's) and "configs" (the GPT-2-small
workload, B8 H12 L1024 d64 p=3, and the wide-head workload, B2 H32 L4096
d128 p=15 with rank-8 correlated Q and K, each as its own whole step on its
seeded inputs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSSAR causal attn fwd TFLOP/s (% bf16 MFMA peak) at L=1K..16K, 1 GPU"
# MI355X published dense peaks (256 CUs, 2.4 GHz)
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# HBM traffic and VALU activity of the attention kernel measured with
# rocprofv3 --pmc (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
# calibration factor; SQ_ACTIVE_INST_VALU), valid only for the kernel source
# whose hash is recorded with them.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_record.json")
N_SIMDS = 256 * 4            # compute units x SIMDs per unit
CLOCK_HZ = 2.4e9             # peak engine clock
# Issue cost per wave64 instruction per SIMD at 4 waves per SIMD, measured by
# issue_rates.hip (profiles/issue_rates_gfx950.md): fp32 VALU, transcendental
# (v_exp_f32 / v_log_f32) and 16x16x32 MFMA; MFMA and VALU issue one after
# the other on a SIMD, so their times add.
ISSUE_NS = {"valu": 1.23, "trans": 3.58, "mfma": 7.68}
KERNEL_SRC = os.path.join(ROOT, "softmax_free_attention_amd", "csrc", "lssar_device.hpp")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_counters(workload: str):
    """The counter record of the attention kernel on this workload, or None
    when there is none or it was taken on other kernel source."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_sha256_16") != kernel_hash():
        return None
    return ent


def recorded_traffic(workload: str):
    ent = recorded_counters(workload)
    return ent.get("bytes_per_launch") if ent else None


def valu_roofline(workload: str, kernel_ms: float):
    """VALU issue against its capacity: the recorded VALU-active SIMD cycles
    per launch over 1024 SIMDs x 2.4 GHz x the launch duration measured
    now.  The kernel's elementwise chain, not its contractions, sets its
    time, so this is the fraction that says how close it runs to its
    bound.  None without a record for the current kernel source."""
    ent = recorded_counters(workload)
    if not ent or "valu_active_simd_cycles" not in ent:
        return None
    cap = N_SIMDS * CLOCK_HZ * kernel_ms * 1e-3
    out = {"active_simd_cycles": ent["valu_active_simd_cycles"],
           "capacity_simd_cycles": round(cap), "frac": round(ent["valu_active_simd_cycles"] / cap, 4),
           "valu_insts": ent.get("valu_insts"), "mfma_insts": ent.get("mfma_insts")}
    if "valu_trans_insts" in ent:
        # issue model: the recorded instruction counts at the measured rates
        trans = ent["valu_trans_insts"]
        model_us = ((ent["valu_insts"] - trans) * ISSUE_NS["valu"] + trans * ISSUE_NS["trans"] +
                    ent["mfma_insts"] * ISSUE_NS["mfma"]) / N_SIMDS * 1e-3
        out["issue_model_us"] = round(model_us, 1)
        out["issue_frac"] = round(model_us / (kernel_ms * 1e3), 4)
    return out


def upload(inp):
    import numpy as np
    import torch
    import lssar_inputs as gen
    out = []
    for a in (inp.q, inp.k, inp.v):
        if inp.wl.dtype == "f32":
            out.append(torch.from_numpy(np.ascontiguousarray(a)).cuda())
        else:
            out.append(torch.from_numpy(gen.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16))
    return out


def time_cold(q, k, v, p, steps, eps=1e-4):
    """Mean time of one lssar_attn_fwd_ws call when each follows a 512 MiB
    write (a fill that evicts the inputs from L2 and the Infinity Cache),
    HIP events around each call on the launch stream."""
    import torch
    import softmax_free_attention_amd as sfa
    ws = sfa.workspace_for(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for s in range(steps):
        scratch.fill_(s & 0xFF)
        ev[s][0].record(stream)
        sfa.lssar_attn_fwd_ws(q, k, v, out, ws, p=p, eps=eps, stream=stream)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    del scratch
    return {"ms": round(ms, 5), "steps": steps, "flush_mib": 512}


def time_path(q, k, v, p, steps, warmup, eps=1e-4, settle_s=0.0, repeats=5):
    """Run warmup + timed steps; returns (wall_s, fwd_ms_mean, prep_ms_mean,
    reps): reps holds ms per step of the timed block and of repeats - 1 more
    blocks of the same steps right after it, for the spread.
    A step is one lssar_attn_fwd_ws call (the prep kernel, then the attention
    kernel); wall_s covers the timed steps, between torch.cuda.synchronize()
    calls.  Then the same number of steps run as lssar_prep and
    lssar_attn_fwd_prepped with HIP events recorded around each kernel on the
    launch stream, for the kernels' own mean durations (the events between
    the two launches add a gap, so that loop is not the timed one).  Before
    the warmup steps the same step runs untimed for settle_s seconds: the GPU
    clock needs a couple of seconds of load to reach its steady state, and a
    few milliseconds of warmup alone would time the ramp."""
    import torch
    import softmax_free_attention_amd as sfa
    ws = sfa.workspace_for(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step():
        sfa.lssar_attn_fwd_ws(q, k, v, out, ws, p=p, eps=eps, stream=stream)

    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    reps = [wall / steps * 1e3]
    for _ in range(repeats - 1):
        t1 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        reps.append((time.perf_counter() - t1) / steps * 1e3)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        ev[s][0].record(stream)
        sfa.lssar_prep(k, ws, stream=stream)
        ev[s][1].record(stream)
        sfa.lssar_attn_fwd_prepped(q, k, v, ws, out, p=p, eps=eps, stream=stream)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    fwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    prep = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    return wall, fwd, prep, reps


def time_variants(q, k, v, p, steps, warmup, eps=1e-4):
    """Mean ms per call of the ablation variants' entry points (prep plus
    attention kernel), HIP events on the launch stream."""
    import torch
    import softmax_free_attention_amd as sfa
    ws = sfa.workspace_for(q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    calls = {
        "sigmoid_reweight": lambda: sfa.lssar_attn_fwd_phi_ws(
            q, k, v, out, ws, p=p, eps=eps, phi=sfa.LSSAR_PHI_SIGMOID, stream=stream),
        "lssa_only": lambda: sfa.lssar_lssa_fwd_ws(q, k, v, out, ws, stream=stream),
    }
    res = {}
    for name, fn in calls.items():
        # untimed load first: the clock drops between phases and needs time
        # under load to come back (see time_path)
        t_end = time.perf_counter() + 1.0
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    return res


def time_configs(names, steps, warmup, backward=True):
    """The other full-size workloads, each as its own whole step (prep plus
    attention kernel, one lssar_attn_fwd_ws call) on its seeded inputs:
    wall time of K back-to-back steps after a second of untimed load, and
    the two kernels' mean durations from HIP events.  With backward, also
    the training pair and the recomputing backward on the same inputs (as
    time_backward)."""
    import lssar_inputs as gen
    res = {}
    for name in names:
        wl = gen.WORKLOADS[name]
        inp = gen.make_inputs(wl)
        q, k, v = upload(inp)
        wall, fwd, prep, _ = time_path(q, k, v, wl.p, steps, warmup, settle_s=1.0, repeats=1)
        ms = wall / steps * 1e3
        res[name] = {"B": wl.B, "H": wl.H, "L": wl.L, "d": wl.d, "p": wl.p, "dtype": wl.dtype,
                     "structure": wl.structure, "ms_per_step": round(ms, 5),
                     "tflops": round(wl.flops / (ms * 1e-3) / 1e12, 2),
                     "pct_bf16_peak": round(100 * wl.flops / (ms * 1e-3) / 1e12 /
                                            PEAK_TFLOPS["bf16"], 3),
                     "tokens_per_s": round(wl.B * wl.L / (ms * 1e-3), 1),
                     "kernel_ms": {"lssar_fwd": round(fwd, 5), "lssar_prep": round(prep, 5)},
                     "kernel_tflops": round(wl.flops / (fwd * 1e-3) / 1e12, 2),
                     "traffic": recorded_traffic(name), "valu": valu_roofline(name, fwd)}
        if backward:
            bt = time_backward(q, k, v, wl.p, max(3, steps // 4), 2)
            bflops = 2 * wl.flops               # 8 d flops per causal pair
            res[name]["backward"] = {
                "ms": round(bt["saved"], 4),
                "tflops": round(bflops / (bt["saved"] * 1e-3) / 1e12, 2),
                "recompute_ms": round(bt["recompute"], 4),
                "train_fwd_ms": round(bt["train_fwd"], 4)}
        del q, k, v, inp
    return res


def time_decode(name, steps, warmup):
    """Mean time of one decode step (lssar_decode_ws: one kernel from 176 bf16
    heads, three below) on a device-generated cache, HIP events on the launch
    stream."""
    import numpy as np
    import torch
    import lssar_inputs as gen
    import softmax_free_attention_amd as sfa
    wl = gen.DECODE_WORKLOADS[name]
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed)
    q = torch.randn((wl.B, wl.H, wl.d), generator=g, device="cuda").to(dt)
    k = torch.randn((wl.B, wl.H, wl.Lmax, wl.d), generator=g, device="cuda").to(dt)
    v = torch.randn((wl.B, wl.H, wl.Lmax, wl.d), generator=g, device="cuda").to(dt)
    lens_np = gen.decode_lens(wl)
    lens = torch.from_numpy(lens_np).cuda()
    ws = sfa.decode_workspace_for(k)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        sfa.lssar_decode_ws(q, k, v, lens, out, ws, p=wl.p, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        sfa.lssar_decode_ws(q, k, v, lens, out, ws, p=wl.p, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    eb = 2 if wl.dtype == "bf16" else 4
    # algorithmic bytes: K and V rows in use read once, q read, out written, lens
    nbytes = 2 * wl.H * wl.d * eb * int(lens_np.sum()) + 2 * wl.B * wl.H * wl.d * eb + 4 * wl.B
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, k, v, ws, out
    return {"B": wl.B, "H": wl.H, "Lmax": wl.Lmax, "d": wl.d, "p": wl.p, "lens": wl.lens,
            "mean_len": round(float(lens_np.mean()), 1), "ms": round(ms, 5),
            "tokens_per_s": round(wl.B / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "bytes": nbytes}}


def time_backward(q, k, v, p, steps, warmup, eps=1e-4):
    """Mean ms of the training forward (lssar_attn_fwd_stats_ws), of the
    backward from its saved row statistics and of the recomputing backward,
    each call timed with HIP events on the launch stream after a second of
    untimed calls; seeded N(0,1) dout."""
    import torch
    import softmax_free_attention_amd as sfa
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(q.dtype)
    ws, fws = sfa.bwd_workspace_for(q), sfa.workspace_for(q)
    out, st = torch.empty_like(q), sfa.stats_for(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream()
    calls = {
        "train_fwd": lambda: sfa.lssar_attn_fwd_stats_ws(q, k, v, out, st, fws, p=p, eps=eps,
                                                         stream=stream),
        "saved": lambda: sfa.lssar_attn_bwd_stats_ws(q, k, v, out, dout, st, dq, dk, dv, ws,
                                                     p=p, eps=eps, stream=stream),
        "recompute": lambda: sfa.lssar_attn_bwd_ws(q, k, v, dout, dq, dk, dv, ws, p=p, eps=eps,
                                                   stream=stream),
    }
    res = {}
    for name, fn in calls.items():
        # untimed load first: the clock drops between phases and needs time
        # under load to come back (see time_path)
        t_end = time.perf_counter() + 1.0
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    return res


def cpu_baseline(inp, seconds: float):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's
    rows (strided over all heads and positions), on all host cores."""
    import numpy as np
    import oracle
    wl = inp.wl
    total_rows = wl.B * wl.H * wl.L
    nthreads = oracle.threads(0)

    def run(rows_per_head, heads):
        flops = 0
        t0 = time.perf_counter()
        for (b, h) in heads:
            stride = max(1, wl.L // rows_per_head)
            rows = np.arange(stride // 2, wl.L, stride)[:rows_per_head]
            oracle.lssar_rows(inp.q[b, h], inp.k[b, h], inp.v[b, h], rows, wl.p, nthreads=nthreads)
            flops += int(4 * wl.d * (rows + 1).sum())
        return time.perf_counter() - t0, flops

    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    cal_t, _ = run(max(1, 4 * nthreads), heads[:1])
    per_row = cal_t / max(1, 4 * nthreads)
    n = int(seconds / per_row / len(heads))
    n = max(nthreads, min(wl.L, n))
    dt, flops = run(n, heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{n * len(heads)} of {total_rows} query rows ({n} evenly strided rows in "
                      f"each of {len(heads)} heads), fp64 literal oracle, {dt:.1f} s",
            "cpu_model": cpu_model(), "one_thread": one_thread_times(),
            "seconds": dt}


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def one_thread_times():
    """The oracle on one thread: the tiny fp32 workload (B1 H1 L128 d64,
    p=3) in full, and the GPT-2-small workload (B8 H12 L1024 d64, p=3) on 4
    of its 96 heads, scaled to all 96."""
    import lssar_inputs as gen
    import oracle
    res = {}
    inp = gen.make_inputs("tiny")
    t0 = time.perf_counter()
    oracle.lssar_fwd(inp.q, inp.k, inp.v, inp.wl.p, nthreads=1)
    res["tiny_s"] = round(time.perf_counter() - t0, 4)
    inp = gen.make_inputs("gpt2s")
    heads = [(0, 0), (2, 5), (5, 7), (7, 11)]
    t0 = time.perf_counter()
    for b, h in heads:
        oracle.lssar_fwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.wl.p, nthreads=1)
    dt = time.perf_counter() - t0
    nh = inp.wl.B * inp.wl.H
    res["gpt2s_s"] = round(dt * nh / len(heads), 2)
    res["gpt2s_sample"] = f"{len(heads)} of {nh} heads in {dt:.2f} s, scaled to {nh}"
    return res


def sweep(steps, warmup):
    import torch
    res = {}
    g = torch.Generator(device="cuda")
    for L in (1024, 2048, 4096, 8192, 16384):
        B = 16384 // L
        g.manual_seed(L)
        shape = (B, 12, L, 64)
        q, k, v = (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
                   .to(torch.bfloat16) for _ in range(3))
        wall, fwd, prep, _ = time_path(q, k, v, 15, steps, warmup, settle_s=0.3, repeats=1)
        flops = 4 * 64 * B * 12 * L * (L + 1) // 2
        res[str(L)] = {"B": B, "tflops": round(flops * steps / wall / 1e12, 2),
                       "kernel_tflops": round(flops / (fwd * 1e-3) / 1e12, 2),
                       "pct_bf16_peak": round(100 * flops * steps / wall / 1e12 / PEAK_TFLOPS["bf16"], 2)}
        del q, k, v
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="x8_planted")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-workloads", default="x8_decode,x8_decode_ragged,wide_decode",
                    help="comma-separated decode workloads to time (a profiler run can take one)")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the GPT-2-small (p=3) and wide-head (d=128) workloads")
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="after timing, run a plain elementwise copy of this many MiB (read N, "
                         "write N), the reference kernel for scaling rocprofv3 FETCH/WRITE_SIZE")
    ap.add_argument("--settle-seconds", type=float, default=3.0,
                    help="untimed load before the warmup steps, for the GPU clock to settle")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps that each follow a 512 MiB write (cold caches)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the LSSAR forward shards over (batch, head) "
              f"units with no communication, so one GPU's share at its real shape is what it "
              f"runs and reports (got --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import lssar_inputs as gen
    import softmax_free_attention_amd as sfa
    sfa.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    wl = gen.WORKLOADS[args.workload]
    log(f"bench: generating {wl.name} inputs")
    inp = gen.make_inputs(wl)
    q, k, v = upload(inp)
    log(f"bench: timing {args.steps} steps after {args.warmup} warmup")
    wall, fwd_ms, prep_ms, reps = time_path(q, k, v, wl.p, args.steps, args.warmup,
                                            settle_s=args.settle_seconds)
    flops = wl.flops
    value = flops * args.steps / wall / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    traffic = recorded_traffic(wl.name)
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "L": wl.L, "d": wl.d, "p": wl.p,
                   "structure": wl.structure, "seed": wl.seed, "eps": 1e-4},
        "pct_of_bf16_mfma_peak": round(100 * value / PEAK_TFLOPS["bf16"], 3),
        "tokens_per_s": round(wl.B * wl.L * args.steps / wall, 1),
        # ms per step of the timed block and four more blocks of K steps
        "repeats": {"n": len(reps), "ms_per_step_median": round(statistics.median(reps), 5),
                    "ms_per_step_min": round(min(reps), 5),
                    "ms_per_step_p90": round(sorted(reps)[max(0, int(0.9 * len(reps) + 0.5) - 1)], 5)},
        "kernel_ms": {"lssar_fwd": round(fwd_ms, 5), "lssar_prep": round(prep_ms, 5)},
        "roofline": {"bound": "mfma", "kernel": "lssar_fwd_bf16_kernel" if wl.dtype == "bf16"
                     else "lssar_fwd_f32_kernel",
                     "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 5), "traffic": traffic,
                     "valu": valu_roofline(wl.name, fwd_ms)},
    }
    if args.calib_mib > 0:
        n = args.calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.add(src, 0.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.cold:
        log("bench: cold-cache steps")
        line["cold"] = time_cold(q, k, v, wl.p, args.steps)
    if not args.no_configs:
        log("bench: other workloads")
        others = [n for n in ("gpt2s", "wide") if n != wl.name]
        line["configs"] = time_configs(others, args.steps, args.warmup,
                                       backward=not args.no_backward)
    if not args.no_variants:
        log("bench: ablation variants")
        vt = time_variants(q, k, v, wl.p, args.steps, args.warmup)
        line["variants"] = {n: {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
                            for n, ms in vt.items()}
    if not args.no_backward:
        log("bench: backward")
        bt = time_backward(q, k, v, wl.p, max(3, args.steps // 4), 2)
        bflops = 2 * flops
        bms = bt["saved"]
        line["backward"] = {"ms": round(bms, 4), "tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
                            "pct_bf16_peak": round(100 * bflops / (bms * 1e-3) / 1e12 /
                                                   PEAK_TFLOPS["bf16"], 3),
                            "row_stats": "saved by the training forward",
                            "recompute_ms": round(bt["recompute"], 4),
                            "train_fwd_ms": round(bt["train_fwd"], 4)}
    if not args.no_decode:
        log("bench: decode")
        line["decode"] = {n: time_decode(n, 50, 10)
                          for n in args.decode_workloads.split(",") if n}
    if not args.no_sweep:
        log("bench: L sweep")
        line["sweep"] = sweep(steps=10, warmup=3)
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cb = cpu_baseline(inp, args.cpu_seconds)
        cb.pop("seconds", None)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
