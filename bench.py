#!/usr/bin/env python3
"""Benchmark of the FlashAttention-2 forward (and backward) on one MI355X.

One step = one forward pass (one fa_fwd launch) over the multi-head causal
workload B=4, H=16, S=4096, D=64, fp16, [B,H,S,D] layout, with q, k, v drawn
from a fixed seed and resident in HBM before timing starts.  The metric is
attention-forward TFLOP/s with FLOPs = 4*B*H*S^2*D, halved for causal, and its
fraction of the MI355X dense fp16 matrix peak (2.5 PFLOP/s).

Prints one JSON line.  Also reported:
  roofline      (mfma_busy_pct, valu_active_pct: SQ_VALU_MFMA_BUSY_CYCLES and
                SQ_ACTIVE_INST_VALU against the kernel's SIMD-cycles, from the
                committed rocprofv3 summary profiles/*_busy.txt of the workload
                while the sources match)
                achieved TFLOP/s of the attention kernel from one pair of HIP
                events around the timed launches, on the stream they run on
                (the average launch duration; events around every launch would
                add about 7 us of stream work per launch), against the peak;
                `traffic` is the HBM bytes per launch measured with rocprofv3
                FETCH_SIZE / WRITE_SIZE (scaled by a copy-kernel calibration),
                taken from the committed summary in profiles/ for this workload
                while the kernel sources still hash to what was profiled, else
                null (--traffic-bytes overrides);
  cpu_baseline  the float64 CPU oracle timed on this host's cores over the
                whole workload (every row of every head), in the same unit;
  backward      fa_bwd_ex (dQ, dK, dV) on the same workload with a seeded dO:
                TFLOP/s with the usual 2.5x-forward FLOP count, HIP-event
                kernel time, and the oracle's gradients over one head as its
                CPU baseline (--no-backward skips it).

  roofline.exp_valu  the vector-side roof: v_exp / v_fma / v_add / v_cvt_pk
                issue rates measured in the same run (libfa_micro.so), turned
                into SIMD-cycles per attended (query, key) pair against the
                MFMA cycles per pair, with the TFLOP/s each side allows alone
                and with no overlap;
  configs       one record per configuration workload and mask (single-head
                fp32, the headless batch both ways, the multi-head causal
                workload, the long bf16 sequence, the 20 sweep points): kernel
                microseconds from a replayed HIP graph (after about 50 ms of
                untimed replays), TFLOP/s, fraction of
                peak, algorithmic HBM GB/s, and the errors of O and lse against
                the float64 oracle over every element (--no-configs,
                --no-parity skip them);
  extended      the same record for grouped K/V heads (the multi-head causal
                workload with 4 K/V heads) and a sliding window (B=2 H=16
                S=8192 D=64 causal, 1024-key left window), with the backward's
                event-timed microseconds and fraction of peak on each.

Timing: about 200 ms of untimed launches of the same forward (`settle`,
--settle-ms; reported in the line) bring a fresh process's GPU to its loaded
clock, then W untimed warmup steps, then exactly K timed steps between two
synchronisations (a cold 20-step run reads about 12 % lower: its
milliseconds run while the clock still rises).

Options: --gpus N (only 1 is supported: the kernel runs on one GPU),
--steps K (timed launches), --warmup W, --settle-ms MS, --workload NAME, --no-cpu-baseline,
--sweep FILE (also time every named workload and write one JSON line per
workload to FILE; sweep kernels are timed from a HIP graph of 20 launches
replayed 10 times, so short kernels carry no host launch overhead).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # dense, MI355X published
PEAK_HBM_GBS = 8000.0


def profiled_traffic(workload):
    """HBM bytes per launch from profiles/*_traffic.txt for this workload, or
    None when no summary matches the current kernel sources."""
    import glob
    from exact_tiled_attention_06_amd import build
    want = build.source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt"))):
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    key, _, val = line.partition(":")
                    kv[key.strip()] = val.strip()
        if kv.get("workload") == workload and kv.get("source_sha256") == want:
            return float(kv["traffic_bytes_per_launch"])
    return None


def profiled_busy(workload):
    """MFMA busy % and VALU active % per kernel ({'mfma_busy_pct_fwd': ..,
    'valu_active_pct_dq': .., ...}) from the committed rocprofv3 summary
    profiles/*_busy.txt of this workload, or {} when none matches the current
    kernel sources."""
    import glob
    from exact_tiled_attention_06_amd import build
    want = build.source_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_busy.txt"))):
        kv = {}
        with open(path) as f:
            for line in f:
                key, sep, val = line.partition(":")
                if sep and not line.startswith(" "):
                    kv[key.strip()] = val.strip()
        if kv.get("workload") == workload and kv.get("source_sha256") == want:
            return {k: float(v) for k, v in kv.items() if k.startswith(("mfma_busy_pct_", "valu_active_pct_"))}
    return {}


def settle(launch, torch, ms):
    """Untimed launches for about `ms` of wall time, so that a short timed run
    starts at the clock the GPU holds under load (a fresh process otherwise
    times its first milliseconds while the clock still rises).  Returns the
    milliseconds spent and the launches made."""
    if ms <= 0:
        return 0.0, 0
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            launch()
        n += 10
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, n


def time_workload(fa, torch, w, causal, steps, warmup, settle_ms=0.0):
    """Wall time of `steps` forwards on the workload, their average duration in
    ms from one pair of HIP events around them on their stream, and the settle
    phase (ms, launches) that ran before the `warmup` untimed steps."""
    import workloads
    q, k, v = (x.to("cuda:0") for x in workloads.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda:0")

    def launch():
        fa.forward(q, k, v, causal=causal, scale=w.scale, out=o, lse=lse, window=w.window)

    settled = settle(launch, torch, settle_ms)
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        launch()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps, settled


def time_graph(fa, torch, w, causal, launches=20, reps=10, settle_ms=50.0):
    """Time per forward from a HIP graph of `launches` fa_fwd_ws calls (with the
    workspace fa_fwd_workspace_bytes asks for, as forward() passes it) on
    preallocated buffers, replayed `reps` times between two events: the GPU
    never waits for the host, so short kernels are timed without the Python
    call's overhead.  Untimed replays for about `settle_ms` first bring the
    clock back up after the host work between records.  Returns the
    milliseconds per forward."""
    import workloads
    q, k, v = (x.to("cuda:0") for x in workloads.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda:0")
    wl, wr = w.window
    code = fa.DTYPE_CODES[q.dtype]
    nbytes = fa.fa_fwd_workspace_bytes(w.B, w.H, k.shape[1], w.S, w.S, w.D, int(causal), wl, wr, code)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")

    def call(stream):
        return fa.fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                            k.shape[1], w.S, w.S, w.D, int(causal), wl, wr, w.scale, code, ws.data_ptr(), nbytes,
                            stream)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(3):
            fa.check(call(side.cuda_stream))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(launches):
            fa.check(call(side.cuda_stream))
    graph.replay()
    torch.cuda.synchronize()
    settle(graph.replay, torch, settle_ms)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (launches * reps)


def backward_call(fa, torch, w, causal):
    """The fa_bwd_ex call the backward timing makes on the workload (the
    forward's O and lse, a seeded dO, outputs preallocated): returns
    (call, (dq, dk, dv))."""
    import workloads
    q, k, v = (x.to("cuda:0") for x in workloads.workload_inputs(w))
    dout = workloads.make_grad(w.B, w.H, w.S, w.D, w.dtype, w.seed + 1000).to("cuda:0")
    window = None if w.window == (-1, -1) else w.window
    o, lse = fa.forward(q, k, v, causal=causal, scale=w.scale, window=window)
    # grouped heads: dK and dV are shaped like k, and the C call takes the
    # K/V head count from k (fa_bwd would take it to be H)
    B, H, S, D = q.shape
    hkv, sk = k.shape[1], k.shape[2]
    if k.shape != (B, hkv, sk, D) or v.shape != k.shape or H % hkv or o.shape != q.shape:
        raise ValueError(f"backward timing: inconsistent shapes {tuple(q.shape)}, {tuple(k.shape)}")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, S), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ptrs = [t.data_ptr() for t in (q, k, v, o, dout, lse, dq, dk, dv, delta)]
    code = fa.DTYPE_CODES[q.dtype]
    wl, wr = w.window

    # the call holds every buffer it passes by address, so none is freed while
    # the call can still run
    buffers = (q, k, v, o, dout, lse, dq, dk, dv, delta)

    def call(_buffers=buffers):
        return fa.fa_bwd_ex(*ptrs, B, H, hkv, S, sk, D, int(causal), wl, wr, w.scale, code, stream.cuda_stream)

    return call, (dq, dk, dv)


def time_backward(fa, torch, w, causal, steps, warmup, settle_ms=0.0):
    """Wall time of `steps` fa_bwd_ex calls (dQ kernel, then dK/dV kernel) on the
    workload, their average duration in ms from one pair of HIP events around
    them on their stream, and the settle phase (ms, launches) before the
    `warmup` untimed calls."""
    call, _ = backward_call(fa, torch, w, causal)
    stream = torch.cuda.current_stream()
    fa.check(call())
    settled = settle(call, torch, settle_ms)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps, settled


def cpu_baseline_backward(w, causal):
    """The float64 oracle's gradients over one head of the workload (a bounded sample)."""
    import oracle
    import workloads
    orc = oracle.default()
    q, k, v = (x[:1, :1].double().numpy() for x in workloads.workload_inputs(w))
    dout = workloads.make_grad(w.B, w.H, w.S, w.D, w.dtype, w.seed + 1000)[:1, :1].double().numpy()
    t0 = time.perf_counter()
    orc.attention_bwd(q, k, v, dout, causal, w.scale, None if w.window == (-1, -1) else w.window)
    dt = time.perf_counter() - t0
    head_flops = 2.5 * w.flops(causal) / (w.B * w.H)
    return {
        "value": head_flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": f"one head of the workload ({w.S} rows, float64, {dt:.2f} s wall), "
                  f"FLOPs counted as 2.5x the forward's",
    }


def cpu_baseline(w, causal):
    import numpy as np
    import oracle
    import workloads
    orc = oracle.default()
    q, k, v = workloads.workload_inputs(w)
    q, k, v = (x.double().numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    orc.attention(q, k, v, causal, w.scale)
    dt = time.perf_counter() - t0
    return {
        "value": w.flops(causal) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": f"whole workload ({w.B * w.H * w.S} rows, float64, {dt:.2f} s wall)",
    }



# The five configurations of the benchmark plan: single-head fp32, the headless
# batch (both masks), the multi-head causal workload, the long bf16 sequence and
# the 20-point causal fp16 sweep.
CONFIG_WORKLOADS = (["single_head_f32", "batch_f16", "multihead_causal", "long_seq_bf16"]
                    + [f"sweep_D{d}_S{s}" for d in (16, 32, 64, 128) for s in (256, 1024, 4096, 8192, 16384)])
# Grouped K/V heads and a sliding window on full-size problems, recorded beside
# the configurations (the headline workload with 4 K/V heads; B=2 H=16 S=8192
# with a 1024-key left window).
EXTENDED_WORKLOADS = ["gqa_causal", "window_causal"]


def config_records(fa, torch, parity=True, names=CONFIG_WORKLOADS, backward=False):
    """One record per configuration workload and mask: kernel microseconds timed
    from a replayed HIP graph, TFLOP/s, fraction of the dense peak of its dtype,
    algorithmic HBM GB/s and, with parity, the errors of O and lse against the
    float64 oracle over every element (max |dO| absolute for fp16/bf16, normwise
    relative for fp32; lse normwise and elementwise relative)."""
    import numpy as np
    import workloads
    recs = []
    for name in names:
        w = workloads.BY_NAME[name]
        win = None if w.window == (-1, -1) else w.window
        for c in w.causal:
            us = time_graph(fa, torch, w, c) * 1e3
            tf = w.flops(c) / (us * 1e-6) / 1e12
            rec = {"workload": name, "causal": c, "dtype": w.dtype, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   **({"H_kv": w.kv_heads} if w.kv_heads != w.H else {}), **({"window": list(win)} if win else {}),
                   "kernel_us": round(us, 2), "tflops": round(tf, 1),
                   "frac": round(tf / PEAK_MFMA_TFLOPS[w.dtype], 4),
                   "hbm_gbs_algorithmic": round(w.hbm_bytes() / (us * 1e-6) / 1e9, 1)}
            if backward and w.dtype in ("f16", "bf16"):
                # the backward on the same problem: 20 calls after 5, event-timed
                _, bavg, _ = time_backward(fa, torch, w, c, 20, 5, settle_ms=50.0)
                btf = 2.5 * w.flops(c) / (bavg * 1e-3) / 1e12
                rec["backward_us"] = round(bavg * 1e3, 2)
                rec["backward_frac"] = round(btf / PEAK_MFMA_TFLOPS[w.dtype], 4)
            if parity:
                import oracle
                q, k, v = workloads.workload_inputs(w)
                o, lse = fa.forward(q.to("cuda:0"), k.to("cuda:0"), v.to("cuda:0"), causal=c, scale=w.scale,
                                    window=win)
                torch.cuda.synchronize()
                o_ref, l_ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), c,
                                                w.scale, win)
                d_o = np.abs(o.cpu().double().numpy() - o_ref)
                d_l = np.abs(lse.cpu().double().numpy() - l_ref)
                rec["max_abs_dO"] = float(d_o.max()) if w.dtype != "f32" else None
                rec["o_rel_normwise"] = float(d_o.max() / np.abs(o_ref).max())
                rec["lse_rel_normwise"] = float(d_l.max() / np.abs(l_ref).max())
                rec["lse_rel_elementwise"] = float((d_l / np.maximum(np.abs(l_ref), 1.0)).max())
            recs.append(rec)
            print(f"config {name} causal={c}: {us:.1f} us, {tf:.1f} TFLOP/s ({100 * rec['frac']:.1f} % of peak)"
                  + (f", max|dO| {rec.get('max_abs_dO')}, lse rel {rec['lse_rel_normwise']:.2e}" if parity else ""),
                  file=sys.stderr, flush=True)
    return recs


def exp_valu_roof(D):
    """The vector-side roof of the attention loop, from instruction rates measured
    now (libfa_micro.so, two waves per SIMD): per attended (query, key) pair the
    forward issues one v_exp_f32, one v_fma_f32 (S*c - m), one v_add_f32 (row
    sum) and half a v_cvt_pk (P to 16 bits) per lane, against 4*D FLOPs of
    32x32x16 MFMA.  Returns SIMD-cycles per pair on each side and the TFLOP/s
    each side alone would allow at the peak's 2.4 GHz on 1024 SIMDs, plus the
    bound with no overlap of the two."""
    from exact_tiled_attention_06_amd import micro
    it = 400
    micro.run(micro.OP_EXP, 4, False, micro.VECTOR, 8, 10)  # warm-up
    per = {}
    for op, name in ((micro.OP_EXP, "exp"), (micro.OP_FMA, "fma"), (micro.OP_ADD, "add"), (micro.OP_CVT, "cvt")):
        c = micro.run(op, 4, False, micro.VECTOR, 8, it)
        per[name] = max(c) / (it * 32) / 2  # SIMD-cycles per wave64 instruction (two waves share a SIMD)
    c = micro.run(micro.OP_EXP, 0, False, micro.PRODUCTS, 8, it)
    mfma = max(c) / (it * 8) / 2
    vec_pair = (per["exp"] + per["fma"] + per["add"] + 0.5 * per["cvt"]) / 64
    mfma_pair = 4 * D / (2 * 32 * 32 * 16) * mfma
    scale = 1024 * 2.4e9 * 4 * D / 1e12
    return {"vector_cycles_per_pair": round(vec_pair, 4), "mfma_cycles_per_pair": round(mfma_pair, 4),
            "issue_cycles": {k: round(v, 2) for k, v in per.items()} | {"mfma_32x32x16": round(mfma, 2)},
            "vector_roof_tflops": round(scale / vec_pair, 1), "mfma_roof_tflops": round(scale / mfma_pair, 1),
            "no_overlap_tflops": round(scale / (vec_pair + mfma_pair), 1),
            "note": "SIMD-cycles per attended pair at two waves per SIMD (measured issue rates); the loop "
                    "cannot run faster than either roof, and runs at the no-overlap bound if vector work and "
                    "MFMAs never overlap"}

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed launches of the same forward for this long before the warmup steps "
                         "(0: none), reported as `settle`")
    ap.add_argument("--workload", default="multihead_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--traffic-bytes-bwd", type=float, default=None,
                    help="HBM bytes per fa_bwd call measured with rocprofv3 counters")
    ap.add_argument("--traffic-bytes", type=float, default=None,
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--sweep", default=None, help="write per-workload JSON lines to this file")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records (graph-timed, with oracle errors)")
    ap.add_argument("--no-parity", action="store_true",
                    help="per-configuration records without the oracle comparison")
    ap.add_argument("--micro", default=None,
                    help="instead of attention, run the instruction-rate microbenchmarks (libfa_micro.so) and "
                         "write their table, one JSON line per probe, to this file")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of attention, run plain device-to-device copies of this many bytes "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this attention forward runs on one GPU "
              "(no sharding or collectives are built). Use --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import exact_tiled_attention_06_amd as fa
    import workloads

    fa.library()  # fails loudly when libfa.so is missing

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    if args.micro:
        from exact_tiled_attention_06_amd import micro
        rows = micro.table()
        with open(args.micro, "w") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")
                print(f"micro {r['kind']:6s} {r['cycles']:8.2f}  {r['unit']}"
                      + (f"  (vector wave {r['vector_wave_cycles']})" if "vector_wave_cycles" in r else ""),
                      flush=True)
        return 0

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": args.warmup + args.steps}), flush=True)
        return 0

    w = workloads.BY_NAME[args.workload]
    causal = w.causal[-1]
    wall, avg_kernel_ms, settled = time_workload(fa, torch, w, causal, args.steps, args.warmup, args.settle_ms)
    flops = w.flops(causal)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / (avg_kernel_ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[w.dtype]
    traffic = args.traffic_bytes if args.traffic_bytes is not None else profiled_traffic(w.name)
    out = {
        "metric": "attention fwd TFLOP/s and % of MI355X dense fp16/bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": round(settled[0], 1), "launches": settled[1],
                   "note": "untimed launches of the same forward before the warmup steps, so that the "
                           "timed steps run at the GPU's loaded clock"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype} "
                        f"{'causal' if causal else 'non-causal'}, [B,H,S,D], randn seed {w.seed}",
            "B": w.B, "H": w.H, "S": w.S, "D": w.D, "causal": causal,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
            "algorithmic_bytes": w.hbm_bytes(),
            "kernel_ms_avg": round(avg_kernel_ms, 5),
            "hbm_gbs_algorithmic": round(w.hbm_bytes() / (avg_kernel_ms * 1e-3) / 1e9, 1),
            "mfma_busy_pct": None,
        },
        "cpu_baseline": None,
    }

    busy = profiled_busy(w.name)
    out["roofline"]["mfma_busy_pct"] = busy.get("mfma_busy_pct_fwd")
    out["roofline"]["valu_active_pct"] = busy.get("valu_active_pct_fwd")

    if not args.no_backward and w.dtype in ("f16", "bf16"):
        bwall, bavg, bsettled = time_backward(fa, torch, w, causal, args.steps, args.warmup, args.settle_ms)
        bflops = 2.5 * flops  # the usual count: five tile products to the forward's two
        executed = 3.5 * flops  # S and dP are formed by both kernels: seven products
        out["backward"] = {
            "metric": "attention bwd TFLOP/s (dQ, dK, dV; FLOPs = 2.5x the forward's)",
            "value": round(bflops / (bwall / args.steps) / 1e12, 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(bwall * 1e3 / args.steps, 5),
            "settle": {"ms": round(bsettled[0], 1), "launches": bsettled[1]},
            "kernels": ["fa_bwd_dq_kernel", "fa_bwd_dkdv_kernel"],
            "roofline": {
                "bound": "mfma",
                "achieved": round(bflops / (bavg * 1e-3) / 1e12, 2),
                "achieved_executed": round(executed / (bavg * 1e-3) / 1e12, 2),
                "peak": peak,
                "unit": "TFLOP/s",
                "frac": round(bflops / (bavg * 1e-3) / 1e12 / peak, 4),
                "frac_executed": round(executed / (bavg * 1e-3) / 1e12 / peak, 4),
                "traffic": args.traffic_bytes_bwd if args.traffic_bytes_bwd is not None
                           else profiled_traffic(w.name + ":backward"),
                "traffic_unit": "bytes per fa_bwd call (both kernels; HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                "kernel_ms_avg": round(bavg, 5),
                "mfma_busy_pct": {"dq": busy.get("mfma_busy_pct_dq"), "dkdv": busy.get("mfma_busy_pct_dkdv")}
                                 if busy else None,
                "valu_active_pct": {"dq": busy.get("valu_active_pct_dq"), "dkdv": busy.get("valu_active_pct_dkdv")}
                                   if busy else None,
            },
            "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_backward(w, causal),
        }

    if args.sweep:
        with open(args.sweep, "w") as f:
            for sw in workloads.ALL:
                for c in sw.causal:
                    avg = time_graph(fa, torch, sw, c)
                    rec = {"workload": sw.name, "causal": c, "dtype": sw.dtype, "B": sw.B, "H": sw.H,
                           "S": sw.S, "D": sw.D, "kernel_ms_avg": avg,
                           "tflops": sw.flops(c) / (avg * 1e-3) / 1e12,
                           "pct_peak": 100 * sw.flops(c) / (avg * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS[sw.dtype],
                           "hbm_gbs": sw.hbm_bytes() / (avg * 1e-3) / 1e9}
                    f.write(json.dumps(rec) + "\n")
                    print(f"sweep {sw.name} causal={c}: {rec['tflops']:.1f} TFLOP/s "
                          f"({avg * 1e3:.1f} us)", file=sys.stderr, flush=True)

    if w.dtype in ("f16", "bf16"):
        out["roofline"]["exp_valu"] = exp_valu_roof(w.D)
    if not args.no_configs:
        out["configs"] = config_records(fa, torch, parity=not args.no_parity)
        out["extended"] = config_records(fa, torch, parity=not args.no_parity, names=EXTENDED_WORKLOADS,
                                         backward=not args.no_backward)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, causal)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
