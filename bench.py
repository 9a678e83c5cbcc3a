#!/usr/bin/env python3
"""Benchmark of the W2A8 BitLinear hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
python bench.py --traffic-probe   (launch pattern for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)

A step is one BitNet-2B-shaped decode layer set at M = 1: the seven projections
(q, k, v, o, gate, up, down; (N, K) = (2560,2560) (640,2560) (640,2560) (2560,2560)
(6912,2560) (6912,2560) (2560,6912)), bf16 activations in, fp32 out, every step of the
path: absmax, quantize, stream and unpack the packed weights, int8 x ternary dot with
int32 accumulation, rescale.  Projections that read the same activations share one
fused quant + GEMV launch (q|k|v, o, gate|up, down: four launches); the same set with
one launch per projection is reported beside it (value_ungrouped).

* Inputs are resident in HBM before timing.  The packed weights are replicated into
  enough copies to exceed 1 GiB and every step uses the next copy, so the weights come
  from HBM rather than the 256 MB Infinity Cache.
* Steps are captured in HIP graphs, ten consecutive steps (each on the next weight
  copy) per graph, so host submission does not pace the GPU; W warmup steps, then
  exactly K steps between two synchronizations timed with events.
* value = packed-weight bytes of the set / step time (GB/s).
* roofline: the fused quant+GEMV kernel, algorithmic bytes (N*K/4 packed bytes per
  launch) / its mean launch duration (a graph of back-to-back launches over the weight
  copies, timed with events), against 8 TB/s; traffic from the committed rocprofv3
  counter summary when it matches the current kernel source.
* gemm: the BitNet-2B-shaped prefill set at M = 512 (tiled int8-MFMA GEMM, bf16 out),
  with the projections that share an input in one grouped launch (q|k|v, o, gate|up,
  down), int8 TOPS against 5.0 POPS dense from the per-launch GEMM durations; the step
  rate with the four quantization launches and the rate of seven ungrouped launches are
  reported beside it.
* cpu_baseline: the CPU oracle on the host cores (test infrastructure, timed only
  here), on the same decode step repeated for ~10 s.
* extras: the same per-launch rooflines at large shapes, where the bandwidth and
  matrix-core bars are reachable: the 70B-shaped decode layer set (M = 1) and the
  8B-shaped prefill MLP GEMMs (M = 2048); the 2B decode MLP as two launches (gate|up
  with the SwiGLU epilogue, then down); the 2B decode set with bf16 activations and no
  activation quantization (W1.58A16); and ceilings measured on this chip: an int8
  matrix-core loop on register operands, a 2 GiB streaming read, and the vendor int8
  GEMM (hipBLASLt, dense int8 weights) at the prefill shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix cores, TOPS
ROTATE_BYTES = 1 << 30        # weight copies per rotation (> 4x the 256 MB MALL)
METRIC = "W2A8 ternary GEMV GB/s (%HBM peak) at M=1; GEMM int8 TOPS (%MFMA) at M=512"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quant_gemv_2b_decode_m1_traffic.txt")
GEMM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "tiled_gemm_2b_prefill_m512_counters.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 70B-shaped decode and 8B-shaped prefill rooflines")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the counter-collection launch pattern and exit (no timing)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="run the prefill GEMM launches for counter collection and exit")
    return ap.parse_args()


def load_summary(path: str, kernel_hash: str):
    """key = value lines of a committed counter summary, if its kernel hash still applies."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals if vals.get("kernel_source_sha256") == kernel_hash else None


def load_traffic(kernel_hash: str):
    """Per-launch HBM bytes from the committed counter summary, if it still applies."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_linear_token_amd as bw
    from ternary_weight_linear_token_amd import build as bw_build
    import workloads

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    bw.lib()
    layer = workloads.LAYER_2B
    print(f"[bench] packing {len(layer)} 2B-shaped projections", file=sys.stderr, flush=True)

    packed0, scales, xs, outs = [], [], [], []
    index = {name: i for i, (name, _, _) in enumerate(layer)}
    groups = [[index[n] for n in grp] for grp in workloads.DECODE_GROUPS]
    for name, N, K in layer:
        W = workloads.latent_weights(N, K, seed=0).to(dev)
        p, s = bw.pack_weights(W)
        del W
        packed0.append(p)
        scales.append(s)
        xs.append(workloads.activations(1, K, seed=0, outliers=True).to(dev))
        outs.append(torch.empty((1, N), dtype=torch.float32, device=dev))
    set_bytes = sum(N * K // 4 for _, N, K in layer)
    R = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    copies = [packed0] + [[p.clone() for p in packed0] for _ in range(R - 1)]
    torch.cuda.synchronize()

    def launch_group(r, grp):
        if len(grp) == 1:
            i = grp[0]
            bw.quant_gemv(xs[i], copies[r][i], scales[i], "f32", out=outs[i])
        else:
            bw.quant_gemv_grouped(xs[grp[0]], [copies[r][i] for i in grp],
                                  [scales[i] for i in grp], "f32", out=[outs[i] for i in grp])

    def launch_set(r):
        for grp in groups:
            launch_group(r, grp)

    def launch_set_ungrouped(r):
        for i in range(len(layer)):
            bw.quant_gemv(xs[i], copies[r][i], scales[i], "f32", out=outs[i])

    if args.traffic_probe:
        traffic_probe(torch, launch_set, R, dev)
        return
    if args.gemm_probe:
        bench_gemm(bw, workloads, torch, np, dev, layer, R_bytes=ROTATE_BYTES,
                   reps=args.kernel_reps, probe=True)
        return

    # Steps are captured STEPS_PER_GRAPH at a time, each on the next weight copy, so the
    # host's graph submissions never pace the GPU; one-step graphs cover the remainder.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch_set(0)  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_step = run_steps(torch, launch_set, R, args.warmup, args.steps)
    value = set_bytes / (ms_step * 1e-3) / 1e9
    ms_step_ungrouped = run_steps(torch, launch_set_ungrouped, R, args.warmup, args.steps)

    # ---- per-launch kernel durations: one graph per launch holding R back-to-back
    # launches (one per weight copy); event time of the replay / R ----
    per_group_us = [graph_launch_us(torch, lambda r, grp=grp: launch_group(r, grp), R,
                                    args.kernel_reps) for grp in groups]
    per_shape_us = [graph_launch_us(torch, lambda r, i=i: bw.quant_gemv(
        xs[i], copies[r][i], scales[i], "f32", out=outs[i]), R, args.kernel_reps)
        for i in range(len(layer))]
    kern_us_total = sum(per_group_us)
    achieved = set_bytes / (kern_us_total * 1e-6) / 1e9
    # the floor of each launch's grid: a plain streaming read of the launch's packed
    # bytes with the same number of 256-thread blocks (one per 16 weight rows)
    from ternary_weight_linear_token_amd import ceilings
    shapes = {name: (N, K) for name, N, K in layer}
    floor_us = [ceilings.same_grid_read_us(
        torch, dev, sum(shapes[n][0] * shapes[n][1] // 4 for n in grp),
        sum((shapes[n][0] + 15) // 16 for n in grp),
        lambda launch, R: graph_launch_us(torch, launch, R, args.kernel_reps))
        for grp in workloads.DECODE_GROUPS]
    kernel_hash = bw_build.kernel_hash("skinny.hip")
    traffic_bytes = load_traffic(kernel_hash)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic_bytes,
        "kernel": "skinny_kernel, fused quant+GEMV, M=1 specialization",
        "launches_per_step": len(groups),
        "mean_launch_us": round(kern_us_total / len(groups), 3),
        "algorithmic_bytes_per_launch": set_bytes / len(groups),
        "per_launch_us": {"|".join(grp): round(us, 3)
                          for grp, us in zip(workloads.DECODE_GROUPS, per_group_us)},
        "same_grid_plain_read_us": {"|".join(grp): round(us, 3)
                                    for grp, us in zip(workloads.DECODE_GROUPS, floor_us)},
        "frac_of_same_grid_plain_read": round(sum(floor_us) / kern_us_total, 4),
        "ungrouped_per_shape_us": {name: round(us, 3)
                                   for (name, _, _), us in zip(layer, per_shape_us)},
        "ungrouped_achieved": round(set_bytes / (sum(per_shape_us) * 1e-6) / 1e9, 1),
    }

    # ---- prefill GEMM, M = 512 ----
    gemm = bench_gemm(bw, workloads, torch, np, dev, layer, R_bytes=ROTATE_BYTES,
                      reps=args.kernel_reps)

    # ---- CPU oracle baseline ----
    cpu = None if args.no_cpu_baseline else cpu_baseline(workloads, layer, args.cpu_seconds)

    # ---- the shapes where the bandwidth and matrix-core bars are reachable ----
    extras = None if args.no_extras else bench_extras(bw, workloads, torch, dev, args.kernel_reps)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "bitnet-2b-decode-layer-set",
            "M": 1,
            "shapes_NK": [[N, K] for _, N, K in layer],
            "entry": "bitnet_quant_gemv_grouped / bitnet_quant_gemv (fused quant + GEMV), "
                     "fp32 out, HIP graphs of steps",
            "launches": ["|".join(grp) for grp in workloads.DECODE_GROUPS],
            "value_ungrouped": round(set_bytes / (ms_step_ungrouped * 1e-3) / 1e9, 1),
            "ms_per_step_ungrouped": round(ms_step_ungrouped, 5),
            "packed_bytes_per_step": set_bytes,
            "weight_copies_rotated": R,
            "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": roofline,
        "gemm": gemm,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(result), flush=True)


STEPS_PER_GRAPH = 10


def run_steps(torch, launch_step, R, warmup, steps):
    """Run `warmup` untimed steps, then time exactly `steps` steps (ms per step).

    Step s uses weight copy s % R.  Steps run as graph replays: graphs of STEPS_PER_GRAPH
    consecutive steps, then one-step graphs for what is left of `steps`."""
    S = STEPS_PER_GRAPH

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(count):
                launch_step((first + j) % R)
        return g

    # the sequence of (first step, count) replays for warmup + timed steps
    def plan(first, count):
        out = []
        while count >= S:
            out.append((first, S))
            first += S
            count -= S
        out += [(first + j, 1) for j in range(count)]
        return out

    graphs = {}
    warm, timed = plan(0, warmup), plan(warmup, steps)
    for first, count in warm + timed:
        key = (first % R, count)
        if key not in graphs:
            graphs[key] = capture(first % R, count)
    torch.cuda.synchronize()
    for first, count in warm:
        graphs[(first % R, count)].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for first, count in timed:
        graphs[(first % R, count)].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def traffic_probe(torch, launch_set, R, dev):
    """Launch pattern for the HBM counters: first three calibration launches of a plain
    elementwise kernel that reads and writes a known number of bytes (torch.neg on int32,
    profiling.COPY_BYTES each, twice the Infinity Cache), then the decode step once per
    weight copy (so the weights come from HBM), eagerly."""
    from ternary_weight_linear_token_amd import profiling
    n = profiling.COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    for r in range(R):
        launch_set(r)
    torch.cuda.synchronize()
    print(f"[bench] traffic probe: {R} decode steps", file=sys.stderr)


def graph_launch_us(torch, launch, R, reps):
    """Mean duration (us) of one launch: R launches (weight copies 0..R-1) captured in a
    graph and replayed back to back, timed with events on the launching stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            launch(r)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (reps * R)


def bench_extras(bw, workloads, torch, dev, reps):
    """Per-launch rooflines at large shapes: the 70B-shaped decode layer set (M = 1, fused
    quant + GEMV, packed GB/s against 8 TB/s) and the 8B-shaped prefill MLP GEMMs
    (M = 2048, quant excluded, int8 TOPS against 5.0 POPS).  Same method as the
    headline: graphs of back-to-back launches over weight copies rotated past 1 GiB."""
    out = {}
    print("[bench] 70B-shaped decode set, M=1", file=sys.stderr, flush=True)
    shapes = {name: (N, K) for name, N, K in workloads.LAYER_70B}
    from ternary_weight_linear_token_amd import ceilings
    per, tot_b, tot_us, tot_floor = {}, 0, 0.0, 0.0
    for grp in workloads.DECODE_GROUPS:
        K = shapes[grp[0]][1]
        ps, ss = [], []
        for name in grp:
            W = workloads.latent_weights(shapes[name][0], K, seed=0).to(dev)
            p, s = bw.pack_weights(W)
            del W
            ps.append(p)
            ss.append(s)
        nbytes = sum(shapes[name][0] * K // 4 for name in grp)
        R = max(2, math.ceil(ROTATE_BYTES / nbytes))
        copies = [ps] + [[p.clone() for p in ps] for _ in range(R - 1)]
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        os_ = [torch.empty((1, shapes[name][0]), dtype=torch.float32, device=dev) for name in grp]
        if len(grp) == 1:
            launch = lambda r: bw.quant_gemv(x, copies[r][0], ss[0], "f32", out=os_[0])
        else:
            launch = lambda r: bw.quant_gemv_grouped(x, copies[r], ss, "f32", out=os_)
        us = graph_launch_us(torch, launch, R, reps)
        del copies, ps
        torch.cuda.empty_cache()
        floor = ceilings.same_grid_read_us(
            torch, dev, nbytes, sum((shapes[name][0] + 15) // 16 for name in grp),
            lambda fn, RR: graph_launch_us(torch, fn, RR, reps))
        per["|".join(grp)] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                              "same_grid_plain_read_us": round(floor, 3)}
        tot_b += nbytes
        tot_us += us
        tot_floor += floor
        torch.cuda.empty_cache()
    out["decode_70b_m1"] = {"bound": "hbm", "achieved": round(tot_b / tot_us / 1e3, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(tot_b / tot_us / 1e3 / HBM_PEAK_GBS, 4),
                            "packed_bytes": tot_b, "per_launch": per,
                            "frac_of_same_grid_plain_read": round(tot_floor / tot_us, 4)}
    print("[bench] 8B-shaped prefill MLP, M=2048", file=sys.stderr, flush=True)
    M, per, tot_ops, tot_us = 2048, {}, 0.0, 0.0
    for name, N, K in workloads.LAYER_8B:
        if name not in ("gate", "down"):
            continue
        W = workloads.latent_weights(N, K, seed=0).to(dev)
        p, s = bw.pack_weights(W)
        del W
        R = max(2, math.ceil(ROTATE_BYTES / (N * K // 4)))
        copies = [p] + [p.clone() for _ in range(R - 1)]
        xq, a = bw.quant_act(workloads.activations(M, K, seed=0, outliers=True).to(dev))
        o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = graph_launch_us(torch, lambda r: bw.gemm(xq, a, copies[r], s, "bf16", out=o), R, reps)
        ops = 2.0 * M * N * K
        per[name] = {"us": round(us, 3), "TFLOP/s": round(ops / us / 1e6, 1)}
        tot_ops += ops
        tot_us += us
        del copies, p
        torch.cuda.empty_cache()
    out["prefill_8b_m2048"] = {"bound": "mfma", "achieved": round(tot_ops / tot_us / 1e6, 1),
                               "peak": INT8_MFMA_PEAK_TOPS, "unit": "TFLOP/s",
                               "frac": round(tot_ops / tot_us / 1e6 / INT8_MFMA_PEAK_TOPS, 4),
                               "per_shape": per}
    # the decode MLP as two launches: gate|up with the SwiGLU epilogue (h in bf16), then
    # down on h (fused quant + GEMV); 2B shapes, M = 1
    print("[bench] 2B decode MLP chain, M=1", file=sys.stderr, flush=True)
    shapes = {name: (N, K) for name, N, K in workloads.LAYER_2B}
    (Ni, Kh), (Nd, Kd) = shapes["gate"], shapes["down"]
    mats = {}
    for seed, name, (N, K) in ((0, "gate", (Ni, Kh)), (1, "up", (Ni, Kh)), (2, "down", (Nd, Kd))):
        mats[name] = bw.pack_weights(workloads.latent_weights(N, K, seed=seed).to(dev))
    nbytes = (2 * Ni * Kh + Nd * Kd) // 4
    R = max(2, math.ceil(ROTATE_BYTES / nbytes))
    copies = [mats] + [{k: (v[0].clone(), v[1]) for k, v in mats.items()} for _ in range(R - 1)]
    x = workloads.activations(1, Kh, seed=0, outliers=True).to(dev)
    h = torch.empty((1, Ni), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, Nd), dtype=torch.float32, device=dev)

    def mlp(r):
        c = copies[r]
        bw.quant_gemv_swiglu(x, c["gate"][0], c["gate"][1], c["up"][0], c["up"][1], "bf16", out=h)
        bw.quant_gemv(h, c["down"][0], c["down"][1], "f32", out=y)

    us = graph_launch_us(torch, mlp, R, reps)
    out["mlp_decode_2b_m1"] = {"launches": 2, "us": round(us, 3),
                               "packed_GB/s": round(nbytes / us / 1e3, 1),
                               "packed_bytes": nbytes}
    del copies, mats
    torch.cuda.empty_cache()

    # bf16 activations times ternary weights (no activation quantization), 2B set at M = 1
    print("[bench] 2B decode set with bf16 activations, M=1", file=sys.stderr, flush=True)
    per, tot_b, tot_us = {}, 0, 0.0
    for name, N, K in workloads.LAYER_2B:
        p, sc = bw.pack_weights(workloads.latent_weights(N, K, seed=0).to(dev))
        R = max(2, math.ceil(ROTATE_BYTES / (N * K // 4)))
        copies = [p] + [p.clone() for _ in range(R - 1)]
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        o = torch.empty((1, N), dtype=torch.float32, device=dev)
        us = graph_launch_us(torch, lambda r: bw.a16_gemv(x, copies[r], sc, "f32", out=o), R, reps)
        per[name] = round(us, 3)
        tot_b += N * K // 4
        tot_us += us
        del copies, p
    torch.cuda.empty_cache()
    out["a16_decode_2b_m1"] = {"achieved_GB/s": round(tot_b / tot_us / 1e3, 1),
                               "per_shape_us": per}

    # what this chip sustains (context for the fractions above)
    print("[bench] ceilings", file=sys.stderr, flush=True)
    mfma = ceilings.mfma_i8_tops(torch, dev)
    read = ceilings.hbm_read_gbs(torch, dev)
    vendor = {f"{M}x{N}x{K}": (None if t is None else round(t, 1)) for (M, N, K), t in
              (((M, N, K), ceilings.vendor_int8_gemm_tops(torch, dev, M, N, K))
               for M, N, K in ((2048, 14336, 4096), (2048, 4096, 14336), (512, 6912, 2560)))}
    out["ceilings"] = {
        "mfma_i8_register_loop_tops": round(mfma, 1),
        "mfma_i8_register_loop_frac_of_peak": round(mfma / INT8_MFMA_PEAK_TOPS, 4),
        "hbm_stream_read_2GiB_gbs": round(read, 1),
        "hbm_stream_read_frac_of_peak": round(read / HBM_PEAK_GBS, 4),
        "vendor_int8_gemm_tops_dense_int8_weights": vendor,
    }
    return out


def bench_gemm(bw, workloads, torch, np, dev, layer, R_bytes, reps, probe=False):
    M = 512
    print(f"[bench] prefill M={M}", file=sys.stderr, flush=True)
    packed0, scales, xs, xqs, avs, outs = [], [], [], [], [], []
    for name, N, K in layer:
        W = workloads.latent_weights(N, K, seed=0).to(dev)
        p, s = bw.pack_weights(W)
        del W
        packed0.append(p)
        scales.append(s)
        x = workloads.activations(M, K, seed=0, outliers=True).to(dev)
        xs.append(x)
        xq, a = bw.quant_act(x)
        xqs.append(xq)
        avs.append(a)
        outs.append(torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    set_bytes = sum(N * K // 4 for _, N, K in layer)
    R = max(2, math.ceil(R_bytes / set_bytes))
    copies = [packed0] + [[p.clone() for p in packed0] for _ in range(R - 1)]
    ops = sum(2.0 * M * N * K for _, N, K in layer)

    # projections that read the same activations share one quantization (q|k|v, gate|up)
    index = {name: i for i, (name, _, _) in enumerate(layer)}
    groups = [[index[n] for n in grp] for grp in workloads.DECODE_GROUPS]

    def grouped(r, grp):
        i0 = grp[0]
        return bw.gemm_grouped(xqs[i0], avs[i0], [copies[r][i] for i in grp],
                               [scales[i] for i in grp], "bf16", out=[outs[i] for i in grp])

    def step(r):
        for grp in groups:
            i0 = grp[0]
            bw.quant_act(xs[i0], xq=xqs[i0], a_scale=avs[i0])
            grouped(r, grp)

    if probe:
        # counter collection: the calibration copies of the traffic probe, then the four
        # grouped GEMM launches once per weight copy (weights from HBM), eagerly
        from ternary_weight_linear_token_amd import profiling
        n = profiling.COPY_BYTES // 4
        src = torch.arange(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        for r in range(R):
            for grp in groups:
                grouped(r, grp)
        torch.cuda.synchronize()
        print(f"[bench] gemm probe: {R} prefill steps", file=sys.stderr)
        return None

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_step = run_steps(torch, step, R, 3, 40)

    per_group_us = [graph_launch_us(torch, lambda r, grp=grp: grouped(r, grp), R, reps)
                    for grp in groups]
    per_shape_us = [graph_launch_us(torch, lambda r, i=i: bw.gemm(
        xqs[i], avs[i], copies[r][i], scales[i], "bf16", out=outs[i]), R, reps)
        for i in range(len(layer))]
    tops = ops / (sum(per_group_us) * 1e-6) / 1e12
    # context: the vendor int8 GEMM (hipBLASLt, dense int8 weights) on the same four
    # products (each group's matrices concatenated along N)
    from ternary_weight_linear_token_amd import ceilings
    shapes = {name: (N, K) for name, N, K in layer}
    vendor_us = 0.0
    for grp in workloads.DECODE_GROUPS:
        N = sum(shapes[n][0] for n in grp)
        K = shapes[grp[0]][1]
        t = ceilings.vendor_int8_gemm_tops(torch, dev, M, N, K)
        vendor_us = None if (t is None or vendor_us is None) else vendor_us + 2.0 * M * N * K / t / 1e6
    from ternary_weight_linear_token_amd import build as bw_build
    counters = load_summary(GEMM_COUNTERS_FILE, bw_build.kernel_hash("tiled.hip"))
    return {
        "metric": "GEMM int8 TOPS at M=512 (prefill layer set, bf16 out)",
        "workload": "bitnet-2b-prefill-layer-set",
        "value": round(tops, 2),
        "unit": "TOPS",
        "launches": ["|".join(grp) for grp in workloads.DECODE_GROUPS],
        "step_tops_incl_quant": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "step": "one quant_act + one grouped tiled GEMM per shared input (q|k|v, o, gate|up, "
                "down)",
        "ms_per_step_incl_quant": round(ms_step, 4),
        "value_ungrouped": round(ops / (sum(per_shape_us) * 1e-6) / 1e12, 2),
        "vendor_int8_gemm_same_products_tops": (None if vendor_us is None else
                                                round(ops / (vendor_us * 1e-6) / 1e12, 2)),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tops, 2),
            "peak": INT8_MFMA_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4),
            "traffic": float(counters["hbm_bytes_per_launch"]) if counters else None,
            "mfma_busy_frac_counters": (float(counters["mfma_busy_frac_weighted"])
                                        if counters else None),
            "kernel": "tiled_kernel (tile plan per launch)",
            "per_launch_us": {"|".join(grp): round(us, 3)
                              for grp, us in zip(workloads.DECODE_GROUPS, per_group_us)},
            "ungrouped_per_shape_us": {name: round(us, 3)
                                       for (name, _, _), us in zip(layer, per_shape_us)},
        },
    }


def cpu_baseline(workloads, layer, seconds):
    """The CPU oracle on the decode step (act quant + accumulate + rescale per shape)."""
    import oracle
    print(f"[bench] cpu oracle baseline (~{seconds:.0f} s)", file=sys.stderr, flush=True)
    prep = []
    for name, N, K in layer:
        packed, w_scale = oracle.pack_weights(workloads.latent_weights(N, K, seed=0).numpy())
        xb = workloads.bf16_bits(workloads.activations(1, K, seed=0, outliers=True))
        prep.append((packed, w_scale, xb, K))
    set_bytes = sum(N * K // 4 for _, N, K in layer)
    n = 0
    t0 = time.perf_counter()
    while True:
        for packed, w_scale, xb, K in prep:
            xq, a = oracle.act_quant(xb)
            acc = oracle.accumulate(xq, packed, K)
            oracle.rescale(acc, a, w_scale)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(set_bytes * n / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"2B decode layer set at M=1 (act quant + accumulate + rescale, pack "
                  f"excluded), {n} passes in {dt:.1f} s",
    }


if __name__ == "__main__":
    main()
