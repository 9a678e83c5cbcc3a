#!/usr/bin/env python3
"""Benchmark of the W2A8 BitLinear hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-sweep]
python bench.py --traffic-probe   (launch pattern for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)
python bench.py --gemm-probe      (prefill GEMM launches for rocprofv3 --pmc)

A step is one BitNet-2B-shaped decode layer set at M = 1: the seven projections
(q, k, v, o, gate, up, down; (N, K) = (2560,2560) (640,2560) (640,2560) (2560,2560)
(6912,2560) (6912,2560) (2560,6912)), bf16 activations in, fp32 out, every step of the
path: absmax, quantize, stream and unpack the packed weights, int8 x ternary dot with
int32 accumulation, rescale.  Projections that read the same activations share one
fused quant + GEMV launch (q|k|v, o, gate|up, down: four launches); the same set with
one launch per projection is reported beside it (value_ungrouped).

* Inputs are resident in HBM before timing.  Every timed graph rotates over copies of
  the weights it reads that together exceed 1 GiB (four times the 256 MB Infinity
  Cache), so the weights come from HBM: the step over copies of the whole set, and each
  per-launch graph over copies of that launch's own matrices.
* Steps are captured in HIP graphs, thirty consecutive steps (each on the next weight
  copy; thirty is the 2B model's layer count, so one graph is one model decode step) per
  graph, so host submission does not pace the GPU; W warmup steps, then exactly K steps
  between two synchronizations timed with events.
* value = packed-weight bytes of the set / step time (GB/s).
* roofline: the fused quant+GEMV kernel, algorithmic bytes (N*K/4 packed bytes per
  launch) / its mean launch duration (a graph of back-to-back launches over the
  launch's weight copies, timed with events on the launching stream), against 8 TB/s;
  traffic from the committed rocprofv3 counter summary when it matches the current
  kernel source.
* gemm: the BitNet-2B-shaped prefill set at M = 512 (tiled int8-MFMA GEMM, bf16 out),
  with the projections that share an input in one grouped launch (q|k|v, o, gate|up,
  down), int8 TOPS against 5.0 POPS dense from the per-launch GEMM durations; the step
  rate with the four quantization launches and the rate of seven ungrouped launches are
  reported beside it.
* sweep: every (shape, M) of the 8B-shaped sweep (M = 1, 4, 16, 64, 256, 2048) and the
  70B-shaped chain (M = 1, 32, 1024): M <= 16 through the fused quant + GEMV entry point,
  larger M through the GEMM entry point on int8 activations (the quantization launch
  timed beside it).  Each entry gives the time, packed GB/s, TOPS, the roofline that
  binds (HBM or int8 MFMA, from the algorithmic bytes and operations), the attainable
  rate min(peak, arithmetic intensity x bandwidth) and the fractions of both.
* cpu_baseline: the CPU oracle on the host cores (test infrastructure, timed only
  here), on the same decode step repeated for ~10 s.
* extras: the 70B-shaped decode layer set at M = 1 with grouped launches and the
  same-grid read floors; the 2B decode MLP as two launches (gate|up with the SwiGLU
  epilogue, then down); the 2B decode set with bf16 activations (W1.58A16); and
  ceilings measured on this chip: an int8 matrix-core loop on register operands with
  the core clock it sustained, a 2 GiB streaming read, and the vendor int8 GEMM
  (hipBLASLt, dense int8 weights) at prefill shapes.
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
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 8B- and 70B-shaped (shape, M) sweep")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 70B decode set, MLP chain, W1.58A16 set and the ceilings")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the counter-collection launch pattern and exit (no timing)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="run the prefill GEMM launches for counter collection and exit")
    ap.add_argument("--large-probe", action="store_true",
                    help="run the 8B M=2048 / 70B M=1024 GEMMs and the 70B M=1 decode "
                         "launches for counter collection and exit")
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


# launches per graph when the activation quantization is timed on its own (its input is
# the same tensor each time, as a layer's input would come from the layer before)
QUANT_LAUNCHES = 32


def rotation(tensors, nbytes):
    """Copies of `tensors` (nbytes together) whose total exceeds ROTATE_BYTES: entry r
    of the returned list is the r-th copy (entry 0 the tensors themselves)."""
    R = max(2, math.ceil(ROTATE_BYTES / nbytes))
    return [list(tensors)] + [[t.clone() for t in tensors] for _ in range(R - 1)]


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
    copies = rotation(packed0, set_bytes)
    R = len(copies)
    torch.cuda.synchronize()

    def launch_group(c, grp):
        """One launch of group grp (indices into layer) on weight list c (by layer index)."""
        if len(grp) == 1:
            i = grp[0]
            bw.quant_gemv(xs[i], c[i], scales[i], "f32", out=outs[i])
        else:
            bw.quant_gemv_grouped(xs[grp[0]], [c[i] for i in grp], [scales[i] for i in grp],
                                  "f32", out=[outs[i] for i in grp])

    def launch_set(r):
        for grp in groups:
            launch_group(copies[r], grp)

    def launch_set_ungrouped(r):
        for i in range(len(layer)):
            bw.quant_gemv(xs[i], copies[r][i], scales[i], "f32", out=outs[i])

    if args.traffic_probe:
        traffic_probe(torch, launch_set, R, dev)
        return
    if args.large_probe:
        del copies
        large_probe(bw, workloads, torch, dev)
        return
    if args.gemm_probe:
        bench_gemm(bw, workloads, torch, dev, layer, reps=args.kernel_reps, probe=True)
        return


    # ---- per-launch kernel durations: one graph per launch holding back-to-back
    # launches over that launch's own weight copies (> 1 GiB together); event time of
    # the replay / launches ----
    shapes = {name: (N, K) for name, N, K in layer}

    def group_us(grp):
        nbytes = sum(shapes[layer[i][0]][0] * shapes[layer[i][0]][1] // 4 for i in grp)
        cp = rotation([packed0[i] for i in grp], nbytes)

        def launch(r):
            c = dict(zip(grp, cp[r]))
            launch_group(c, grp)

        us = graph_launch_us(torch, launch, len(cp), args.kernel_reps)
        del cp
        torch.cuda.empty_cache()
        return us

    per_group_us = [group_us(grp) for grp in groups]
    per_shape_us = [group_us([i]) for i in range(len(layer))]
    kern_us_total = sum(per_group_us)
    achieved = set_bytes / (kern_us_total * 1e-6) / 1e9
    # the floor of each launch: a plain streaming read of the launch's packed bytes with
    # one 256-thread block per 16 weight rows (the kernel's grid, or twice it where the
    # kernel's blocks take 32 rows), and with 1/2, 2 and 4 times as many blocks
    from ternary_weight_linear_token_amd import ceilings
    grid_factors = (1, 0.5, 2, 4)
    floor_sweep = [[ceilings.same_grid_read_us(
        torch, dev, sum(shapes[n][0] * shapes[n][1] // 4 for n in grp),
        max(1, int(f * sum((shapes[n][0] + 15) // 16 for n in grp))),
        lambda launch, RR: graph_launch_us(torch, launch, RR, args.kernel_reps))
        for f in grid_factors] for grp in workloads.DECODE_GROUPS]
    floor_us = [fs[0] for fs in floor_sweep]
    counters = load_summary(TRAFFIC_FILE, bw_build.kernel_hash("skinny.hip"))
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": float(counters["hbm_bytes_per_launch"]) if counters else None,
        "kernel": "skinny_kernel, fused quant+GEMV, M=1 specialization",
        "launches_per_step": len(groups),
        "mean_launch_us": round(kern_us_total / len(groups), 3),
        "algorithmic_bytes_per_launch": set_bytes / len(groups),
        "per_launch_us": {"|".join(grp): round(us, 3)
                          for grp, us in zip(workloads.DECODE_GROUPS, per_group_us)},
        "same_grid_plain_read_us": {"|".join(grp): round(us, 3)
                                    for grp, us in zip(workloads.DECODE_GROUPS, floor_us)},
        "frac_of_same_grid_plain_read": round(sum(floor_us) / kern_us_total, 4),
        "plain_read_half_2x_4x_blocks_us": {"|".join(grp): [round(u, 3) for u in fs[1:]]
                                            for grp, fs in zip(workloads.DECODE_GROUPS, floor_sweep)},
        "frac_of_best_grid_plain_read": round(sum(min(fs) for fs in floor_sweep) / kern_us_total, 4),
        "ungrouped_per_shape_us": {name: round(us, 3)
                                   for (name, _, _), us in zip(layer, per_shape_us)},
        "ungrouped_achieved": round(set_bytes / (sum(per_shape_us) * 1e-6) / 1e9, 1),
    }
    # ---- the step: timed after the per-launch measurements above, so that it runs on a
    # GPU already at its working clocks rather than ramping up from idle during a short
    # timed region.  Steps are captured STEPS_PER_GRAPH at a time, each on the next
    # weight copy, so the host's graph submissions never pace the GPU; one shorter graph
    # covers the remainder. ----
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch_set(0)  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_step = run_steps(torch, launch_set, R, args.warmup, args.steps)
    value = set_bytes / (ms_step * 1e-3) / 1e9
    ms_step_ungrouped = run_steps(torch, launch_set_ungrouped, R, args.warmup, args.steps)
    del copies
    torch.cuda.empty_cache()
    del packed0
    torch.cuda.empty_cache()

    # ---- prefill GEMM, M = 512 ----
    gemm = bench_gemm(bw, workloads, torch, dev, layer, reps=args.kernel_reps)

    # ---- CPU oracle baseline ----
    cpu = None if args.no_cpu_baseline else cpu_baseline(workloads, layer, args.cpu_seconds)

    # ---- every (shape, M) of the 8B-shaped sweep and the 70B-shaped chain ----
    sweep = None if args.no_sweep else bench_sweep(bw, workloads, torch, dev, args.kernel_reps)

    # ---- large-shape decode set, MLP chain, bf16 activations, measured ceilings ----
    extras = None if args.no_extras else bench_extras(bw, workloads, torch, dev, args.kernel_reps)
    if extras is not None and sweep is not None:
        extras.update(sweep_summaries(sweep))

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
        "sweep": sweep,
        "extras": extras,
    }
    print(json.dumps(result), flush=True)


# Layer steps per captured graph: 30, the layer count of the 2B model, i.e. one graph per
# model decode step, as a serving loop would replay it.  A graph replay costs a few µs of
# its own (about 8 µs here), which this spreads over the step's layers.
STEPS_PER_GRAPH = 30


def run_steps(torch, launch_step, R, warmup, steps):
    """Run `warmup` untimed steps, then time exactly `steps` steps (ms per step).

    Step s uses weight copy s % R.  Steps run as graph replays: graphs of STEPS_PER_GRAPH
    consecutive steps, then one graph of what is left of `steps`."""
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
        while count > 0:
            c = min(S, count)
            out.append((first, c))
            first += c
            count -= c
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


def calibration_copies(torch, dev):
    """Three launches of a plain elementwise kernel that reads and writes a known number
    of bytes (torch.neg on int32, profiling.COPY_BYTES each, twice the Infinity Cache):
    the reference the HBM byte counters are scaled by."""
    from ternary_weight_linear_token_amd import profiling
    n = profiling.COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def traffic_probe(torch, launch_set, R, dev):
    """Launch pattern for the HBM counters: the calibration copies, then the decode step
    once per weight copy (so the weights come from HBM), eagerly."""
    calibration_copies(torch, dev)
    for r in range(R):
        launch_set(r)
    torch.cuda.synchronize()
    print(f"[bench] traffic probe: {R} decode steps", file=sys.stderr)


# the launches of --large-probe, in order: (name, M, N per group, K); each runs once per
# weight copy of a rotation past 1 GiB, eagerly, after the calibration copies
LARGE_PROBE_GEMM = [("8b_gate_m2048", 2048, (14336,), 4096), ("8b_down_m2048", 2048, (4096,), 14336),
                    ("70b_gate_up_m1024", 1024, (28672, 28672), 8192),
                    ("70b_down_m1024", 1024, (8192,), 28672)]


def large_probe(bw, workloads, torch, dev):
    """Counter-collection pattern for the large shapes: the calibration copies, the 70B
    decode set at M = 1 (grouped fused quant + GEMV launches), then the large prefill
    GEMMs (int8 in, bf16 out), each over weight copies rotated past 1 GiB."""
    calibration_copies(torch, dev)
    shapes = {name: (N, K) for name, N, K in workloads.LAYER_70B}
    for grp in workloads.DECODE_GROUPS:
        K = shapes[grp[0]][1]
        ps, ss = [], []
        for name in grp:
            p, s = bw.pack_weights(workloads.latent_weights_on(dev, shapes[name][0], K, seed=0))
            ps.append(p)
            ss.append(s)
        cp = rotation(ps, sum(shapes[n][0] * K // 4 for n in grp))
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        for c in cp:
            if len(grp) == 1:
                bw.quant_gemv(x, c[0], ss[0], "f32")
            else:
                bw.quant_gemv_grouped(x, c, ss, "f32")
        torch.cuda.synchronize()
        del cp, ps
        torch.cuda.empty_cache()
    for name, M, Ns, K in LARGE_PROBE_GEMM:
        ps, ss = [], []
        for N in Ns:
            p, s = bw.pack_weights(workloads.latent_weights_on(dev, N, K, seed=0))
            ps.append(p)
            ss.append(s)
        cp = rotation(ps, sum(N * K // 4 for N in Ns))
        xq, a = bw.quant_act(workloads.activations(M, K, seed=0, outliers=True).to(dev))
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for N in Ns]
        for c in cp:
            if len(Ns) == 1:
                bw.gemm(xq, a, c[0], ss[0], "bf16", out=outs[0])
            else:
                bw.gemm_grouped(xq, a, c, ss, "bf16", out=outs)
        torch.cuda.synchronize()
        del cp, ps
        torch.cuda.empty_cache()
    print("[bench] large probe done", file=sys.stderr)


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


def roofline_entry(us, ops, nbytes):
    """Bound, attainable rate and fractions of one launch of `ops` int8 operations over
    `nbytes` algorithmic HBM bytes that took `us` microseconds.  The ideal time is the
    larger of ops / int8-MFMA peak and bytes / HBM peak; attainable = min(peak, AI x BW)
    in TOPS."""
    t_mfma = ops / (INT8_MFMA_PEAK_TOPS * 1e6)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e3)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    ai = ops / nbytes
    attainable = min(INT8_MFMA_PEAK_TOPS, ai * HBM_PEAK_GBS / 1e3)
    e = {"bound": bound, "ops_per_byte": round(ai, 2), "attainable_TOPS": round(attainable, 1),
         "frac_of_attainable": round(max(t_mfma, t_hbm) / us, 4)}
    if bound == "hbm":
        e["frac_hbm_peak"] = round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)
    else:
        e["frac_mfma_peak"] = round(ops / us / 1e6 / INT8_MFMA_PEAK_TOPS, 4)
    return e


def bench_sweep(bw, workloads, torch, dev, reps):
    """Every (shape, M) of the 8B-shaped sweep and the 70B-shaped chain: M <= 16 through
    the fused quant + GEMV entry point (bf16 in, fp32 out), larger M through the GEMM
    entry point (int8 in, bf16 out; the quantization launch is timed beside it).  Each
    launch is a graph of back-to-back launches over weight copies rotated past 1 GiB."""
    entries = []
    for wl, tag in (("8b_sweep", "8b"), ("70b_chain", "70b")):
        spec = workloads.WORKLOADS[wl]
        print(f"[bench] {tag}-shaped sweep, M in {spec['Ms']}", file=sys.stderr, flush=True)
        for name, N, K in workloads.distinct_shapes(spec["layer"]):
            W = workloads.latent_weights_on(dev, N, K, seed=0)
            p, s = bw.pack_weights(W)
            del W
            torch.cuda.empty_cache()
            cp = rotation([p], N * K // 4)
            R = len(cp)
            for M in spec["Ms"]:
                x = workloads.activations(M, K, seed=0, outliers=True).to(dev)
                two_launch_us = None
                if M <= bw.GEMV_MAX_M:
                    o = torch.empty((M, N), dtype=torch.float32, device=dev)
                    us = graph_launch_us(torch, lambda r: bw.quant_gemv(x, cp[r][0], s, "f32", out=o),
                                         R, reps)
                    nbytes = N * K // 4 + 4 * N + 2 * M * K + 4 * M * N
                    entry, quant_us = "bitnet_quant_gemv", None
                    if M > 1:
                        # the same product as two launches: quantization, then the int8
                        # product (what the bitlinear helper runs above 4 tokens or M * K = 32768)
                        xq, a = bw.quant_act(x)

                        def two(r):
                            bw.quant_act(x, xq=xq, a_scale=a)
                            bw.gemm(xq, a, cp[r][0], s, "f32", out=o)

                        two_launch_us = graph_launch_us(torch, two, R, reps)
                else:
                    xq, a = bw.quant_act(x)
                    o = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                    us = graph_launch_us(torch, lambda r: bw.gemm(xq, a, cp[r][0], s, "bf16", out=o),
                                         R, reps)
                    quant_us = graph_launch_us(torch, lambda r: bw.quant_act(x, xq=xq, a_scale=a),
                                               QUANT_LAUNCHES, reps)
                    nbytes = N * K // 4 + 4 * N + M * K + 4 * M + 2 * M * N
                    entry = "bitnet_w2a8_gemm"
                ops = 2.0 * M * N * K
                e = {"workload": tag, "shape": name, "N": N, "K": K, "M": M, "entry": entry,
                     "us": round(us, 3), "packed_GB/s": round(N * K / 4 / us / 1e3, 1),
                     "TOPS": round(ops / us / 1e6, 1)}
                e.update(roofline_entry(us, ops, nbytes))
                if quant_us is not None:
                    e["quant_us"] = round(quant_us, 3)
                if two_launch_us is not None:
                    e["quant_then_gemm_us"] = round(two_launch_us, 3)
                entries.append(e)
                del o, x
            del cp, p
            torch.cuda.empty_cache()
    return entries


def sweep_summaries(sweep):
    """Set-level figures from the sweep: the 8B MLP GEMMs at M = 2048 and the 70B chain's
    seven projections at M = 1024 (int8 TOPS against 5.0 POPS)."""
    def set_tops(tag, M, names):
        by = {(e["workload"], e["shape"], e["M"]): e for e in sweep}
        ops = us = 0.0
        per = {}
        for n in names:
            # projections of equal shape are measured once (v as k, o as q, up as gate)
            e = by.get((tag, n, M)) or by.get((tag, {"v": "k", "o": "q", "up": "gate"}.get(n, n), M))
            if e is None:
                return None
            ops += 2.0 * M * e["N"] * e["K"]
            us += e["us"]
            per[n] = {"us": e["us"], "TFLOP/s": e["TOPS"]}
        t = ops / us / 1e6
        return {"bound": "mfma", "achieved": round(t, 1), "peak": INT8_MFMA_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(t / INT8_MFMA_PEAK_TOPS, 4), "per_shape": per}

    out = {}
    s8 = set_tops("8b", 2048, ["gate", "down"])
    if s8:
        out["prefill_8b_m2048"] = s8
    s70 = set_tops("70b", 1024, ["q", "k", "v", "o", "gate", "up", "down"])
    if s70:
        out["prefill_70b_m1024_chain"] = s70
    return out


def bench_extras(bw, workloads, torch, dev, reps):
    """The 70B-shaped decode layer set (M = 1, grouped fused quant + GEMV launches, packed
    GB/s against 8 TB/s, with the same-grid read floors), the 2B decode MLP chain, the 2B
    decode set with bf16 activations, and the measured ceilings."""
    out = {}
    print("[bench] 70B-shaped decode set, M=1", file=sys.stderr, flush=True)
    shapes = {name: (N, K) for name, N, K in workloads.LAYER_70B}
    from ternary_weight_linear_token_amd import ceilings
    per, tot_b, tot_us, tot_floor, tot_best = {}, 0, 0.0, 0.0, 0.0
    for grp in workloads.DECODE_GROUPS:
        K = shapes[grp[0]][1]
        ps, ss = [], []
        for name in grp:
            W = workloads.latent_weights_on(dev, shapes[name][0], K, seed=0)
            p, s = bw.pack_weights(W)
            del W
            ps.append(p)
            ss.append(s)
        nbytes = sum(shapes[name][0] * K // 4 for name in grp)
        copies = rotation(ps, nbytes)
        R = len(copies)
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        os_ = [torch.empty((1, shapes[name][0]), dtype=torch.float32, device=dev) for name in grp]
        if len(grp) == 1:
            launch = lambda r: bw.quant_gemv(x, copies[r][0], ss[0], "f32", out=os_[0])
        else:
            launch = lambda r: bw.quant_gemv_grouped(x, copies[r], ss, "f32", out=os_)
        us = graph_launch_us(torch, launch, R, reps)
        del copies, ps
        torch.cuda.empty_cache()
        # the plain read of the same bytes with one 256-thread block per 16 weight rows
        # (the kernel's grid, or twice it where its blocks take 32 rows), and with 1/2, 2
        # and 4 times as many blocks: whether another grid would lower the floor
        blocks = sum((shapes[name][0] + 15) // 16 for name in grp)
        floors = [ceilings.same_grid_read_us(torch, dev, nbytes, max(1, int(blocks * f)),
                                             lambda fn, RR: graph_launch_us(torch, fn, RR, reps))
                  for f in (1, 0.5, 2, 4)]
        floor = floors[0]
        per["|".join(grp)] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                              "same_grid_plain_read_us": round(floor, 3),
                              "plain_read_half_2x_4x_blocks_us": [round(f, 3) for f in floors[1:]]}
        tot_b += nbytes
        tot_us += us
        tot_floor += floor
        tot_best += min(floors)
        torch.cuda.empty_cache()
    out["decode_70b_m1"] = {"bound": "hbm", "achieved": round(tot_b / tot_us / 1e3, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(tot_b / tot_us / 1e3 / HBM_PEAK_GBS, 4),
                            "packed_bytes": tot_b, "per_launch": per,
                            "frac_of_same_grid_plain_read": round(tot_floor / tot_us, 4),
                            "frac_of_best_grid_plain_read": round(tot_best / tot_us, 4)}
    # the decode MLP as two launches: gate|up with the SwiGLU epilogue (h in bf16), then
    # down on h (fused quant + GEMV); 2B shapes, M = 1
    print("[bench] 2B decode MLP chain, M=1", file=sys.stderr, flush=True)
    shapes = {name: (N, K) for name, N, K in workloads.LAYER_2B}
    (Ni, Kh), (Nd, Kd) = shapes["gate"], shapes["down"]
    mats = {}
    for seed, name, (N, K) in ((0, "gate", (Ni, Kh)), (1, "up", (Ni, Kh)), (2, "down", (Nd, Kd))):
        mats[name] = bw.pack_weights(workloads.latent_weights(N, K, seed=seed).to(dev))
    nbytes = (2 * Ni * Kh + Nd * Kd) // 4
    order = ("gate", "up", "down")
    cp = rotation([mats[k][0] for k in order], nbytes)
    R = len(cp)
    x = workloads.activations(1, Kh, seed=0, outliers=True).to(dev)
    h = torch.empty((1, Ni), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, Nd), dtype=torch.float32, device=dev)

    def mlp(r):
        g, u, d = cp[r]
        bw.quant_gemv_swiglu(x, g, mats["gate"][1], u, mats["up"][1], "bf16", out=h)
        bw.quant_gemv(h, d, mats["down"][1], "f32", out=y)

    us = graph_launch_us(torch, mlp, R, reps)
    out["mlp_decode_2b_m1"] = {"launches": 2, "us": round(us, 3),
                               "packed_GB/s": round(nbytes / us / 1e3, 1),
                               "packed_bytes": nbytes}
    del cp, mats
    torch.cuda.empty_cache()

    # bf16 activations times ternary weights (no activation quantization), 2B set at M = 1
    print("[bench] 2B decode set with bf16 activations, M=1", file=sys.stderr, flush=True)
    per, tot_b, tot_us = {}, 0, 0.0
    for name, N, K in workloads.LAYER_2B:
        p, sc = bw.pack_weights(workloads.latent_weights(N, K, seed=0).to(dev))
        cp = rotation([p], N * K // 4)
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        o = torch.empty((1, N), dtype=torch.float32, device=dev)
        us = graph_launch_us(torch, lambda r: bw.a16_gemv(x, cp[r][0], sc, "f32", out=o),
                             len(cp), reps)
        per[name] = round(us, 3)
        tot_b += N * K // 4
        tot_us += us
        del cp, p
        torch.cuda.empty_cache()
    out["a16_decode_2b_m1"] = {"achieved_GB/s": round(tot_b / tot_us / 1e3, 1),
                               "per_shape_us": per}

    for key, layer, M in (("prefill_8b_m2048_layer_grouped", workloads.LAYER_8B, 2048),
                          ("prefill_70b_m1024_layer_grouped", workloads.LAYER_70B, 1024)):
        print(f"[bench] {key}", file=sys.stderr, flush=True)
        out[key] = bench_layer_grouped(bw, workloads, torch, dev, layer, M, reps)
    out["b3_decode_70b_m1"] = bench_b3(bw, workloads, torch, dev, reps)

    # what this chip sustains (context for the fractions above)
    print("[bench] ceilings", file=sys.stderr, flush=True)
    mfma, ghz = ceilings.mfma_i8_tops(torch, dev)
    # the same loop on 16 CUs only: little power drawn, so the clock it reads is the
    # unthrottled one (checks the clock reading itself)
    _, ghz_light = ceilings.mfma_i8_tops(torch, dev, blocks=16, iters=20000)
    read = ceilings.hbm_read_gbs(torch, dev)
    vendor = {f"{M}x{N}x{K}": (None if t is None else round(t, 1)) for (M, N, K), t in
              (((M, N, K), ceilings.vendor_int8_gemm_tops(torch, dev, M, N, K))
               for M, N, K in ((2048, 14336, 4096), (2048, 4096, 14336), (512, 6912, 2560)))}
    out["ceilings"] = {
        "mfma_i8_register_loop_tops": round(mfma, 1),
        "mfma_i8_register_loop_frac_of_peak": round(mfma / INT8_MFMA_PEAK_TOPS, 4),
        "mfma_i8_register_loop_core_clock_ghz": None if ghz is None else round(ghz, 3),
        "mfma_i8_peak_at_that_clock_tops": (None if ghz is None else
                                            round(INT8_MFMA_PEAK_TOPS * ghz / 2.4, 1)),
        "core_clock_ghz_same_loop_on_16_cus": None if ghz_light is None else round(ghz_light, 3),
        "hbm_stream_read_2GiB_gbs": round(read, 1),
        "hbm_stream_read_frac_of_peak": round(read / HBM_PEAK_GBS, 4),
        "vendor_int8_gemm_tops_dense_int8_weights": vendor,
    }
    return out


def bench_layer_grouped(bw, workloads, torch, dev, layer, M, reps):
    """A whole layer's seven projections at M tokens as the four launches a layer runs
    (q|k|v and gate|up grouped on their shared input, o, down), int8 in, bf16 out: each
    launch is a graph over copies of its own weights rotated past 1 GiB.  int8 TOPS of
    the set against 5.0 POPS."""
    shapes = {name: (N, K) for name, N, K in layer}
    per, ops, tot_us = {}, 0.0, 0.0
    for grp in workloads.DECODE_GROUPS:
        K = shapes[grp[0]][1]
        ps, ss = [], []
        for name in grp:
            W = workloads.latent_weights_on(dev, shapes[name][0], K, seed=0)
            p, s = bw.pack_weights(W)
            del W
            ps.append(p)
            ss.append(s)
        x = workloads.activations(M, K, seed=0, outliers=True).to(dev)
        xq, a = bw.quant_act(x)
        del x
        outs = [torch.empty((M, shapes[n][0]), dtype=torch.bfloat16, device=dev) for n in grp]
        copies = rotation(ps, sum(shapes[n][0] * K // 4 for n in grp))
        if len(grp) == 1:
            launch = lambda r: bw.gemm(xq, a, copies[r][0], ss[0], "bf16", out=outs[0])
        else:
            launch = lambda r: bw.gemm_grouped(xq, a, copies[r], ss, "bf16", out=outs)
        us = graph_launch_us(torch, launch, len(copies), reps)
        g_ops = sum(2.0 * M * shapes[n][0] * K for n in grp)
        per["|".join(grp)] = {"us": round(us, 3), "TFLOP/s": round(g_ops / us / 1e6, 1)}
        ops += g_ops
        tot_us += us
        del copies, ps, outs, xq
        torch.cuda.empty_cache()
    t = ops / tot_us / 1e6
    return {"bound": "mfma", "achieved": round(t, 1), "peak": INT8_MFMA_PEAK_TOPS,
            "unit": "TFLOP/s", "frac": round(t / INT8_MFMA_PEAK_TOPS, 4), "M": M,
            "launches": per}


def bench_b3(bw, workloads, torch, dev, reps):
    """The 70B-shaped decode layer (seven projections, one launch each, M = 1, fused
    quantization) with weights five per byte (1.6 bits) against the same launches on the
    2-bit format; weight copies rotated past 1 GiB for both."""
    print("[bench] 70B decode set, 1.6-bit weights against 2-bit, M=1", file=sys.stderr,
          flush=True)
    per, t2, t3, b2, b3b = {}, 0.0, 0.0, 0, 0
    for name, N, K in workloads.distinct_shapes(workloads.LAYER_70B):
        count = sum(1 for n, NN, KK in workloads.LAYER_70B if (NN, KK) == (N, K))
        W = workloads.latent_weights_on(dev, N, K, seed=0)
        p, s = bw.pack_weights(W)
        del W
        q = bw.pack_b3(p, K)
        x = workloads.activations(1, K, seed=0, outliers=True).to(dev)
        o = torch.empty((1, N), dtype=torch.float32, device=dev)
        cp = rotation([p], N * K // 4)
        us2 = graph_launch_us(torch, lambda r: bw.quant_gemv(x, cp[r][0], s, "f32", out=o),
                              len(cp), reps)
        del cp
        cq = rotation([q], q.numel())
        us3 = graph_launch_us(torch, lambda r: bw.quant_gemv_b3(x, cq[r][0], s, "f32", out=o),
                              len(cq), reps)
        del cq, p, q
        torch.cuda.empty_cache()
        per[name] = {"us_2bit": round(us2, 3), "us_1p6bit": round(us3, 3),
                     "launches_per_layer": count}
        t2 += count * us2
        t3 += count * us3
        b2 += count * N * K // 4
        b3b += count * N * bw.b3_row_bytes(K)
    return {"packed_bytes_2bit": b2, "packed_bytes_1p6bit": b3b,
            "us_2bit": round(t2, 3), "us_1p6bit": round(t3, 3),
            "speedup_1p6_over_2bit": round(t2 / t3, 4),
            "GB/s_2bit": round(b2 / t2 / 1e3, 1), "GB/s_1p6bit_bytes": round(b3b / t3 / 1e3, 1),
            "per_shape": per}


def bench_gemm(bw, workloads, torch, dev, layer, reps, probe=False):
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
    ops = sum(2.0 * M * N * K for _, N, K in layer)

    # projections that read the same activations share one quantization (q|k|v, gate|up)
    index = {name: i for i, (name, _, _) in enumerate(layer)}
    groups = [[index[n] for n in grp] for grp in workloads.DECODE_GROUPS]

    def grouped(c, grp):
        """One grouped launch of grp on weight list c (by layer index)."""
        i0 = grp[0]
        return bw.gemm_grouped(xqs[i0], avs[i0], [c[i] for i in grp],
                               [scales[i] for i in grp], "bf16", out=[outs[i] for i in grp])

    def group_copies(grp):
        cp = rotation([packed0[i] for i in grp], sum(layer[i][1] * layer[i][2] // 4 for i in grp))
        return [dict(zip(grp, c)) for c in cp]

    if probe:
        # counter collection: the calibration copies, then the four grouped GEMM launches
        # once per weight copy of the whole set (weights from HBM), eagerly
        copies = rotation(packed0, set_bytes)
        calibration_copies(torch, dev)
        for c in copies:
            for grp in groups:
                grouped(c, grp)
        torch.cuda.synchronize()
        print(f"[bench] gemm probe: {len(copies)} prefill steps", file=sys.stderr)
        return None

    copies = rotation(packed0, set_bytes)

    def step(r):
        for grp in groups:
            i0 = grp[0]
            bw.quant_act(xs[i0], xq=xqs[i0], a_scale=avs[i0])
            grouped(copies[r], grp)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_step = run_steps(torch, step, len(copies), 3, 40)
    del copies
    torch.cuda.empty_cache()

    per_group_us = []
    for grp in groups:
        cp = group_copies(grp)
        per_group_us.append(graph_launch_us(torch, lambda r, grp=grp: grouped(cp[r], grp),
                                            len(cp), reps))
        del cp
    per_shape_us = []
    for i in range(len(layer)):
        cp = group_copies([i])
        per_shape_us.append(graph_launch_us(torch, lambda r, i=i: bw.gemm(
            xqs[i], avs[i], cp[r][i], scales[i], "bf16", out=outs[i]), len(cp), reps))
        del cp
    torch.cuda.empty_cache()
    quant_us = {"|".join(g): round(graph_launch_us(
        torch, lambda r, i0=index[g[0]]: bw.quant_act(xs[i0], xq=xqs[i0], a_scale=avs[i0]),
        QUANT_LAUNCHES,
        reps), 3) for g in workloads.DECODE_GROUPS}
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
    alg_bytes = sum(N * K // 4 + 4 * N + 2 * M * N for _, N, K in layer) + sum(
        M * layer[g[0]][2] + 4 * M for g in groups)
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
        "quant_act_us": quant_us,
        "value_ungrouped": round(ops / (sum(per_shape_us) * 1e-6) / 1e12, 2),
        "vendor_int8_gemm_same_products_tops": (None if vendor_us is None else
                                                round(ops / (vendor_us * 1e-6) / 1e12, 2)),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tops, 2),
            "peak": INT8_MFMA_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4),
            "attainable_TOPS": round(min(INT8_MFMA_PEAK_TOPS,
                                         ops / alg_bytes * HBM_PEAK_GBS / 1e3), 1),
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
