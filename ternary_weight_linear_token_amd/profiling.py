"""Short text summaries of rocprofv3 runs, as kept next to the measured numbers.

Kernel durations (a `rocprofv3 --kernel-trace --stats --output-format csv` run):

    python -m ternary_weight_linear_token_amd.profiling kernels --dir DIR --out FILE --cmd "..."

HBM traffic of the decode kernel (two `rocprofv3 --pmc` runs of `bench.py --traffic-probe`,
one with FETCH_SIZE and one with WRITE_SIZE):

    python -m ternary_weight_linear_token_amd.profiling traffic --fetch DIR1 --write DIR2 \
        --out FILE --cmd "..."

Matrix-core use and HBM traffic of the prefill GEMM (three `rocprofv3 --pmc` runs of
`bench.py --gemm-probe`: SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU
SQ_INSTS_MFMA GRBM_GUI_ACTIVE, then FETCH_SIZE, then WRITE_SIZE):

    python -m ternary_weight_linear_token_amd.profiling gemm --util DIR0 --fetch DIR1 \
        --write DIR2 --out FILE --cmd "..."

FETCH_SIZE and WRITE_SIZE read in KiB per dispatch.  They are scaled by what the same
counters read for a plain elementwise kernel of known size that the probe runs first (it
reads and writes COPY_BYTES each), so the reported bytes are in the units of that copy.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os
import statistics
import sys

COPY_BYTES = 512 << 20    # bytes read (and written) by each calibration launch of the probe
COPY_KERNEL = "elementwise"  # torch's elementwise kernel family (torch.neg on int32)
COPY_TAG = "neg"


def _short(name: str) -> str:
    n = name.replace("bitnet::(anonymous namespace)::", "").replace("bitnet::", "")
    n = n.replace("void ", "")
    return n.split("(")[0] if "(" in n else n


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernels(d: str, out: str, cmd: str) -> str:
    trace = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    stats = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    lines = ["# rocprofv3 kernel summary", f"# command: {cmd}", "",
             "## --stats (every dispatch of the run)",
             f"{'kernel':72s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for r in stats:
        lines.append(f"{_short(r['Name'])[:72]:72s} {r['Calls']:>6s} "
                     f"{float(r['AverageNs']) / 1e3:9.3f} {float(r['MinNs']) / 1e3:9.3f} "
                     f"{float(r['MaxNs']) / 1e3:9.3f}")
    lines += ["", "## library kernels per launch shape (kernel trace; grid in work-items)",
              f"{'kernel':60s} {'grid':>8s} {'lds':>6s} {'n':>5s} {'mean_us':>9s} {'median_us':>9s}"]
    agg = collections.defaultdict(list)
    for r in trace:
        if "bitnet" not in r["Kernel_Name"]:
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["LDS_Block_Size"]))
        agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, ds in sorted(agg.items()):
        lines.append(f"{k[0][:60]:60s} {k[1]:8d} {k[2]:6d} {len(ds):5d} "
                     f"{statistics.mean(ds):9.3f} {statistics.median(ds):9.3f}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _counter_rows(d: str, counter: str):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                rows.append(r)
    if not rows:
        raise FileNotFoundError(f"no {counter} rows under {d}")
    return rows


def _per_dispatch(rows):
    """{dispatch id: (kernel name, grid, value summed over the counter's instances)}"""
    acc = {}
    for r in rows:
        key = r["Dispatch_Id"]
        name, grid, val = r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])
        if key in acc:
            acc[key] = (name, grid, acc[key][2] + val)
        else:
            acc[key] = (name, grid, val)
    return acc


def traffic(fetch_dir: str, write_dir: str, out: str, cmd: str, source_hash: str,
            algorithmic_bytes: float) -> str:
    fetch = _per_dispatch(_counter_rows(fetch_dir, "FETCH_SIZE"))
    write = _per_dispatch(_counter_rows(write_dir, "WRITE_SIZE"))

    def calib(table):
        vals = [v for n, g, v in table.values()
                if COPY_KERNEL in n and COPY_TAG in n and "bitnet" not in n]
        if not vals:
            raise RuntimeError("the calibration copy was not found in the counter output")
        vals = vals[1:] if len(vals) > 1 else vals  # the first launch warms up
        return COPY_BYTES / (statistics.median(vals) * 1024.0), len(vals)

    f_fetch, n_cf = calib(fetch)
    f_write, n_cw = calib(write)

    def gemv(table):
        by = collections.defaultdict(list)
        for n, g, v in table.values():
            if "skinny_kernel" in n:
                by[(_short(n), g)].append(v * 1024.0)
        return by

    fb, wb = gemv(fetch), gemv(write)
    lines = ["# HBM traffic of the fused quant+GEMV kernel, BitNet-2B decode set at M = 1",
             f"# command: {cmd}",
             f"# calibration: {COPY_BYTES} B read and written per copy launch; FETCH_SIZE reads "
             f"{1 / f_fetch:.4f}x, WRITE_SIZE {1 / f_write:.4f}x of that ({n_cf}, {n_cw} launches)",
             "# per shape: kernel, grid (work-items), launches, HBM read bytes, HBM write bytes "
             "per launch (calibrated)"]
    total_r, total_w, n_all = 0.0, 0.0, 0
    for key in sorted(fb):
        r = statistics.mean(fb[key]) * f_fetch
        w = statistics.mean(wb.get(key, [0.0])) * f_write
        cnt = len(fb[key])
        lines.append(f"#   {key[0][:60]:60s} {key[1]:8d} {cnt:5d} {r:12.0f} {w:10.0f}")
        total_r += r * cnt
        total_w += w * cnt
        n_all += cnt
    per_launch = (total_r + total_w) / n_all
    lines += [f"kernel_source_sha256 = {source_hash}",
              f"fetch_calibration = {f_fetch:.6f}",
              f"write_calibration = {f_write:.6f}",
              f"hbm_read_bytes_per_launch = {total_r / n_all:.0f}",
              f"hbm_write_bytes_per_launch = {total_w / n_all:.0f}",
              f"hbm_bytes_per_launch = {per_launch:.0f}",
              f"algorithmic_bytes_per_launch = {algorithmic_bytes:.0f}",
              f"traffic_over_algorithmic = {per_launch / algorithmic_bytes:.4f}"]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs
XCDS = 8         # GRBM_GUI_ACTIVE is counted per XCD; the summary sums the eight


def gemm(util_dir: str, fetch_dir: str, write_dir: str, out: str, cmd: str, source_hash: str,
         launches) -> str:
    """Matrix-core use and HBM traffic of the tiled GEMM launches of `bench.py --gemm-probe`.

    launches: [(name, M, N, K)] of one prefill step, in launch order.  Per launch shape
    (grid): int8 operations counted by the matrix cores (SQ_INSTS_VALU_MFMA_MOPS_I8 x 512)
    against 2 M N K, matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs
    / (GRBM_GUI_ACTIVE per XCD x SIMDs); the dispatch's active cycles include what the
    counter collection adds around it, so this reads low against the unprofiled rate),
    VALU instructions per matrix product, and calibrated HBM bytes."""
    mops = _per_dispatch(_counter_rows(util_dir, "SQ_INSTS_VALU_MFMA_MOPS_I8"))
    busy = _per_dispatch(_counter_rows(util_dir, "SQ_VALU_MFMA_BUSY_CYCLES"))
    valu = _per_dispatch(_counter_rows(util_dir, "SQ_INSTS_VALU"))
    mfma = _per_dispatch(_counter_rows(util_dir, "SQ_INSTS_MFMA"))
    gui = _per_dispatch(_counter_rows(util_dir, "GRBM_GUI_ACTIVE"))
    fetch = _per_dispatch(_counter_rows(fetch_dir, "FETCH_SIZE"))
    write = _per_dispatch(_counter_rows(write_dir, "WRITE_SIZE"))

    def calib(table):
        vals = [v for n, g, v in table.values()
                if COPY_KERNEL in n and COPY_TAG in n and "bitnet" not in n]
        if not vals:
            raise RuntimeError("the calibration copy was not found in the counter output")
        vals = vals[1:] if len(vals) > 1 else vals
        return COPY_BYTES / (statistics.median(vals) * 1024.0)

    f_fetch, f_write = calib(fetch), calib(write)

    def tiled(table, scale=1.0):
        """dispatches of the tiled kernel in launch order: [(name, grid, value)]"""
        rows = [(int(k), n, g, v * scale) for k, (n, g, v) in table.items() if "tiled_kernel" in n]
        return [r[1:] for r in sorted(rows)]

    t_mops, t_busy, t_valu, t_mfma, t_gui = (tiled(mops), tiled(busy), tiled(valu), tiled(mfma),
                                             tiled(gui, 1.0 / XCDS))
    t_fetch, t_write = tiled(fetch, 1024.0 * f_fetch), tiled(write, 1024.0 * f_write)
    nl = len(launches)
    if len(t_mops) % nl or len(t_fetch) % nl or len(t_write) % nl:
        raise RuntimeError("the tiled dispatches are not whole prefill steps")
    lines = ["# Matrix-core use and HBM traffic of the tiled GEMM, BitNet-2B prefill set at "
             "M = 512 (four grouped launches)",
             f"# command: {cmd}",
             f"# calibration: FETCH_SIZE reads {1 / f_fetch:.4f}x, WRITE_SIZE "
             f"{1 / f_write:.4f}x of a {COPY_BYTES}-byte copy",
             "# per launch: kernel, steps, int8 ops counted / 2MNK, matrix-core busy, VALU per "
             "product, HBM read MB, HBM write MB, algorithmic MB (packed weights + int8 "
             "activations + bf16 out)"]
    tot_busy_w, tot_gui, tot_bytes, tot_alg = 0.0, 0.0, 0.0, 0.0
    for i, (name, M, N, K) in enumerate(launches):
        sel = lambda t: [v for j, (_, _, v) in enumerate(t) if j % nl == i]
        kern = _short(t_mops[i][0])
        ops = statistics.mean(sel(t_mops)) * 512
        b = statistics.mean(sel(t_busy))
        gcy = statistics.mean(sel(t_gui))
        vpm = statistics.mean(sel(t_valu)) / max(1.0, statistics.mean(sel(t_mfma)))
        rd, wr = statistics.mean(sel(t_fetch)), statistics.mean(sel(t_write))
        alg = N * K / 4 + M * K + 2 * M * N
        lines.append(f"#   {name:8s} {kern[:44]:44s} {len(sel(t_mops)):3d} "
                     f"{ops / (2.0 * M * N * K):6.3f} {b / (gcy * SIMDS):6.3f} {vpm:6.2f} "
                     f"{rd / 1e6:8.2f} {wr / 1e6:7.2f} {alg / 1e6:7.2f}")
        tot_busy_w += b
        tot_gui += gcy
        tot_bytes += rd + wr
        tot_alg += alg
    lines += [f"kernel_source_sha256 = {source_hash}",
              f"mfma_busy_frac_weighted = {tot_busy_w / (tot_gui * SIMDS):.4f}",
              f"hbm_bytes_per_launch = {tot_bytes / nl:.0f}",
              f"algorithmic_bytes_per_launch = {tot_alg / nl:.0f}",
              f"traffic_over_algorithmic = {tot_bytes / tot_alg:.4f}"]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _durations(d: str):
    """{dispatch id: duration in ns} from the kernel traces under d (runs with --kernel-trace)."""
    out = {}
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        for r in csv.DictReader(open(path)):
            out[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def large(util_dir: str, fetch_dir: str, write_dir: str, out: str, cmd: str, hashes: dict,
          launches) -> str:
    """Counters of `bench.py --large-probe`: per launch configuration (kernel, grid) in
    dispatch order -- `launches` gives their names and algorithmic bytes and operations --
    the mean duration under counter collection, the core clock (GRBM_GUI_ACTIVE per XCD /
    duration, for dispatches of 50 us or more), matrix-core busy fraction, VALU per matrix product and calibrated HBM
    bytes against the algorithmic ones."""
    util = {c: _per_dispatch(_counter_rows(util_dir, c)) for c in
            ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")}
    fetch = _per_dispatch(_counter_rows(fetch_dir, "FETCH_SIZE"))
    write = _per_dispatch(_counter_rows(write_dir, "WRITE_SIZE"))
    dur = _durations(util_dir)

    def calib(table):
        vals = [v for n, g, v in table.values()
                if COPY_KERNEL in n and COPY_TAG in n and "bitnet" not in n]
        if not vals:
            raise RuntimeError("the calibration copy was not found in the counter output")
        vals = vals[1:] if len(vals) > 1 else vals
        return COPY_BYTES / (statistics.median(vals) * 1024.0)

    f_fetch, f_write = calib(fetch), calib(write)

    def groups(table):
        """[(kernel, grid, [dispatch ids])] of library product kernels: runs of consecutive
        dispatches with the same kernel and grid, in dispatch order (the probe runs each
        launch configuration over all its weight copies before the next)"""
        runs = []
        for k in sorted(table, key=int):
            n, g, _ = table[k]
            if "skinny_kernel" not in n and "tiled_kernel" not in n:
                continue
            key = (_short(n), g)
            if not runs or runs[-1][0] != key:
                runs.append((key, []))
            runs[-1][1].append(k)
        return [(key[0], key[1], ids) for key, ids in runs]

    gu, gf, gw = groups(util["SQ_INSTS_MFMA"]), groups(fetch), groups(write)
    if not (len(gu) == len(gf) == len(gw) == len(launches)):
        raise RuntimeError(f"expected {len(launches)} launch configurations, found "
                           f"{len(gu)} / {len(gf)} / {len(gw)}")
    lines = ["# Counters of the large-shape launches: 70B decode set at M = 1, 8B and 70B "
             "prefill GEMMs",
             f"# command: {cmd}",
             f"# calibration: FETCH_SIZE reads {1 / f_fetch:.4f}x, WRITE_SIZE "
             f"{1 / f_write:.4f}x of a {COPY_BYTES}-byte copy",
             "# per launch: name, kernel, launches, mean us (under counters), core GHz, "
             "matrix-core busy, VALU per product, HBM read MB, write MB, algorithmic MB, "
             "traffic / algorithmic"]
    for (name, alg_bytes), (kern, grid, ids), (_, _, fid), (_, _, wid) in zip(launches, gu, gf, gw):
        mean = lambda tbl, ks: statistics.mean(tbl[k][2] for k in ks)
        us = statistics.mean(dur[k] for k in ids if k in dur) / 1e3 if dur else float("nan")
        gui = mean(util["GRBM_GUI_ACTIVE"], ids) / XCDS
        # short dispatches: the busy window counted around them exceeds their duration,
        # so the clock is read on long ones only
        ghz = gui / (us * 1e3) if us == us and us >= 50.0 else float("nan")
        busy = mean(util["SQ_VALU_MFMA_BUSY_CYCLES"], ids) / (gui * SIMDS)
        vpm = mean(util["SQ_INSTS_VALU"], ids) / max(1.0, mean(util["SQ_INSTS_MFMA"], ids))
        rd = mean(fetch, fid) * 1024.0 * f_fetch
        wr = mean(write, wid) * 1024.0 * f_write
        lines.append(f"#   {name:18s} {kern[:44]:44s} {len(ids):4d} {us:9.2f} {ghz:6.3f} {busy:6.3f} "
                     f"{vpm:6.2f} {rd / 1e6:9.2f} {wr / 1e6:8.2f} {alg_bytes / 1e6:9.2f} "
                     f"{(rd + wr) / alg_bytes:6.3f}")
        lines.append(f"{name}.traffic_over_algorithmic = {(rd + wr) / alg_bytes:.4f}")
        lines.append(f"{name}.mfma_busy_frac = {busy:.4f}")
        if ghz == ghz:
            lines.append(f"{name}.core_clock_ghz = {ghz:.4f}")
    for k, v in hashes.items():
        lines.append(f"{k} = {v}")
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m ternary_weight_linear_token_amd.profiling")
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--dir", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    gm = sub.add_parser("gemm")
    gm.add_argument("--util", required=True)
    gm.add_argument("--fetch", required=True)
    gm.add_argument("--write", required=True)
    gm.add_argument("--out", required=True)
    gm.add_argument("--cmd", required=True)
    lg = sub.add_parser("large")
    lg.add_argument("--util", required=True)
    lg.add_argument("--fetch", required=True)
    lg.add_argument("--write", required=True)
    lg.add_argument("--out", required=True)
    lg.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "kernels":
        sys.stdout.write(kernels(a.dir, a.out, a.cmd))
    elif a.what == "large":
        from . import build
        sys.path.insert(0, build.ROOT)
        import workloads
        import bench
        shapes = {name: (N, K) for name, N, K in workloads.LAYER_70B}
        launches = [("70b_m1_" + "_".join(g), sum(shapes[n][0] * shapes[n][1] // 4 for n in g))
                    for g in workloads.DECODE_GROUPS]
        launches += [(name, sum(N * K / 4 + 2 * M * N for N in Ns) + M * K)
                     for name, M, Ns, K in bench.LARGE_PROBE_GEMM]
        hashes = {"skinny_source_sha256": build.kernel_hash("skinny.hip"),
                  "tiled_source_sha256": build.kernel_hash("tiled.hip")}
        sys.stdout.write(large(a.util, a.fetch, a.write, a.out, a.cmd, hashes, launches))
    elif a.what == "gemm":
        from . import build
        sys.path.insert(0, build.ROOT)
        import workloads
        shapes = {name: (N, K) for name, N, K in workloads.LAYER_2B}
        launches = [("|".join(g), 512, sum(shapes[n][0] for n in g), shapes[g[0]][1])
                    for g in workloads.DECODE_GROUPS]
        sys.stdout.write(gemm(a.util, a.fetch, a.write, a.out, a.cmd,
                              build.kernel_hash("tiled.hip"), launches))
    else:
        from . import build
        sys.path.insert(0, build.ROOT)
        import workloads
        layer = workloads.LAYER_2B
        # one decode step's packed bytes over its launches (grouped projections)
        alg = sum(N * K // 4 for _, N, K in layer) / len(workloads.DECODE_GROUPS)
        sys.stdout.write(traffic(a.fetch, a.write, a.out, a.cmd, build.kernel_hash("skinny.hip"), alg))


if __name__ == "__main__":
    main()
