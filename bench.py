"""Benchmark of the mixed-adapter LoRA layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stress_70b]
    python bench.py --trace-summary DIR     (summarise a rocprofv3 kernel trace)

The default workload is the largest one that fits one GPU: the 70B-shaped
layer set with heterogeneous ranks (4608 rows: 512 decode tokens and two
prefill chunks of 2048; q, o, gate, up, down; 256 adapter slots of ranks
8-64 padded to 64).

One step = one pass of the whole layer over one batch: every projection of
the workload through lora_linear_forward (segments built once per batch and
reused across projections in SGMV mode).  The timed region holds exactly K
steps (and is preceded by exactly W warm-up steps), bracketed by device
synchronisations; inputs are resident in HBM.  Workloads whose working set
fits in the 256 MB Infinity Cache rotate through several copies of
(x, W, pool, y) so every step reads HBM.

Prints ONE JSON line: tokens/s of the whole step, plus
  roofline:     the dominant kernel's algorithmic flops (or bytes) per launch
                over its average duration, measured with HIP events on the
                stream it runs on, against the MI355X peak;
  cpu_baseline: the fp64 CPU oracle on a bounded row sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("mixed-adapter LoRA-layer tokens/s; shrink/expand HBM GB/s and base-GEMM MFMA % of peak")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 MFMA
MFMA_FP8_PEAK_TFS = 5000.0     # dense fp8 MFMA
FP32_VALU_PEAK_TFS = 157.3     # fp32 vector
RIDGE = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
RIDGE_FP8 = MFMA_FP8_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
MALL_BYTES = 256 * 2 ** 20
CSRC = os.path.join(ROOT, "rank_adapter_gemm_amd", "csrc")
KERNEL_SOURCE = {"gemm_expand": ["gemm.hip", "gemm_common.hpp", "expand.hip"], "gemm": ["gemm.hip", "gemm_common.hpp"],
                 "shrink": ["shrink.hip", "fp8_common.hpp"],
                 "segments": ["segments.hip"], "expand": ["expand.hip"],
                 "forward": ["api.hip", "gemm.hip", "gemm_common.hpp", "shrink.hip", "fp8_common.hpp",
                             "segments.hip", "expand.hip"],
                 "forward_fp8": ["api.hip", "gemm_fp8.hip", "gemm_common.hpp", "fp8_common.hpp", "shrink.hip",
                                 "segments.hip", "expand.hip"]}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="stress_70b")
    ap.add_argument("--mode", default="auto", choices=["auto", "bgmv", "sgmv"])
    ap.add_argument("--separate-expand", action="store_true")
    ap.add_argument("--no-slices", action="store_true",
                    help="one lora_linear_forward per projection, also where projections share x")
    ap.add_argument("--cold-sets", type=int, default=None, help="copies of the working set to rotate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU work of the oracle sample")
    ap.add_argument("--residency", action="store_true",
                    help="also measure the adapter cache's host-to-HBM promotion rate")
    ap.add_argument("--fp8-base", action="store_true",
                    help="E4M3 base weights (lora_linear_forward_fp8); reported apart from the bf16 headline")
    ap.add_argument("--single-adapter", action="store_true",
                    help="context run: every row that has an adapter uses the batch's most frequent one")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain fp32 copy kernel of known size (for counter scaling)")
    ap.add_argument("--packed-pool", action="store_true",
                    help="packed adapter pools (each slot its adapter's rank rows, no padding to max_rank)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-entry-point timings (short profiling runs); the roofline "
                         "kernel and the forward calls are still timed")
    ap.add_argument("--counter-summary", default=None, metavar="DIR",
                    help="print per-kernel means of a rocprofv3 --pmc csv output directory and exit")
    ap.add_argument("--record-traffic", nargs=6, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "KEY", "KERNEL_SUBSTRING", "GRID", "SOURCE"),
                    help="store one kernel's HBM bytes per launch (counter runs with --calib-copy) in "
                         "profiles/traffic.json and exit")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="print a per-kernel, per-grid summary of a rocprofv3 --kernel-trace output "
                         "directory and exit (no GPU use)")
    return ap.parse_args()


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCE[kernel] + ["common.hpp"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def trace_summary(path: str) -> None:
    """Per-kernel, per-grid summary of a rocprofv3 --kernel-trace run: the
    kernel_stats file groups launches by name only, which mixes the shapes of
    one template; this groups them by (name, grid size) as well."""
    import csv
    import glob
    import statistics

    import sqlite3

    files = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    dbs = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
    if not files and not dbs:
        print("no *kernel_trace.csv or *_results.db under %s" % path, file=sys.stderr)
        sys.exit(1)
    groups = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name", "?")
                grid = row.get("Grid_Size_X") or row.get("Grid_Size") or "?"
                if row.get("Grid_Size_Y") not in (None, "", "1"):
                    grid = "%sx%s" % (grid, row["Grid_Size_Y"])
                wg = row.get("Workgroup_Size_X") or row.get("Workgroup_Size") or "?"
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                groups.setdefault((name, grid, wg), []).append(dur)
    for f in dbs:                      # rocpd output (the default format of rocprofv3)
        con = sqlite3.connect(f)
        for name, grid, gy, wg, start, end in con.execute(
                "select name, grid_x, grid_y, workgroup_x, start, end from kernels"):
            g = str(grid) if gy in (None, 1) else "%sx%s" % (grid, gy)
            groups.setdefault((name, g, str(wg)), []).append((end - start) / 1e3)
        con.close()
    print("| calls | avg us | min us | max us | total us | grid (threads) | wg | kernel |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) <= 110 else name[:107] + "..."
        print("| %d | %.3f | %.3f | %.3f | %.1f | %s | %s | `%s` |" % (
            len(d), statistics.fmean(d), min(d), max(d), sum(d), grid, wg, short))


def _counter_rows(path: str):
    """(kernel name, grid size, counter, value, duration us) of every dispatch
    in a rocprofv3 --pmc --output-format csv directory."""
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        print("no *counter_collection.csv under %s" % path, file=sys.stderr)
        sys.exit(1)
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                yield (row["Kernel_Name"], row["Grid_Size"], row["Counter_Name"], float(row["Counter_Value"]),
                       (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)


def counter_summary(path: str) -> None:
    """Per-kernel, per-grid means of each counter of a rocprofv3 --pmc run
    (kernels of this library, and the calibration copy)."""
    import statistics

    groups = {}
    for name, grid, ctr, val, dur in _counter_rows(path):
        if "lora::" not in name and "AUnaryFunctor" not in name:
            continue
        if any(k in name for k in ("k_upload", "k_fill", "k_set_meta", "k_ws_init")):
            continue
        groups.setdefault((name, grid, ctr), []).append((val, dur))
    print("| calls | mean value | mean us | counter | grid | kernel |")
    print("|---|---|---|---|---|---|")
    for (name, grid, ctr), v in sorted(groups.items(), key=lambda kv: (kv[0][2], -statistics.fmean(x[1] for x in kv[1]))):
        short = name if len(name) <= 100 else name[:97] + "..."
        print("| %d | %.1f | %.1f | %s | %s | `%s` |" % (len(v), statistics.fmean(x[0] for x in v),
                                                       statistics.fmean(x[1] for x in v), ctr, grid, short))


def record_traffic(fetch_dir: str, write_dir: str, key: str, kernel_sub: str, grid: str, source: str) -> None:
    """HBM bytes per launch of a launch group (kernels matched by name
    substrings and grid sizes in threads, '+'-separated lists of equal
    length; one launch of each per unit) from a FETCH_SIZE run and a
    WRITE_SIZE run, each scaled by what the same counter reads for the 1 GiB
    calibration copy of --calib-copy, stored in profiles/traffic.json under
    `key` with the hash of the kernels' source files (KERNEL_SOURCE[source])."""
    import statistics

    subs, grids = kernel_sub.split("+"), grid.split("+")
    if len(subs) != len(grids):
        print("--record-traffic: as many grids as kernel substrings", file=sys.stderr)
        sys.exit(2)

    def mean_of(path, ctr):
        vals = [[] for _ in subs]
        calib = []
        for name, g, c, val, dur in _counter_rows(path):
            if c != ctr:
                continue
            if "AUnaryFunctor" in name and g == "67108864":
                calib.append(val)
            for i, (sub, gr) in enumerate(zip(subs, grids)):
                if sub in name and g == gr:
                    vals[i].append(val)
        if not all(vals) or not calib:
            print("%s: no matching dispatches (kernels %s, calibration %d)" % (
                path, [len(v) for v in vals], len(calib)), file=sys.stderr)
            sys.exit(1)
        # the calibration copy moves 1 GiB each way; the counter reads KiB
        factor = (1 << 30) / (statistics.fmean(calib) * 1024)
        return sum(statistics.fmean(v) for v in vals) * 1024 * factor, factor

    fetch, ff = mean_of(fetch_dir, "FETCH_SIZE")
    write, wf = mean_of(write_dir, "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = {"hbm_bytes_per_launch": int(round(fetch + write)), "fetch_bytes": int(round(fetch)),
                 "write_bytes": int(round(write)), "fetch_factor": round(ff, 3), "write_factor": round(wf, 3),
                 "kernel": kernel_sub, "grid": grid, "source_sha": source_sha(source)}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({key: data[key]}))


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single "
              "MI355X (rows are independent; see the sharding notes in the design document). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rank_adapter_gemm_amd import lora as L
    from rank_adapter_gemm_amd.workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.load()
    dev = "cuda"
    wl = make_workload(args.workload, device=dev)
    mode = {"auto": L.LORA_MODE_AUTO, "bgmv": L.LORA_MODE_BGMV, "sgmv": L.LORA_MODE_SGMV}[args.mode]
    sgmv = mode == L.LORA_MODE_SGMV or (mode == L.LORA_MODE_AUTO and wl.T >= L.LORA_AUTO_SGMV_MIN_ROWS)
    eb = 4 if wl.dtype == torch.float32 else 2
    T, R = wl.T, wl.max_rank
    if args.single_adapter:
        # same rows, same base-only rows; one adapter (the batch's most used) for the rest
        live = (wl.ids >= 0) & (wl.ids < wl.n_slots)
        if live.any():
            top = int(np.bincount(wl.ids[live]).argmax())
            wl.ids = np.where(live, top, wl.ids).astype(np.int32)
    ids = torch.as_tensor(wl.ids, device=dev)

    # ---- pools (one per projection) ----
    pools = []
    # packed pools: each slot holds its adapter's rank rows, rounded up to 8
    capacity = ([max(8, (int(r) + 7) // 8 * 8) for r in wl.ranks] if args.packed_pool else None)
    for pr in wl.projections:
        pool = L.AdapterPool(wl.n_slots, pr.d_in, pr.d_out, R, wl.dtype, device=dev, capacity=capacity)
        for s in range(wl.n_slots):
            r = int(wl.ranks[s])
            if r > 0:
                pool.upload(s, pr.A[s], pr.B[s], r, float(wl.alphas[s]), lda=R, ldb=pr.d_out)
        pools.append(pool)
    torch.cuda.synchronize()
    for pr in wl.projections:          # the host-side sources are no longer needed
        pr.A = pr.B = None

    # ---- working-set copies for cache-cold timing ----
    fp8 = args.fp8_base
    if fp8 and wl.dtype != torch.bfloat16:
        print("--fp8-base takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    wb = 1 if fp8 else eb                        # bytes per base weight read by the step
    set_bytes = sum(p.W.numel() * wb + pl.nbytes + T * p.d_out * eb for p, pl in zip(wl.projections, pools))
    set_bytes += sum(x.numel() * eb for x in wl.xs.values())
    n_sets = args.cold_sets
    if n_sets is None:
        n_sets = 1 if set_bytes >= 2 * MALL_BYTES else min(16, math.ceil(2 * MALL_BYTES / set_bytes))
    sets = []
    for k in range(n_sets):
        if k == 0:
            xs = wl.xs
            Ws = [p.W for p in wl.projections]
            ps = [pl.pool for pl in pools]
            keep = []
        else:
            xs = {g: x.clone() for g, x in wl.xs.items()}
            Ws = [p.W.clone() for p in wl.projections]
            ps, keep = [], []
            for pl in pools:
                a, b, sc, rk = pl.a.clone(), pl.b.clone(), pl.scale.clone(), pl.rank.clone()
                r0 = pl.row0.clone() if pl.row0 is not None else None
                keep += [a, b, sc, rk, r0]
                q = L.lora_pool_t(pl.pool.n_slots, pl.pool.d_in, pl.pool.d_out, pl.pool.max_rank,
                                  pl.pool.dtype, a.data_ptr(), b.data_ptr(), sc.data_ptr(), rk.data_ptr(),
                                  r0.data_ptr() if r0 is not None else None, pl.pool.row0_host)
                ps.append(q)
        ys = [torch.empty(T, p.d_out, dtype=wl.dtype, device=dev) for p in wl.projections]
        W8 = [L.Fp8Weight(W) for W in Ws] if fp8 else None
        sets.append(dict(xs=xs, Ws=Ws, pools=ps, ys=ys, keep=keep, W8=W8))
    # Projections that share an input (consecutive, same x) run as slices of
    # one lora_linear_forward_sliced call: one shrink, one read of x.
    groups = []
    for k, pr in enumerate(wl.projections):
        if (not args.no_slices and not fp8 and groups and wl.projections[groups[-1][0]].x_group == pr.x_group
                and len(groups[-1]) < 4 and (len(groups[-1]) + 1) * R <= 128):
            groups[-1].append(k)
        else:
            groups.append([k])
    # d_out: the widest call (a sliced call plans its GEMM over all its slices)
    ws = L.Workspace(T, wl.n_slots, R, max(sum(wl.projections[k].d_out for k in g) for g in groups), device=dev,
                     n_slices=max(len(g) for g in groups),
                     fp8_d_in=max(p.d_in for p in wl.projections) if fp8 else 0)
    v = torch.empty(T, R, dtype=torch.float32, device=dev)
    # lora_gemm takes its split-K scratch from the start of the buffer it is
    # given; a buffer of its own keeps the segments in ws intact
    gemm_ws = torch.empty(128 << 20, dtype=torch.uint8, device=dev)
    if fp8:
        xq8 = torch.empty(T, max(p.d_in for p in wl.projections), dtype=torch.uint8, device=dev)
        xs8 = torch.empty(T, dtype=torch.float32, device=dev)
    flags0 = L.LORA_FLAG_SEPARATE_EXPAND if args.separate_expand else 0
    torch.cuda.synchronize()

    def forward_group(gi, i):
        s_ = sets[i % n_sets]
        grp = groups[gi]
        fl = flags0 | (L.LORA_FLAG_SEGMENTS_READY if (sgmv and gi > 0) else 0)
        x = s_["xs"][wl.projections[grp[0]].x_group]
        if fp8:
            k = grp[0]
            L.lora_linear_forward_fp8(x, s_["W8"][k].codes, s_["W8"][k].scale, s_["ys"][k], T, s_["pools"][k],
                                      ids, mode, fl, ws.buf)
        elif len(grp) == 1:
            k = grp[0]
            L.lora_linear_forward(x, s_["Ws"][k], s_["ys"][k], T, s_["pools"][k], ids, mode, fl, ws.buf)
        else:
            L.lora_linear_forward_sliced(x, [s_["Ws"][k] for k in grp], [s_["ys"][k] for k in grp], T,
                                         [s_["pools"][k] for k in grp], ids, mode, fl, ws.buf)

    def step(i):
        for gi in range(len(groups)):
            forward_group(gi, i)

    # The step is captured into HIP graphs so host-side launch overhead is not
    # part of the timing: one graph per working-set copy (one step each), and
    # for rotated sets one graph that replays every copy once.  Step i runs
    # on copy i % n_sets; exactly the requested number of steps is run.
    step(0)
    torch.cuda.synchronize()
    g_one = []
    for j in range(n_sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(j)
        g_one.append(g)
    g_all = None
    if n_sets > 1:
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for j in range(n_sets):
                step(j)
    torch.cuda.synchronize()

    def run_steps(n, i0=0):
        i = i0
        while n > 0:
            if g_all is not None and i % n_sets == 0 and n >= n_sets:
                g_all.replay()
                i += n_sets
                n -= n_sets
            else:
                g_one[i % n_sets].replay()
                i += 1
                n -= 1
        return i

    if args.steps is None:
        # default counts: at least 50 timed steps and 100 ms, 10 warm-up steps
        t0 = time.perf_counter()
        run_steps(max(n_sets, 2))
        torch.cuda.synchronize()
        est = max((time.perf_counter() - t0) / max(n_sets, 2), 1e-6)
    steps = args.steps if args.steps is not None else int(min(20000, max(50, math.ceil(0.1 / est))))
    warmup = args.warmup if args.warmup is not None else 10
    if steps < 1 or warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    i_next = run_steps(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(steps, i_next)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps
    value = T * steps / elapsed
    est = max(elapsed / steps, 1e-6)
    assert L.lora_get_device_error(ws.buf) == -1

    # ---- per-kernel durations ----
    # Each entry point of the decomposed step (segments, shrink, GEMM with the
    # fused expand) is captured alone, REPS launches in a row over the rotated
    # working sets, and timed with HIP events around graph replays on the
    # current stream -- the stream the kernels run on.
    names = (["segments"] if sgmv else []) + ["shrink", "gemm_expand"]
    if args.separate_expand:
        names = (["segments"] if sgmv else []) + ["shrink", "gemm", "expand"]
    if fp8:
        names = (["segments"] if sgmv else []) + ["quantize", "shrink", "gemm_fp8"]
    # the base product alone (no adapters), for the LoRA overhead
    if "gemm" not in names and not fp8:
        names.append("gemm")
    if args.no_breakdown:             # only what the roofline needs
        names = ["gemm_fp8"] if fp8 else (["gemm"] if args.separate_expand else ["gemm_expand"])
    smode = L.LORA_MODE_SGMV if sgmv else L.LORA_MODE_BGMV

    def call(name, k, i):
        s_ = sets[i % n_sets]
        pr = wl.projections[k]
        x, W, y, pool = s_["xs"][pr.x_group], s_["Ws"][k], s_["ys"][k], s_["pools"][k]
        if name == "segments":
            L.lora_build_segments(ids, T, wl.n_slots, R, ws.buf)
        elif name == "shrink":
            L.lora_shrink(x, T, pool, ids, smode, v, ws.buf)
        elif name == "gemm":
            L.lora_gemm(x, W, y, T, pr.d_in, pr.d_out, L.dtype_code(wl.dtype), ws=gemm_ws)
        elif name == "expand":
            L.lora_expand(v, T, pool, ids, smode, y, ws.buf)
        elif name == "quantize":
            L.lora_quantize_rows_fp8(x, T, pr.d_in, xq8, xs8)
        elif name == "gemm_fp8":
            w8 = s_["W8"][k]
            L.lora_gemm_fp8(xq8, xs8, w8.codes, w8.scale, y, T, pr.d_in, pr.d_out, ws.buf)
        else:
            L.lora_gemm_expand(x, W, y, T, pool, ids, v, smode, ws.buf)

    def forward_segments():
        # the segments (and GEMM row order) the step's forward builds
        if sgmv:
            forward_group(0, 0)

    forward_segments()
    per_launch = {}          # (name, proj) -> average ms per launch
    reps = n_sets if args.no_breakdown else max(n_sets, 8)
    for name in names:
        projs = [0] if name == "segments" else range(len(wl.projections))
        for k in projs:
            for i in range(2):
                call(name, k, i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    call(name, k, i)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            n_rep = 2 if args.no_breakdown else max(3, int(0.2 / max(est, 1e-6) / reps))
            e0.record()
            for _ in range(n_rep):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            per_launch[(name, k)] = e0.elapsed_time(e1) / (n_rep * reps)
            del g
        if name == "segments":          # the public builder groups every segment
            forward_segments()

    # The step itself calls lora_linear_forward once per projection; time each
    # of those calls alone the same way (segments already built for k > 0).
    fwd = {}
    for gi in range(len(groups)):
        for i in range(2):
            forward_group(gi, i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                forward_group(gi, i)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        n_rep = 2 if args.no_breakdown else max(3, int(0.2 / max(est, 1e-6) / reps))
        e0.record()
        for _ in range(n_rep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        fwd[gi] = e0.elapsed_time(e1) / (n_rep * reps)
        del g

    # ---- algorithmic bytes / flops per launch ----
    ids_np = wl.ids
    used = np.unique(ids_np[(ids_np >= 0) & (ids_np < wl.n_slots)])
    sum_r = int(sum(int(wl.ranks[a]) for a in used))
    t_a = int(((ids_np >= 0) & (ids_np < wl.n_slots)).sum())
    r_row = np.where((ids_np >= 0) & (ids_np < wl.n_slots), wl.ranks[np.clip(ids_np, 0, None)], 0)
    sum_row_r = int(r_row.sum())

    def work(name, pr):
        d_in, d_out = pr.d_in, pr.d_out
        if name == "segments":
            return 3 * T * 4, 0
        if name == "shrink":
            return T * d_in * eb + sum_r * d_in * eb + T * R * 4, 2 * sum_row_r * d_in
        if name == "gemm":
            return (T * d_in + d_in * d_out + T * d_out) * eb, 2 * T * d_in * d_out
        if name == "expand":
            return T * R * 4 + sum_r * d_out * eb + 2 * T * d_out * eb, 2 * sum_row_r * d_out
        if name == "gemm_expand":
            by = (T * d_in + d_in * d_out + T * d_out) * eb + T * R * 4 + sum_r * d_out * eb
            return by, 2 * T * d_in * d_out + 2 * sum_row_r * d_out
        if name == "quantize":
            return T * d_in * eb + T * d_in + 4 * T, 0
        if name == "gemm_fp8":
            return T * d_in + 4 * T + d_in * d_out + 4 * d_out + T * d_out * eb, 2 * T * d_in * d_out
        raise KeyError(name)

    def fwd_work(gi):
        """One forward call of group gi: x read once (shrink and base
        products share it), each slice's W and y, the used adapters' A and B,
        segments for the first call of an SGMV step."""
        by = fl = 0
        for j, k in enumerate(groups[gi]):
            pr = wl.projections[k]
            b_g, f_g = work("gemm", pr)
            if fp8:                                      # codes and column scales instead of bf16 W
                b_g += pr.d_in * pr.d_out * (1 - eb) + 4 * pr.d_out
            b_s, f_s = work("shrink", pr)
            b_e, f_e = work("expand", pr)
            by += b_g + (b_s - T * pr.d_in * eb - T * R * 4) + (b_e - T * R * 4 - 2 * T * pr.d_out * eb)
            if j > 0:
                by -= T * pr.d_in * eb                   # x is shared by the slices
            fl += f_g + f_s + f_e
        if sgmv and gi == 0:
            by += work("segments", wl.projections[groups[0][0]])[0]
        return by, fl

    breakdown = {}
    for name in names:
        tot_b = tot_f = 0
        tot_ms = 0.0
        for k, pr in enumerate(wl.projections):
            if (name, k) not in per_launch:
                continue
            b_, f_ = work(name, pr)
            tot_b += b_
            tot_f += f_
            tot_ms += per_launch[(name, k)]
        breakdown[name] = dict(us_per_step=round(1e3 * tot_ms, 3), bytes=tot_b, flops=tot_f,
                               gbs=round(tot_b / (tot_ms * 1e-3) / 1e9, 1) if tot_ms else None,
                               tflops=round(tot_f / (tot_ms * 1e-3) / 1e12, 2) if tot_ms else None)
    # Roofline.  The slowest forward call of the step (all the kernels that
    # one lora_linear_forward call enqueues) is reported as `forward_call`.
    # Where that call is MFMA-bound (bf16), the roofline unit is its dominant
    # kernel alone: the base GEMM with the fused expand of its slowest
    # projection (one k_gemm_bf16 launch, timed through lora_gemm_expand in
    # the same launch configuration).  Otherwise (HBM-bound decode, fp32,
    # FP8) it is the forward call.
    kd = max(fwd, key=lambda k: fwd[k])
    by_d, fl_d = fwd_work(kd)
    t_d = fwd[kd] * 1e-3
    ai = fl_d / by_d
    if wl.dtype == torch.float32:
        roof = dict(bound="alu", achieved=round(fl_d / t_d / 1e12, 2), peak=FP32_VALU_PEAK_TFS, unit="TFLOP/s")
    elif fp8 and ai >= RIDGE_FP8:
        roof = dict(bound="mfma", achieved=round(fl_d / t_d / 1e12, 2), peak=MFMA_FP8_PEAK_TFS, unit="TFLOP/s")
    elif not fp8 and ai >= RIDGE:
        roof = dict(bound="mfma", achieved=round(fl_d / t_d / 1e12, 2), peak=MFMA_BF16_PEAK_TFS, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=round(by_d / t_d / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = "forward"
    roof["projection"] = "+".join(wl.projections[k].name for k in groups[kd])
    roof["launches_per_step"] = 1
    roof["avg_launch_us"] = round(fwd[kd] * 1e3, 3)
    roof["algorithmic_bytes_per_launch"] = int(by_d)
    roof["algorithmic_flops_per_launch"] = int(fl_d)
    roof["traffic"] = stored_traffic("forward_fp8" if fp8 else "forward", args.workload, roof["projection"])
    forward_call = dict(roof)
    gname = "gemm" if args.separate_expand else "gemm_expand"
    if roof["bound"] == "mfma" and not fp8:
        cand = [(per_launch[(gname, k)], k) for k in groups[kd] if (gname, k) in per_launch]
        t_k, kk = max(cand)
        pk = wl.projections[kk]
        b_k, f_k = work(gname, pk)
        roof = dict(bound="mfma", achieved=round(f_k / (t_k * 1e-3) / 1e12, 2), peak=MFMA_BF16_PEAK_TFS,
                    unit="TFLOP/s")
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["kernel"] = ("k_gemm_bf16 (base GEMM, no adapters: the expand is a separate pass)"
                          if args.separate_expand else
                          "k_gemm_bf16 (base GEMM + fused expand of the long segments) + k_expand_short "
                          "(per-row expand of the short segments), one lora_gemm_expand call" if sgmv else
                          "k_gemm_bf16 (base GEMM + fused expand)")
        roof["projection"] = pk.name
        roof["shape"] = [T, pk.d_in, pk.d_out]
        roof["launches_per_step"] = sum(1 for p in wl.projections if (p.d_in, p.d_out) == (pk.d_in, pk.d_out))
        roof["avg_launch_us"] = round(t_k * 1e3, 3)
        roof["algorithmic_bytes_per_launch"] = int(b_k)
        roof["algorithmic_flops_per_launch"] = int(f_k)
        roof["traffic"] = stored_traffic(gname, args.workload, pk.name)
    # LoRA overhead: the step's forward calls against the base products alone
    base_ms = sum(per_launch[(n_, k)] for (n_, k) in per_launch if n_ in ("gemm", "gemm_fp8", "quantize"))
    overhead = dict(forward_us=round(1e3 * sum(fwd.values()), 3), base_only_us=round(1e3 * base_ms, 3) if base_ms else None,
                    overhead=round(sum(fwd.values()) / base_ms - 1.0, 4) if base_ms else None)
    breakdown["forward"] = dict(us_per_step=round(1e3 * sum(fwd.values()), 3),
                                per_call_us={"+".join(wl.projections[k].name for k in groups[gi]):
                                             round(1e3 * v, 3) for gi, v in fwd.items()})

    # ---- calibration copy kernel (counter scaling runs) ----
    if args.calib_copy:
        n = 256 * 2 ** 20 // 4 * 4                # 1 GiB of fp32 in, 1 GiB out
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print("calib-copy bytes_read=%d bytes_written=%d" % (a.numel() * 4, b.numel() * 4), file=sys.stderr)

    residency = measure_residency(wl, pools, dev) if args.residency else None

    # ---- CPU baseline: the fp64 oracle on a bounded sample of this batch ----
    cpu = None
    if not args.no_cpu_baseline and not fp8:      # the baseline belongs to the bf16 headline line
        cpu = cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == torch.float32 else ("e4m3+bf16" if fp8 else "bf16"),
        "data": "synthetic (seeded; random-init adapters and weights)",
        "config": {
            "workload": wl.name, "T": T, "projections": [[p.name, p.d_in, p.d_out] for p in wl.projections],
            "n_slots": wl.n_slots, "max_rank": R, "distinct_adapters": int(used.size),
            "mode": ("sgmv" if sgmv else "bgmv") + ("" if args.mode != "auto" else " (auto)"),
            "expand": "separate" if args.separate_expand else "fused into the base GEMM",
            "base": ("fp8 e4m3 (per-row x, per-column W scales); bf16 adapters" if fp8 else
                     ("fp32" if wl.dtype == torch.float32 else "bf16")),
            "calls": ["+".join(wl.projections[k].name for k in g) for g in groups],
            "adapters": "single (most frequent)" if args.single_adapter else "mixed",
            "pool": "packed (slot = its rank rows)" if args.packed_pool else "padded to max_rank",
            "cold_sets": n_sets, "working_set_MB": round(set_bytes / 1e6, 1),
        },
        "roofline": roof,
        "forward_call": forward_call,
        "breakdown": breakdown,
        "lora_overhead": overhead,
        "cpu_baseline": cpu,
    }
    if residency is not None:
        line["residency"] = residency
    print(json.dumps(line), flush=True)


def measure_residency(wl, pools, dev):
    """Promotion rate of the adapter cache: 2 x Bn adapters packed in pinned
    host memory, a cache of Bn slots over every projection's pool, and maps
    that alternate between the two halves, so each map copies Bn adapters
    into evicted slots.  Timed with events on the copy stream."""
    import torch

    from rank_adapter_gemm_amd import lora as L

    R = wl.max_rank
    per_adapter = sum(R * (p.d_in + p.d_out) * (4 if wl.dtype == torch.float32 else 2) for p in wl.projections)
    bn = int(max(1, min(16, wl.n_slots // 2, (512 << 20) // (2 * per_adapter))))
    cache = L.AdapterCache(bn, [pl.pool for pl in pools], 2 * bn)
    code = L.dtype_code(wl.dtype)
    keep = []
    for a in range(2 * bn):
        ha, hb = [], []
        for pr in wl.projections:
            A = (torch.randn(pr.d_in, R) * 0.02).to(wl.dtype)
            B = (torch.randn(R, pr.d_out) * 0.02).to(wl.dtype)
            sa = torch.empty(R * pr.d_in, dtype=wl.dtype).pin_memory()
            sb = torch.empty(R * pr.d_out, dtype=wl.dtype).pin_memory()
            L.lora_pack_host(pr.d_in, pr.d_out, R, code, A, B, R, sa, sb)
            ha.append(sa)
            hb.append(sb)
        cache.register(a, ha, hb, R, 2.0 * R)
        keep.append((ha, hb))
    copy = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    halves = [list(range(bn)), list(range(bn, 2 * bn))]
    for i in range(2):
        cache.map(halves[i % 2], compute, copy)
        cache.commit(compute)
    torch.cuda.synchronize()
    rounds = 8
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    b0 = cache.stats()["bytes"]
    e0.record(copy)
    for i in range(rounds):
        cache.map(halves[i % 2], compute, copy)
        cache.commit(compute)
    e1.record(copy)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    moved = cache.stats()["bytes"] - b0
    cache.close()
    return {"h2d_gbs": round(moved / (ms * 1e-3) / 1e9, 2), "adapters_per_s": round(rounds * bn / (ms * 1e-3), 1),
            "bytes_per_adapter": per_adapter, "adapters_per_map": bn, "maps": rounds,
            "host_memory": "pinned, slot layout"}


def stored_traffic(kernel: str, workload: str, projection: str | None = None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    key = "%s/%s" % (workload, kernel)
    ent = data.get(key + ("/" + projection if projection else ""))
    if ent is None and projection:
        # a record may cover several projections of one launch shape
        # ("gate,up": the counter means were taken over both launches)
        for k, v in data.items():
            if k.startswith(key + "/") and projection in k[len(key) + 1:].split(","):
                ent = v
                break
    if not ent or ent.get("source_sha") != source_sha(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(wl, target_s):
    import numpy as np
    import torch

    from oracle import BF16, F32, affinity_cores, default_threads, lora_scale, oracle_rows

    def host(t):
        t = t.detach().contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    # every core of the affinity mask, within the host's declared CPU share
    # (OMP_NUM_THREADS) where one is set
    cores = default_threads()
    mask = affinity_cores()
    code = F32 if wl.dtype == torch.float32 else BF16
    # The adapters were released after upload: redraw them the same way (same seed) on the host side
    from rank_adapter_gemm_amd.workloads import make_workload
    wl2 = make_workload(wl.name, device="cuda")
    xs = {g: host(x) for g, x in wl2.xs.items()}
    rng = np.random.default_rng(12345)
    order = rng.permutation(wl.T)
    scales = [lora_scale(float(a), int(r)) for a, r in zip(wl2.alphas, wl2.ranks)]
    # Row chunks grow until the sample holds about target_s of CPU work; a
    # batch smaller than that is cycled through again (each row is a full,
    # independent evaluation of every projection).
    rows_done, elapsed, n = 0, 0.0, 8 * cores
    per_proj = []
    for pr in wl2.projections:
        per_proj.append(dict(W=host(pr.W), A=pr.A, B=pr.B, x=xs[pr.x_group]))
    while elapsed < target_s:
        take = order[np.arange(rows_done, rows_done + n) % wl.T]
        used = sorted({int(wl.ids[t]) for t in take if 0 <= wl.ids[t] < wl.n_slots})
        for pp in per_proj:
            A = [None] * wl.n_slots
            B = [None] * wl.n_slots
            for s in used:
                r = int(wl2.ranks[s])
                A[s] = host(pp["A"][s, :, :r])
                B[s] = host(pp["B"][s, :r, :])
            t0 = time.perf_counter()
            oracle_rows(code, pp["x"], pp["W"], wl.ids, A, B, [int(r) for r in wl2.ranks], scales,
                        rows=take, n_threads=cores)
            elapsed += time.perf_counter() - t0
        rows_done += len(take)
        n = min(2 * n, 4096)
    share = os.environ.get("OMP_NUM_THREADS")
    return {"value": round(rows_done / elapsed, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "affinity_cores": mask, "cpu_share": int(share) if share and share.isdigit() else None,
            "sample": "%d token rows drawn from the %d-row %s batch (seeded order, cycled), all %d "
                      "projection(s), fp64 C oracle, %d threads, %.1f s" % (
                          rows_done, wl.T, wl.name, len(wl2.projections), cores, elapsed)}


if __name__ == "__main__":
    main()
