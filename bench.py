#!/usr/bin/env python3
"""Throughput of the gfx950 ragged-M grouped GEMM on one MI355X.

One step = one launch of the whole path (device tile schedule, per-expert tile
height, bf16 matrix-core K loop, register-direct epilogue) over one batch of
synthetic, seeded inputs already resident in HBM. Default workload: the
uniform large batch of the Blackwell worklog's headline runs (64 experts x 256
routed rows, K=1024, N=2688, 90.2 GFLOP useful). The other full-size
workloads (the decode shape, the skewed 16k batch, the small skewed batch
with wide weights) are timed after it, outside its timed region, and reported
under "other_configs".

Prints one JSON line:
  value      useful TFLOP/s = 2*M_tot*K*N / (time per step)
  roofline   the kernel against its bound: algorithmic bytes (A once, B once
             per expert with rows, C once) per launch over the average
             launch time (HIP events on the launch stream), vs 8 TB/s HBM3E;
             or useful flops vs 2.5 PFLOP/s dense bf16 when the workload's
             arithmetic intensity is above the ridge point. "traffic" is the
             measured HBM bytes per launch from the committed rocprofv3
             counter summary, when that summary matches the current kernel
             sources, else null.
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
             (best of 3 passes on all its threads, and on one thread).

    python bench.py [--steps K] [--warmup W] [--config uniform16k] [--bm 0]
                    [--out fp32|bf16|swiglu] [--also decode,skew16k,skew2k_wide]

--out bf16 times the bf16-output entry point (C rounded to bf16 in the
epilogue); its algorithmic bytes count C at 2 bytes per element. --out swiglu
times the fused gate/up entry point (B's columns read as interleaved gate and
up pairs, bf16 H of N/2 columns written); its output counts at 1 byte per
product column. --gather and --combine time the entry points that reach rows
by index (a seeded top-1 permutation); --combine adds weight * row into fp32
output rows with atomics, counted as a read and a write of every output
element. --weights fp8 times fp8 weights with bf16 activations (widened to
bf16 before the matrix cores); --weights fp8 --acts fp8 times fp8 activations
and weights on the fp8 matrix cores, against the fp8 peak (5.0 PFLOP/s).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "useful TFLOP/s (2*M_tot*K*N/t) + HBM GB/s, % of roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
KERNEL_NAME = "grouped_gemm_kernel"

DESCRIPTIONS = {
    "tiny": "tiny ragged grouped GEMM: E=4, K=256, N=256, m=[3,0,17,9]",
    "decode": "decode shape: E=32 experts x 16 rows (M_tot=512), K=6144, N=4096",
    "uniform16k": "uniform large batch: E=64 x 256 rows (M_tot=16384), K=1024, N=2688",
    "skew16k": "skewed routing rank^-1.2: E=64, M_tot=16384, K=1024, N=2688",
    "skew2k_wide": "small skewed batch, wide weights: E=32, M_tot=2048 rank^-1.2, K=6144, N=4096",
    "skew16k_page": "page skew law (e+1)^-1.2: E=64, M_tot=16384, K=1024, N=2688",
}


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank space taken out, so
    that a change to a comment does not mark the measured counters stale. The
    blocks only the tracing build compiles (#ifdef GG_TILE_TRACE) are taken
    out too: the product library is built without them."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_ragged_grouped_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"#ifdef GG_TILE_TRACE\b.*?#endif", " ", text, flags=re.S)
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(fn.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_key(config, bm, out="fp32", weights="bf16", rows="grouped"):
    """Key of a workload and entry point in profiles/traffic.json."""
    return ("%s/bm%d" % (config, bm) + ("" if out == "fp32" else "/" + out)
            + ("" if weights == "bf16" else "/%sw" % weights)
            + ("" if rows == "grouped" else "/" + rows))


def measured_traffic(config, bm, out="fp32", weights="bf16", rows="grouped"):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        key = traffic_key(config, bm, out, weights, rows)
        rec = json.load(open(path)).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s=12.0):
    """Time the CPU oracle on a bounded sample of the workload.

    The sample is the first n experts with rows (whole rows, full K and N),
    n chosen so that one pass takes about a quarter of the budget on all the
    oracle's threads; the figure is the best of 3 passes. The same is done on
    one thread with a sample sized to about a tenth of the budget.
    """
    import numpy as np

    import oracle

    nz = [e for e in range(w.E) if w.sizes[e] > 0]

    def run(n):
        e1 = nz[n - 1] + 1
        off = w.offsets[: e1 + 1].copy()
        rows = int(off[-1])
        t0 = time.perf_counter()
        oracle.grouped_gemm(w.A[:rows], w.B[:e1], off, M_cap=rows)
        return time.perf_counter() - t0, 2.0 * rows * w.K * w.N, rows, e1

    def leg(target_s):
        run(1)  # first touch of the pages
        dt1 = run(1)[0]
        n = int(max(1, min(len(nz), target_s / max(dt1, 1e-6))))
        best = None
        for _ in range(3):
            dt, flops, rows, e1 = run(n)
            best = dt if best is None else min(best, dt)
        return flops / best / 1e12, best, rows, e1

    threads = oracle.threads()
    v, dt, rows, e1 = leg(budget_s / 4)
    oracle.set_threads(1)
    try:
        v1, dt1, rows1, e11 = leg(budget_s / 10)
    finally:
        oracle.set_threads(threads)
    return {
        "value": v,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "experts 0..%d of the %s workload (%d routed rows, full K=%d and N=%d), fp64 "
                  "accumulation plus the sum|ab| bound, best of 3 passes of %.2f s on %d threads" % (
                      e1 - 1, w.name, rows, w.K, w.N, dt, threads),
        "nproc": os.cpu_count(),
        "one_thread": {"value": v1, "unit": "TFLOP/s",
                       "sample": "experts 0..%d (%d rows), best of 3 passes of %.2f s" % (
                           e11 - 1, rows1, dt1)},
    }


def launch_counts(sizes, K, N, args):
    """Useful flops, algorithmic bytes and the matrix-core peak of one launch.

    Useful flops are 2 * M_tot * K * N. The bytes count what the method must
    move, once: A's routed rows, B of every expert with rows, and C, each at
    its own element size (fp8 operands with their fp32 scales). Padding,
    repeated reads and empty experts' weights are not counted. Gathered rows
    add their two index lists; the combine adds a read of each output element
    and a weight per row."""
    import numpy as np
    sizes = np.asarray(sizes)
    M_tot = int(sizes.sum())
    useful = 2.0 * M_tot * K * N
    c_bytes = {"fp32": 4, "bf16": 2, "swiglu": 1}[args.out]  # per product column
    active = int((sizes > 0).sum())
    b_bytes = 2 * K * N * active if args.weights == "bf16" else (K + 4) * N * active
    a_bytes = 2 * M_tot * K if args.acts == "bf16" else (K + 4) * M_tot
    alg_bytes = (a_bytes + b_bytes + c_bytes * M_tot * N
                 + (8 * M_tot if args.gather else 0)
                 # the combine reads each output element before adding, and a weight per row
                 + (4 * M_tot * N + 4 * M_tot if args.combine else 0))
    # the matrix-core peak of the operand type: fp8 x fp8 on the fp8 cores,
    # otherwise bf16 (fp8 weights are widened to bf16 for the matrix cores)
    mfma_peak = MFMA_FP8_PEAK_TFLOPS if args.acts == "fp8" else MFMA_BF16_PEAK_TFLOPS
    return useful, alg_bytes, mfma_peak


def prepare(w, args, dev):
    """Device inputs for one workload and the launch a step makes.

    Returns a dict with the step function and the byte and flop counts of
    one launch. The inputs are drawn and quantized on the host (untimed)."""
    import numpy as np
    import torch

    import moe_ragged_grouped_amd as gg
    import workloads as wl

    A = torch.from_numpy(w.A.view(np.int16)).to(dev).view(torch.bfloat16)
    off = torch.from_numpy(w.offsets).to(dev)
    c_dtype = torch.float32 if args.out == "fp32" else torch.bfloat16
    C = torch.empty((w.M_cap, w.N // 2 if args.out == "swiglu" else w.N), dtype=c_dtype,
                    device=dev)
    B = Bq = Bs = Aq = As = X = perm = gate = None
    if args.weights == "fp8":
        # fp8 E4M3 weights with per-(expert, column) fp32 scales, quantized
        # from the bf16 weights on the host (input recipe, untimed)
        q_np, sc_np = wl.fp8_weights(w)
        Bq = torch.from_numpy(q_np).to(dev)
        Bs = torch.from_numpy(sc_np).to(dev)
        del q_np
    else:
        B = torch.from_numpy(w.B.view(np.int16)).to(dev).view(torch.bfloat16)
    if args.acts == "fp8":
        aq_np, as_np = wl.fp8_activations(w)
        Aq = torch.from_numpy(aq_np).to(dev)
        As = torch.from_numpy(as_np).to(dev)
    if args.gather:
        # rows reached by index: X holds the routed rows in a seeded random
        # (token) order, grouped row r reads X[perm[r]] and is written back to
        # C[perm[r]] (top-1 routing: permute in, GEMM, permute out)
        perm_np = np.random.default_rng(w.seed + 500).permutation(w.M_cap).astype(np.int32)
        X = torch.empty_like(A)
        X[torch.from_numpy(perm_np).long().to(dev)] = A
        perm = torch.from_numpy(perm_np).to(dev)
        if args.combine:
            # gate weights in (0, 1]; C accumulates across steps (the kernel's
            # work does not depend on its values, and clearing it inside the
            # timed region would time a fill kernel too)
            gate = torch.from_numpy(np.random.default_rng(w.seed + 501).uniform(
                0.05, 1.0, w.M_cap).astype(np.float32)).to(dev)
            C.zero_()

    def step():
        if args.acts == "fp8" and args.out == "swiglu":
            gg.grouped_gemm_fp8_swiglu(Aq, As, Bq, Bs, off, out=C, bm=args.bm)
        elif args.acts == "fp8":
            gg.grouped_gemm_fp8(Aq, As, Bq, Bs, off, out=C, bm=args.bm)
        elif args.weights == "fp8":
            gg.grouped_gemm_fp8w(A, Bq, Bs, off, out=C, bm=args.bm)
        elif args.combine:
            gg.grouped_gemm_gather_combine(X, perm, B, off, perm, gate, out=C, bm=args.bm)
        elif args.gather:
            gg.grouped_gemm_gather(X, perm, B, off, dst_rows=perm, out=C, bm=args.bm)
        elif args.out == "swiglu":
            gg.grouped_gemm_swiglu(A, B, off, out=C, bm=args.bm)
        else:
            gg.grouped_gemm(A, B, off, out=C, bm=args.bm)

    useful, alg_bytes, mfma_peak = launch_counts(w.sizes, w.K, w.N, args)
    return {"step": step, "useful": useful, "alg_bytes": alg_bytes, "mfma_peak": mfma_peak,
            "off": off, "A": A, "B": B, "C": C}


def library_yardstick(w, run, args, stream):
    """The same products through the vendor GEMM library (hipBLASLt via torch),
    timed like the grouped launch, on the same resident bf16 inputs and with
    fp32 outputs: a strided-batched product when every expert has the same row
    count, and one library GEMM per expert with rows (the E launches a grouped
    GEMM replaces). A measuring stick only: nothing of it is the library's
    path, and its results are not compared."""
    import numpy as np
    import torch

    A, B = run["A"], run["B"]
    C = torch.empty((w.M_cap, w.N), dtype=torch.float32, device=A.device)
    off = [int(x) for x in w.offsets]
    experts = [e for e in range(w.E) if off[e + 1] > off[e]]
    cases = {}
    if len(set(int(off[e + 1] - off[e]) for e in range(w.E))) == 1 and w.M_tot > 0:
        m = w.M_tot // w.E
        A3 = A[: w.M_tot].view(w.E, m, w.K)
        C3 = C[: w.M_tot].view(w.E, m, w.N)
        cases["bmm_strided_batched"] = lambda: torch.bmm(A3, B, out_dtype=torch.float32, out=C3)
    views = [(A[off[e]:off[e + 1]], B[e], C[off[e]:off[e + 1]]) for e in experts]
    # the same flops as one dense product with a single expert's weights
    # (M_tot x K times K x N): no weight stream, the library's best case
    if experts:
        A2, B2, C2 = A[: w.M_tot], B[experts[0]], C[: w.M_tot]
        cases["dense_one_weight_matrix"] = lambda: torch.mm(A2, B2, out_dtype=torch.float32, out=C2)

    def loop():
        for a, b, c in views:
            torch.mm(a, b, out_dtype=torch.float32, out=c)
    cases["mm_per_expert_loop"] = loop
    # the same loop captured in a HIP graph: the host's per-launch cost drops out
    loop()
    gs = torch.cuda.Stream(A.device)
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        loop()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        loop()
    torch.cuda.synchronize()
    cases["mm_per_expert_loop_graph"] = graph.replay
    cases["grouped_gemm (this library)"] = run["step"]
    out = {}
    for name, f in cases.items():
        f()
        ramp(f, args.ramp_ms)
        for _ in range(args.warmup):
            f()
        t, _ = time_launches(f, args.steps, stream)
        out[name] = {"avg_us": round(t * 1e6, 2),
                     "useful_tflops": round(2.0 * w.M_tot * w.K * w.N / t / 1e12, 2),
                     "launches": len(views) if name.startswith("mm_per_expert") else 1}
    del graph
    # the library's rate on a large square bf16 product (bf16 output), for
    # scale: what its kernels reach where the shape does not limit them
    n = 8192
    X = torch.randn(n, n, device=A.device).to(torch.bfloat16)
    Y = torch.randn(n, n, device=A.device).to(torch.bfloat16)
    Z = torch.empty(n, n, device=A.device, dtype=torch.bfloat16)
    sq = lambda: torch.mm(X, Y, out=Z)
    ramp(sq, args.ramp_ms)
    t, _ = time_launches(sq, 10, stream)
    out["square_8192_bf16_mm"] = {"avg_us": round(t * 1e6, 2),
                                  "tflops": round(2.0 * n ** 3 / t / 1e12, 2), "launches": 1}
    return out


def tile_trace_summary(tr, khz, wg_total, n_tiles):
    """Summary of one traced launch (gg_trace_grouped_gemm_bf16's records):
    times in microseconds from the earliest workgroup start."""
    import numpy as np
    import moe_ragged_grouped_amd as gg
    us = 1000.0 / khz
    W = gg.TRACE_WORKGROUPS
    wg = tr[:wg_total]
    tl = tr[W:W + n_tiles]
    assert (tl[:, 0] > 0).all() and (tl[:, 2] >= tl[:, 1]).all() and \
        (tl[:, 1] >= tl[:, 0]).all(), "a tile has no record"
    assert int(wg[:, 3].sum()) == n_tiles, "the workgroups ran %d of %d tiles" % (
        int(wg[:, 3].sum()), n_tiles)
    t0 = int(wg[:, 0].min())
    start = (tl[:, 0] - t0) * us
    decoded = (tl[:, 1] - t0) * us
    end = (tl[:, 2] - t0) * us
    dur = end - start
    height = tl[:, 3]
    owner = tl[:, 4]
    finish = np.zeros(wg_total)
    busy = np.zeros(wg_total)
    np.maximum.at(finish, owner, end)
    np.add.at(busy, owner, dur)
    gaps = []
    for b in range(wg_total):
        s_b = np.sort(start[owner == b])
        e_b = np.sort(end[owner == b])
        if len(s_b) > 1:
            gaps.extend((s_b[1:] - e_b[:-1]).tolist())
    xcc = (wg[:, 2] >> 6).astype(int)
    first = np.full(wg_total, np.inf)
    np.minimum.at(first, owner, start)
    entry = (wg[:, 0] - t0) * us
    out = {
        "span_us": round(float(end.max()), 2),
        "entry_to_first_tile_us": round(float(np.mean(first[np.isfinite(first)] -
                                                      entry[np.isfinite(first)])), 2),
        "schedule_build_us": round(float(np.mean((wg[:, 1] - wg[:, 0]) * us)), 2),
        "workgroup_finish_us": {"min": round(float(finish.min()), 1),
                                "mean": round(float(finish.mean()), 1),
                                "max": round(float(finish.max()), 1)},
        "workgroup_busy_us": {"mean": round(float(busy.mean()), 1),
                              "max": round(float(busy.max()), 1)},
        "gap_between_tiles_us": ({"median": round(float(np.median(gaps)), 2),
                                  "p90": round(float(np.percentile(gaps, 90)), 2),
                                  "count": len(gaps)} if gaps else None),
        "tile_decode_us": {"median": round(float(np.median(decoded - start)), 2),
                           "p90": round(float(np.percentile(decoded - start, 90)), 2)},
        "tiles_by_height": {int(h): {"count": int((height == h).sum()),
                                     "mean_us": round(float(dur[height == h].mean()), 1)}
                            for h in sorted(set(height.tolist()))},
        "xcd_busy_mean_us": [round(float(busy[xcc == x].mean()), 1) if (xcc == x).any() else None
                             for x in range(8)],
        # the launch order assumes workgroup b runs on XCD b % 8
        "workgroups_on_xcd_b_mod_8": round(float(np.mean(xcc == np.arange(wg_total) % 8)), 4),
    }
    # the tallest tiles by when they start: early (first 30% of the span)
    # against late (after 60%)
    tall = height == height.max()
    early, late = tall & (start < 0.3 * end.max()), tall & (start > 0.6 * end.max())
    if early.any() and late.any():
        out["tallest_tile_us_by_start"] = {"first_30pct": round(float(dur[early].mean()), 1),
                                           "after_60pct": round(float(dur[late].mean()), 1)}
    # mean duration per first column, where the launch has few column positions
    col0 = tl[:, 7]
    if len(set(col0.tolist())) <= 16:
        out["tile_us_by_col0"] = {int(c): round(float(dur[col0 == c].mean()), 1)
                                  for c in sorted(set(col0.tolist()))}
    return out


def ramp(step, ms):
    """Untimed launches for at least ms milliseconds; returns their count."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    return n


def time_launches(step, steps, stream):
    """Average launch time over steps back-to-back launches (HIP events on the
    launch stream) and the host's wall time around them."""
    import torch
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_s = ev0.elapsed_time(ev1) / 1e3
    return ev_s / steps, wall


def roofline(useful, alg_bytes, launch_s, mfma_peak):
    """The bound of a launch and its achieved fraction of it."""
    intensity = useful / alg_bytes
    hbm_gbs = alg_bytes / launch_s / 1e9
    tflops = useful / launch_s / 1e12
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4)}
    return roof, hbm_gbs, tflops


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="uniform16k", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--also", default="decode,skew16k,skew2k_wide",
                    help="other workloads timed after the headline one, outside its timed "
                         "region (comma-separated, or none)")
    ap.add_argument("--bm", type=int, default=0, help="0 = per-expert tile height chosen on the device")
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="untimed launches for at least this long before the warmup steps, so "
                         "the GPU clocks have left their idle state when timing starts")
    ap.add_argument("--out", default="fp32", choices=("fp32", "bf16", "swiglu"),
                    help="what the epilogue writes: fp32 C, bf16 C, or bf16 SwiGLU of "
                         "(gate, up) column pairs")
    ap.add_argument("--acts", default="bf16", choices=("bf16", "fp8"),
                    help="activations: bf16, or fp8 E4M3 with per-row scales (needs "
                         "--weights fp8; fp8 matrix cores)")
    ap.add_argument("--weights", default="bf16", choices=("bf16", "fp8"),
                    help="fp8: E4M3 weights with per-column scales (a separate precision)")
    ap.add_argument("--gather", action="store_true",
                    help="time the gather/scatter entry point (A rows and C rows by index)")
    ap.add_argument("--combine", action="store_true",
                    help="time the gather + weighted-combine entry point (fp32 atomic adds "
                         "into the token rows; with --gather's top-1 permutation)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-timings", action="store_true",
                    help="skip the graph-captured and cold-cache timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="time only plain device-wide streams through torch (a 1 GiB copy, the "
                         "sum of two 1 GiB buffers and a 1 GiB read-only reduction) for the "
                         "box's practical HBM rate")
    ap.add_argument("--tile-trace", action="store_true",
                    help="time only the launch's per-tile timeline, through the tracing build "
                         "(bf16 weights, fp32 C, grouped rows): workgroup finish times, tile "
                         "durations by height, time per XCD")
    ap.add_argument("--trace-out", default=None,
                    help="with --tile-trace: also save the raw records of the three traced "
                         "launches (int64 [3, records, values]) to this .npy file")
    ap.add_argument("--library-yardstick", action="store_true",
                    help="time only the same products through hipBLASLt (torch) beside this "
                         "library's launch (bf16 weights, fp32 output, grouped rows)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU "
              "runs the kernel on its own experts' share; the exchanges sit outside it); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.combine:
        args.gather = True
    if args.weights == "fp8" and ((args.out != "fp32" and args.acts == "bf16") or args.gather):
        raise SystemExit("--weights fp8 times the fp32-output grouped-row entry point")
    if args.acts == "fp8" and (args.weights != "fp8" or args.gather):
        raise SystemExit("--acts fp8 needs --weights fp8 and grouped rows")
    if args.gather and args.out != "fp32":
        raise SystemExit("--gather times the fp32-output gather entry point")

    import numpy as np
    import torch

    import moe_ragged_grouped_amd as gg
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5}))
        return

    if args.hbm_ceiling:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        src2 = torch.ones_like(src)
        dst = torch.empty_like(src)
        acc = torch.empty((), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream(dev)
        res = {}
        # the sum of two buffers reads two bytes per byte written, near the
        # grouped product's own mix at fp32 output (about 69% of its bytes read)
        for name, f, moved in (("copy_read_plus_write", lambda: dst.copy_(src), 2 * n),
                               ("add_two_reads_one_write",
                                lambda: torch.add(src, src2, out=dst), 3 * n),
                               ("sum_read_only", lambda: torch.sum(src, dim=0, out=acc), n)):
            ramp(f, args.ramp_ms)
            t, _ = time_launches(f, 20, stream)
            res[name] = {"avg_us": round(t * 1e6, 2), "bytes": moved,
                         "gbs": round(moved / t / 1e9, 1),
                         "frac_of_8tbs": round(moved / t / 1e9 / HBM_PEAK_GBS, 4)}
        print(json.dumps({"hbm_ceiling": res}), flush=True)
        return

    print("bench: drawing workload %s" % args.config, file=sys.stderr, flush=True)
    w = wl.make_workload(args.config)
    run = prepare(w, args, dev)
    step = run["step"]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    if args.library_yardstick:
        if args.weights != "bf16" or args.out != "fp32" or args.gather:
            raise SystemExit("--library-yardstick times bf16 weights, fp32 C, grouped rows")
        print(json.dumps({"library_yardstick": library_yardstick(w, run, args, stream),
                          "workload": DESCRIPTIONS[args.config], "name": args.config,
                          "steps": args.steps, "warmup": args.warmup}), flush=True)
        return
    if args.tile_trace:
        if args.weights != "bf16" or args.out != "fp32" or args.gather or args.acts != "bf16":
            raise SystemExit("--tile-trace traces bf16 weights, fp32 C, grouped rows")
        _, n_tiles = gg.tile_schedule(run["off"], w.N, w.M_cap, bm=args.bm)
        shape = (gg.TRACE_WORKGROUPS + int(n_tiles), gg.TRACE_RECORD)
        scratch = torch.zeros(shape, dtype=torch.int64, device=dev)
        traces = [torch.zeros(shape, dtype=torch.int64, device=dev) for _ in range(3)]

        def traced(buf):
            return gg.traced_grouped_gemm(run["A"], run["B"], run["off"], n_tiles, out=run["C"],
                                          bm=args.bm, trace=buf)[2]
        traced(scratch)  # loads the tracing build's code before anything is timed
        ramp(step, args.ramp_ms)
        launch_s, _ = time_launches(step, args.steps, stream)
        # A pause of the host leaves the next ~100 launches of the 16k shapes
        # slow while the clocks recover, so the recorded launches come after
        # a ramp of traced launches and 120 more without a wait.
        ramp(lambda: traced(scratch), args.ramp_ms)
        for _ in range(120):
            khz = traced(scratch)
        for buf in traces:
            traced(buf)
        torch.cuda.synchronize()
        if args.trace_out:
            np.save(args.trace_out, np.stack([t.cpu().numpy() for t in traces]))
        wg_total = int((traces[-1][:gg.TRACE_WORKGROUPS, 0] > 0).sum().item())
        last = [tile_trace_summary(t.cpu().numpy(), khz, wg_total, int(n_tiles))
                for t in traces]
        print(json.dumps({"tile_trace": last, "workload": DESCRIPTIONS[args.config],
                          "name": args.config, "workgroups": wg_total, "tiles": int(n_tiles),
                          "clock_khz": khz, "product_launch_us": round(launch_s * 1e6, 2)}),
              flush=True)
        return
    step()  # correctness launch position of the protocol
    # Clock ramp: after the seconds of host-side input generation the GPU sits
    # at idle clocks, and a few milliseconds of warmup launches do not bring
    # it back up (a 10-launch warmup times the 16k shape about 18% slow).
    ramp_launches = ramp(step, args.ramp_ms)
    print("bench: clock ramp %d launches, warmup %d launches" % (ramp_launches, args.warmup),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    print("bench: timing %d launches" % args.steps, file=sys.stderr, flush=True)
    launch_s, wall = time_launches(step, args.steps, stream)
    step_s = max(wall / args.steps, launch_s)  # the step as the host sees it

    useful, alg_bytes, mfma_peak = run["useful"], run["alg_bytes"], run["mfma_peak"]
    roof, hbm_gbs, tflops_launch = roofline(useful, alg_bytes, launch_s, mfma_peak)
    rows_mode = "combine" if args.combine else "gather" if args.gather else "grouped"
    weights_key = "fp8a" if args.acts == "fp8" else args.weights
    roof["traffic"] = measured_traffic(args.config, args.bm, args.out, weights_key, rows_mode)
    roof["kernel"] = KERNEL_NAME
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["avg_launch_us"] = round(launch_s * 1e6, 2)

    # the device's tile list for this launch (untimed): tile count, tile
    # heights and row efficiency eta = routed rows / scheduled rows
    tiles, n_tiles = gg.tile_schedule(run["off"], w.N, w.M_cap, bm=args.bm)
    tl = tiles.cpu().numpy()
    first = tl[tl[:, 3] == 0]  # one entry per M tile (its first column tile)
    heights = {int(h): int((first[:, 4] == h).sum()) for h in sorted(set(first[:, 4].tolist()))}
    schedule = {"tiles": int(n_tiles), "m_tiles": int(len(first)), "m_tiles_by_height": heights,
                "eta": round(float(first[:, 2].sum()) / max(1.0, float(first[:, 4].sum())), 4)}

    # Two more timings of the same launch, outside the timed region above:
    #  graph: launches captured in a HIP graph (no host launch cost, as the
    #    worklog and the Pearl Pulse page time their kernels), median per launch;
    #  cold: each launch timed alone after a 512 MB write has pushed the
    #    inputs out of the L2s and the 256 MB Infinity Cache, median.
    extra = {}
    if not args.no_extra_timings:
        n_rep = 20
        gs = torch.cuda.Stream(dev)
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            step()  # settle allocations on the capture stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for _ in range(n_rep):
                step()
        torch.cuda.synchronize()
        # The capture leaves the GPU idle for tens of milliseconds, and after
        # such a pause the first ~100 launches of the 16k shapes run up to 40%
        # slow while the clocks recover: replay untimed first.
        ramp(graph.replay, args.ramp_ms)
        times = []
        for _ in range(5):
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            graph.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            times.append(g0.elapsed_time(g1) * 1e3 / n_rep)
        extra["graph_median_us"] = round(float(np.median(times)), 2)
        del graph
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ramp(step, args.ramp_ms)
        cold = []
        for i in range(n_rep):
            flush.fill_(i & 0xFF)
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1) * 1e3)
        extra["cold_median_us"] = round(float(np.median(cold)), 2)
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w)

    # The other full-size workloads with the same entry point, each timed the
    # same way after its own clock ramp and warmup.
    others = {}
    del run, step
    also = [] if args.also in ("", "none") else args.also.split(",")
    for name in [x for x in also if x and x != args.config]:
        if name not in DESCRIPTIONS:
            raise SystemExit("unknown workload %s" % name)
        print("bench: drawing workload %s" % name, file=sys.stderr, flush=True)
        wo = wl.make_workload(name)
        ro = prepare(wo, args, dev)
        ro["step"]()
        ramp(ro["step"], args.ramp_ms)
        for _ in range(args.warmup):
            ro["step"]()
        torch.cuda.synchronize()
        print("bench: timing %s, %d launches" % (name, args.steps), file=sys.stderr, flush=True)
        lo, _ = time_launches(ro["step"], args.steps, stream)
        r_o, gbs_o, tf_o = roofline(ro["useful"], ro["alg_bytes"], lo, ro["mfma_peak"])
        others[name] = {"workload": DESCRIPTIONS[name], "avg_launch_us": round(lo * 1e6, 2),
                        "useful_tflops": round(tf_o, 2), "hbm_gbs": round(gbs_o, 1),
                        "hbm_frac": round(gbs_o / HBM_PEAK_GBS, 4),
                        "mfma_frac": round(tf_o / ro["mfma_peak"], 4),
                        "roofline": {"bound": r_o["bound"], "frac": r_o["frac"]},
                        "algorithmic_bytes_per_launch": ro["alg_bytes"]}
        del ro, wo
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(useful / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ramp_launches": ramp_launches,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8" if args.acts == "fp8" else "bf16" if args.weights == "bf16"
                  else "fp8w-bf16"),
        "data": "synthetic (seeded normal draws rounded to bf16, no dataset)",
        "config": {"workload": DESCRIPTIONS[args.config], "name": args.config, "E": w.E, "K": w.K,
                   "N": w.N, "M_tot": w.M_tot, "bm": args.bm or "per-expert", "out_dtype": args.out,
                   "rows": ("gathered, weighted combine by fp32 atomics" if args.combine else
                            "gathered/scattered by index" if args.gather else "grouped"),
                   "weights": "bf16" if args.weights == "bf16"
                   else "fp8 e4m3 + fp32 scale per expert column",
                   "activations": "bf16" if args.acts == "bf16"
                   else "fp8 e4m3 + fp32 scale per row"},
        "hbm_gbs": round(hbm_gbs, 1),
        "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops_launch / mfma_peak, 4),
        "roofline": roof,
        "schedule": schedule,
        "timings": extra,
        "cpu_baseline": cpu,
        "other_configs": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
