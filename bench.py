#!/usr/bin/env python3
"""Benchmark of the sparse x dense multiply C = A_sparse * B_dense on one MI355X.

A step is one spmm_execute (every kernel the plan launches) over one dense B
that is already resident in HBM; packing and planning are one-time costs,
reported separately.  For the sampled dense-dense workloads (format sddmm) a
step is one spmm_execute_sddmm over resident X and Y, and n is the inner
dimension kd.  The default workload is the largest one-GPU case: the
block-sparse prefill layer, A 18944 x 3584 bf16 in 64 x 64 blocks with 90% of
the blocks zero, times B of 65,536 token columns (the 7B-model prefill at 90%
block sparsity and 64K tokens of the AsyncSparse page's abstract); the other
workloads of the catalogue run with --workload.

Prints one JSON line:
  value      effective GFLOP/s = 2 * nnz * n / (time per step)  (n = kd for sddmm),
             warm: K back-to-back steps between two HIP events
  roofline   the dominant kernel against its bound: the larger of the HBM
             time (algorithmic bytes at 8 TB/s) and the MFMA time
             (algorithmic flops at the dtype's dense peak), from HIP events
             over the timed region on the stream the kernels run on;
             `traffic` is the HBM bytes per launch the hardware counters saw
             (profiles/hbm_traffic.md), or null when the library source has
             changed since they were taken
  cold       each of --cold-steps launches timed alone right after a 512 MB
             fill on the same stream (no operand left in L2 or the Infinity
             Cache): median, min, max, stdev, and the roofline of the median
  cpu_baseline  the CPU oracle timed on a bounded sample of rows of the same
             workload (a reported baseline, not a target), with the host's
             CPU model
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SpMM effective GFLOP/s (2*nnz*N) and % of HBM/MFMA roofline on 1 MI355X"
HEADLINE = "bcsr_prefill_18944x3584"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "i8": 5000.0}

# kernel whose launch dominates a step, per format
DOMINANT_KERNEL = {"bcsr": "bcsr_bf16_mfma", "wcsr": "wcsr_stream", "sp24": "sp24_i8_smfmac",
                   "sddmm": "sddmm_csr", "sddmm_bcsr": "sddmm_bcsr_mfma", "bcsr_csr": "bcsr_bf16_mfma",
                   "tvw": "sp24_i8_smfmac", "slide": "sp24_i8_smfmac"}
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def dominant_kernel(w, pinfo=None) -> str:
    """Kernel whose launch dominates a step; a BCSR plan with 128-row tiles
    (paired block rows) runs the paired kernel."""
    if w.fmt in ("tvw", "sp24") and w.elem == "bf16":
        return "sp24_bf16_smfmac"
    if w.fmt in ("bcsr", "bcsr_csr") and pinfo is not None and pinfo["tile_m"] == 128:
        return "bcsr_bf16_pair"
    return DOMINANT_KERNEL[w.fmt]
CSRC = os.path.join(ROOT, "sparse_dense_matrix_amd", "csrc")


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", type=int, default=0, metavar="G",
                    help="capture G steps into one HIP graph and replay it (steps rounded "
                         "up to a multiple of G); 0 launches every step from Python")
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="launches timed one by one, each after overwriting a 512 MB buffer "
                         "(L2 and Infinity Cache evicted); their median is reported as `cold` "
                         "beside the warm line (0 skips it)"),
    ap.add_argument("--dense-baseline", action="store_true",
                    help="BCSR workloads: also time the dense product of the same shape "
                         "(torch.matmul on the zero-filled bf16 A) to show where block "
                         "sparsity stops paying")
    ap.add_argument("--window-rows", type=int, default=None)
    ap.add_argument("--max-chunk-nnz", type=int, default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB (read 1 GiB, write 1 GiB), "
                         "to scale the HBM byte counters")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a markdown table of per-kernel durations from the rocprofv3 "
                         "kernel-trace database(s) under DIR, and exit")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="print the mean per dispatch of every counter in the rocprofv3 "
                         "counter CSVs under DIR, per kernel, and exit")
    return ap.parse_args()


def setup(w, S, args):
    """Draw inputs, pack and plan.  Returns a dict describing the workload."""
    import synth
    t0 = time.perf_counter()
    a = synth.make_a(w)
    B = synth.make_xy(w) if w.fmt in ("sddmm", "sddmm_bcsr") else synth.make_b(w)
    t_gen = time.perf_counter() - t0
    t0 = time.perf_counter()
    if w.fmt in ("bcsr", "sddmm_bcsr"):
        M = S.spmm_pack_bcsr(a["dense"], w.block, w.block)
        types = (S.BF16, S.BF16)
    elif w.fmt == "bcsr_csr":
        M = S.spmm_pack_bcsr_csr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals_bf16"],
                                 reorder=w.reorder)
        types = (S.BF16, S.BF16)
    elif w.fmt in ("wcsr", "sddmm"):
        W = args.window_rows or S.DEFAULT_WINDOW_ROWS
        T = args.max_chunk_nnz or S.DEFAULT_MAX_CHUNK_NNZ
        M = S.spmm_pack_wcsr(w.m, w.k, a["row_ptr"], a["col_idx"], a["vals"], W, T)
        types = (S.F32, S.F32)
    elif w.fmt == "tvw":
        M = S.spmm_pack_tvw(a["dense"], synth.TVW_TILE_M, synth.TVW_TILE_K)
        types = (S.BF16, S.BF16) if w.elem == "bf16" else (S.I8, S.I32)
    elif w.fmt == "slide":
        M = S.spmm_pack_slide(a["dense"], w.nm_group)
        types = (S.I8, S.I32)
    else:
        M = S.spmm_pack_24(a["dense"])
        types = (S.BF16, S.BF16) if w.elem == "bf16" else (S.I8, S.I32)
    t_pack = time.perf_counter() - t0
    t0 = time.perf_counter()
    if w.fmt == "sddmm":
        P = S.spmm_plan_sddmm(M, w.n, {"bf16": S.BF16, "i8": S.I8}.get(w.elem, S.F32))
    elif w.fmt == "sddmm_bcsr":
        P = S.spmm_plan_sddmm(M, w.n, S.BF16 if w.elem == "bf16" else S.I8)
    else:
        P = S.spmm_plan(M, w.n, *types)
    t_plan = time.perf_counter() - t0
    info = S.spmm_matrix_info(M)
    return {"a": a, "B": B, "M": M, "P": P, "info": info, "t_gen": t_gen, "t_pack": t_pack,
            "t_plan": t_plan}


def algorithmic(w, d):
    """(flops, bytes, dtype) of one step.  bytes = compulsory HBM traffic:
    the packed operand once, every B row the sparse operand touches once, and
    C written once."""
    info = d["info"]
    n = w.n
    flops = 2.0 * info["nnz"] * n
    if w.fmt == "bcsr_csr":
        # effective work counts the CSR entries (the stored zeros of the blocks
        # are overhead); bytes as for BCSR: the packed blocks, the B rows of
        # touched block columns and C once
        import sparse_dense_matrix_amd as S
        nnzb = info["nnzb"]
        cols = np.unique(S.spmm_matrix_array(d["M"], S.ARRAY_COL_IDX))
        flops = 2.0 * int(d["a"]["row_ptr"][-1]) * n
        a_bytes = nnzb * w.block * w.block * 2 + 4 * (w.m // w.block + 1) + 4 * nnzb
        return flops, a_bytes + len(cols) * w.block * n * 2 + w.m * n * 2, "bf16"
    if w.fmt == "sddmm_bcsr":
        # every element of every stored block: 2 * nnzb * 4096 * kd; X rows of
        # block rows with blocks and Y rows of block columns with blocks once,
        # the block table and the output blocks once
        import sparse_dense_matrix_amd as S
        nnzb = info["nnzb"]
        rp = np.asarray(S.spmm_matrix_array(d["M"], S.ARRAY_ROW_PTR))
        ci = np.asarray(S.spmm_matrix_array(d["M"], S.ARRAY_COL_IDX))
        e = 2 if w.elem == "bf16" else 1
        x_rows = int(np.count_nonzero(np.diff(rp))) * w.block
        y_rows = len(np.unique(ci)) * w.block
        out_b = nnzb * w.block * w.block * (2 if w.elem == "bf16" else 4)
        flops = 2.0 * nnzb * w.block * w.block * n
        return flops, (x_rows + y_rows) * n * e + out_b + 4 * (len(rp) + nnzb), w.elem
    if w.fmt == "bcsr":
        nnzb = info["nnzb"]
        mb = w.m // w.block
        import sparse_dense_matrix_amd as S
        cols = np.unique(S.spmm_matrix_array(d["M"], S.ARRAY_COL_IDX))
        a_bytes = nnzb * w.block * w.block * 2 + 4 * (mb + 1) + 4 * nnzb
        b_bytes = len(cols) * w.block * n * 2
        c_bytes = w.m * n * 2
        return flops, a_bytes + b_bytes + c_bytes, "bf16"
    if w.fmt == "wcsr":
        nnz = info["nnz"]
        touched = len(np.unique(d["a"]["col_idx"]))
        a_bytes = 8 * (w.m + 1) + 8 * nnz
        return flops, a_bytes + touched * n * 4 + w.m * n * 4, "f32"
    if w.fmt == "sddmm":
        # row_ptr, col_idx and out once; each X row with entries and each
        # touched Y row once (n is the inner dimension kd)
        nnz = info["nnz"]
        e, eo, dt = {"bf16": (2, 2, "bf16"), "i8": (1, 4, "i8")}.get(w.elem, (4, 4, "f32"))
        x_rows = int(np.count_nonzero(np.diff(d["a"]["row_ptr"])))
        y_rows = len(np.unique(d["a"]["col_idx"]))
        return flops, 8 * (w.m + 1) + (4 + eo) * nnz + (x_rows + y_rows) * n * e, dt
    if w.fmt == "slide":
        # effective work counts the kept (2N-2)/2N of A; bytes: the lifted 2:4
        # operand (values and index bytes), B and C once
        kept = w.m * w.k * (w.nm_group - 2) // w.nm_group
        lifted = info["nnz"]                     # m * k_lift / 2 kept values
        return 2.0 * kept * n, lifted + lifted // 4 + w.k * n + w.m * n * 4, "i8"
    if w.fmt == "tvw":
        # the stored tiles (kept values and index bytes), the B rows of
        # k-steps any tile row stores, C once
        import sparse_dense_matrix_amd as S
        e, ec = (2, 2) if w.elem == "bf16" else (1, 4)
        steps = np.unique(S.spmm_matrix_array(d["M"], S.ARRAY_COL_IDX))
        a_bytes = info["nnz"] * e + info["nnz"] // 4 + 4 * (w.m // synth_tile_m() + 1 + info["nnzb"])
        return (flops, a_bytes + len(steps) * synth_tile_k() * n * e + w.m * n * ec,
                "bf16" if w.elem == "bf16" else "i8")
    e, ec = (2, 2) if w.elem == "bf16" else (1, 4)
    a_bytes = w.m * w.k // 2 * e + w.m * w.k // 8
    return flops, a_bytes + w.k * n * e + w.m * n * ec, "bf16" if w.elem == "bf16" else "i8"


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU: the multiply shards by columns "
                                   "of B with no communication, but only the one-GPU path is "
                                   "built and measured; run with --gpus 1"}), flush=True)
        sys.exit(2)
    import torch
    import synth
    import sparse_dense_matrix_amd as S
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch, args)
        return
    cat = dict(synth.WORKLOADS)
    cat.update(synth.SMALL)
    if args.workload not in cat:
        log(f"unknown workload {args.workload}; choose from {sorted(cat)}")
        sys.exit(2)
    w = cat[args.workload]
    log(f"workload {w.describe}")
    d = setup(w, S, args)
    log(f"generated in {d['t_gen']:.1f}s, packed in {d['t_pack']:.2f}s, planned in {d['t_plan']:.2f}s")

    # device operands
    if w.fmt in ("sddmm", "sddmm_bcsr"):
        Xh, Yh = d["B"]
        if Xh.dtype == np.uint16:
            Xh, Yh = Xh.view(np.int16), Yh.view(np.int16)
        Xt = torch.from_numpy(Xh).cuda()
        Yt = torch.from_numpy(Yh).cuda()
        if w.fmt == "sddmm":
            odt = {"bf16": torch.int16, "i8": torch.int32}.get(w.elem, torch.float32)
            Ot = torch.empty(max(d["info"]["nnz"], 1), dtype=odt, device="cuda")
        else:
            odt = torch.int16 if w.elem == "bf16" else torch.int32
            Ot = torch.empty((max(d["info"]["nnzb"], 1), w.block, w.block), dtype=odt, device="cuda")

        def step(stream):
            S.spmm_execute_sddmm(d["P"], Xt, Yt, Ot, stream=stream)
    else:
        B = d["B"]
        Bh = torch.from_numpy(B.view(np.int16) if B.dtype == np.uint16 else B)
        Bt = Bh.cuda()
        cdt = {"bcsr": torch.int16, "bcsr_csr": torch.int16, "wcsr": torch.float32,
               "sp24": torch.int32, "tvw": torch.int32, "slide": torch.int32}[w.fmt]
        if w.fmt in ("tvw", "sp24") and w.elem == "bf16":
            cdt = torch.int16
        Ct = torch.empty((w.m, w.n), dtype=cdt, device="cuda")

        def step(stream):
            S.spmm_execute(d["P"], Bt, Ct, stream=stream)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    graph = None
    if args.graph > 0:
        # the same launches, recorded once: replaying G steps costs one graph
        # launch instead of G calls from Python
        args.steps = -(-args.steps // args.graph) * args.graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(args.graph):
                step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        with torch.cuda.stream(stream):
            for _ in range(args.steps // args.graph):
                graph.replay()
    else:
        for _ in range(args.steps):
            step(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    log(f"{args.steps} steps: {ms_total:.3f} ms on the stream, {wall * 1e3:.3f} ms wall")

    flops, nbytes, dtype = algorithmic(w, d)
    gflops = flops / (ms_step * 1e-3) / 1e9
    pinfo = S.spmm_plan_info(d["P"])
    kernel = dominant_kernel(w, pinfo)
    roof, other = roofline(w, kernel, flops, nbytes, dtype, ms_step)

    cold = None
    if args.cold_steps > 0:
        # each launch timed on its own after a 512 MB fill on the same stream,
        # which leaves no operand in L2 or the Infinity Cache
        flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        with torch.cuda.stream(stream):
            for i, (e0, e1) in enumerate(evs):
                flush.fill_(float(i))
                e0.record(stream)
                step(stream)
                e1.record(stream)
        torch.cuda.synchronize()
        times = np.array(sorted(e0.elapsed_time(e1) for e0, e1 in evs))
        ms_cold = float(np.median(times))
        roof_c, other_c = roofline(w, kernel, flops, nbytes, dtype, ms_cold)
        cold = {"launches": args.cold_steps, "ms_median": round(ms_cold, 6),
                "ms_min": round(float(times[0]), 6), "ms_max": round(float(times[-1]), 6),
                "ms_stdev": round(float(times.std(ddof=1)) if len(times) > 1 else 0.0, 6),
                "value": round(flops / (ms_cold * 1e-3) / 1e9, 1), "roofline": roof_c,
                "roofline_other_bound": other_c,
                "what": "each launch alone after a 512 MB fill on the same stream (L2 and "
                        "Infinity Cache hold no operand); median over the launches"}
        log(f"cold: median {ms_cold:.4f} ms over {args.cold_steps} launches "
            f"(min {times[0]:.4f}, max {times[-1]:.4f})")
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, args.cpu_seconds)
    dense = None
    if args.dense_baseline and (w.fmt == "bcsr" or (w.fmt in ("tvw", "sp24") and w.elem == "bf16")):
        dense = dense_baseline(torch, w, d, Bt, stream, args, ms_step)
    elif args.dense_baseline and w.fmt in ("tvw", "sp24", "slide"):
        dense = dense_baseline_i8(torch, w, d, Bt, stream, args, ms_step)

    out = {
        "metric": METRIC,
        "value": round(gflops, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded; shapes and sparsity of the pages' workloads)",
        "config": {"workload": w.name, "format": w.fmt, "m": w.m, "k": w.k, "n": w.n,
                   "nnz": d["info"]["nnz"], "nnzb": d["info"]["nnzb"],
                   "num_chunks": d["info"]["num_chunks"],
                   "window_rows": d["info"]["window_rows"],
                   "max_chunk_nnz": d["info"]["max_chunk_nnz"],
                   "split_rows": pinfo["num_split_rows"], "grid": pinfo["grid"],
                   "tile_m": pinfo["tile_m"], "tile_n": pinfo["tile_n"], "kernel": kernel,
                   **({"csr_nnz": int(d["a"]["row_ptr"][-1]), "reordered": w.reorder,
                       "scramble_seed": w.scramble} if w.scramble else {}),
                   "launch": (f"HIP graph of {args.graph} steps, replayed" if args.graph
                              else "one spmm_execute call per step"),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_other_bound": other,
        "algorithmic": {"flops": flops, "bytes": int(nbytes)},
        "one_time_s": {"generate": round(d["t_gen"], 3), "pack": round(d["t_pack"], 3),
                       "plan": round(d["t_plan"], 3)},
        "cpu_baseline": cpu,
    }
    if dense is not None:
        out["dense_baseline"] = dense
    if cold is not None:
        out["cold"] = cold
    print(json.dumps(out), flush=True)


def library_digest() -> str:
    """sha256 (first 16 hex digits) over every library source file: traffic
    counters taken with another digest no longer describe the library as built."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from profiles/hbm_traffic.md for (workload,
    kernel), or None when absent or recorded for another library digest."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    digest = library_digest()
    with open(TRAFFIC_TABLE) as f:
        for line in f:
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) >= 7 and cells[0] == workload and cells[1] == kernel:
                if cells[2] != digest:
                    return None
                try:
                    return int(float(cells[6]))
                except ValueError:
                    return None
    return None


def dense_baseline(torch, w, d, Bt, stream, args, ms_sparse):
    """Time the dense bf16 product of the same shape (the zero-filled A times
    B, torch.matmul) on the same stream; a comparison point, not part of the
    library."""
    A = torch.from_numpy(d["a"]["dense"].view(np.int16)).cuda().view(torch.bfloat16)
    B = Bt.view(torch.bfloat16)
    C = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(max(2, args.warmup)):
            torch.matmul(A, B, out=C)
    torch.cuda.synchronize()
    steps = max(5, args.steps // 4)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(steps):
            torch.matmul(A, B, out=C)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    flops = 2.0 * w.m * w.k * w.n
    log(f"dense bf16 product of the same shape: {ms:.3f} ms")
    return {"ms_per_step": round(ms, 6), "tflops_dense": round(flops / (ms * 1e-3) / 1e12, 2),
            "sparse_speedup": round(ms / ms_sparse, 3), "steps": steps,
            "what": "torch.matmul on the zero-filled bf16 A, same B, bf16 C"}


def dense_baseline_i8(torch, w, d, Bt, stream, args, ms_sparse):
    """Time the dense int8 product of the same shape (torch._int_mm on the
    unpruned A) on the same stream; a comparison point, not part of the
    library.  None when this torch build has no int8 matrix product."""
    if not hasattr(torch, "_int_mm"):
        return None
    A = torch.from_numpy(d["a"]["dense"]).cuda()
    C = torch.empty((w.m, w.n), dtype=torch.int32, device="cuda")
    try:
        with torch.cuda.stream(stream):
            for _ in range(max(2, args.warmup)):
                torch._int_mm(A, Bt, out=C)
        torch.cuda.synchronize()
    except (RuntimeError, TypeError) as e:
        log(f"dense int8 product unavailable: {e}")
        return None
    steps = max(5, args.steps // 4)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(steps):
            torch._int_mm(A, Bt, out=C)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    ops = 2.0 * w.m * w.k * w.n
    log(f"dense int8 product of the same shape: {ms:.3f} ms")
    return {"ms_per_step": round(ms, 6), "tops_dense": round(ops / (ms * 1e-3) / 1e12, 2),
            "sparse_speedup": round(ms / ms_sparse, 3), "steps": steps,
            "what": "torch._int_mm on the unpruned int8 A, same B, int32 C"}


def roofline(w, kernel, flops, nbytes, dtype, ms_step):
    """(roofline of the binding bound, the other bound).  The binding bound is
    the one whose time at peak is longer; `kernel` is the step's dominant
    kernel, whose counters give `traffic`."""
    t = ms_step * 1e-3
    traffic = measured_traffic(w.name, kernel)
    hbm = {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": PEAK_HBM_GBS,
           "unit": "GB/s", "frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
           "traffic": traffic}
    if traffic is not None:
        hbm["traffic_GB_s"] = round(traffic / t / 1e9, 1)
    if dtype not in PEAK_MFMA_TFLOPS:
        return hbm, None
    peak = PEAK_MFMA_TFLOPS[dtype]
    mfma = {"bound": "mfma", "achieved": round(flops / t / 1e12, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / peak, 4), "traffic": traffic}
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (peak * 1e12)
    return (hbm, mfma) if t_hbm >= t_mfma else (mfma, hbm)


def copy_calibration(torch, args):
    """A plain elementwise copy kernel over 1 GiB of float32 (reads 1 GiB,
    writes 1 GiB): what FETCH_SIZE / WRITE_SIZE read for it scales the
    counters of the SpMM kernels to bytes."""
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(args.warmup + args.steps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                                           "launches": args.warmup + args.steps}}), flush=True)


def short_kernel_name(name: str) -> str:
    """Bare function name of a demangled kernel signature: no return type,
    namespaces, template arguments or parameters."""
    name = name.replace("(anonymous namespace)::", "")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):          # end of the name: first '<' or '(' at depth 0
        if ch in "<(" and depth == 0:
            cut = i
            break
    return name[:cut].split("::")[-1].split(" ")[-1]


def trace_summary(root):
    """Per-kernel call count and duration statistics (microseconds) from the
    rocprofv3 kernel-trace databases under root."""
    import collections
    import sqlite3
    durs = collections.defaultdict(list)
    for dirpath, _, files in os.walk(root):
        for fn in files:
            if not fn.endswith("_results.db"):
                continue
            con = sqlite3.connect(os.path.join(dirpath, fn))
            for name, dur in con.execute("select name, duration from kernels"):
                durs[short_kernel_name(name)].append(dur / 1000.0)
            con.close()
    print("| kernel | calls | avg us | median us | min us | max us | total ms |")
    print("|---|---|---|---|---|---|---|")
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        print(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | {v[0]:.2f} | "
              f"{v[-1]:.2f} | {sum(v) / 1000:.3f} |")


def pmc_summary(root):
    """Mean per dispatch of each counter, per kernel, over rocprofv3 CSVs."""
    import collections
    import csv
    agg = collections.defaultdict(list)
    for dirpath, _, files in os.walk(root):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(dirpath, fn)) as f:
                for r in csv.DictReader(f):
                    name = short_kernel_name(r["Kernel_Name"])
                    agg[(name, r["Counter_Name"])].append(float(r["Counter_Value"]))
    print(f"library digest {library_digest()}")
    for (k, c), v in sorted(agg.items()):
        print(f"{k:32s} {c:32s} dispatches={len(v):4d} mean={sum(v) / len(v):.6g}")


def synth_tile_m():
    import synth
    return synth.TVW_TILE_M


def synth_tile_k():
    import synth
    return synth.TVW_TILE_K


def synth_f32(B):
    """B as float32 for the CSR oracle (bf16 bit patterns widen exactly)."""
    import synth
    return synth.bf16_bits_to_f32(B) if B.dtype == np.uint16 else B


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, d, target_s):
    """Time the oracle on a growing sample of rows until it takes about
    target_s; report effective GFLOP/s over the sampled rows."""
    import oracle
    a, B = d["a"], d["B"]
    r = np.random.default_rng(0)
    if w.fmt == "bcsr":
        rp, ci, v = oracle.pack_bcsr(a["dense"], w.block, w.block)
        row_nnz = np.repeat(np.diff(rp).astype(np.int64) * w.block, w.block)

        def run(rows):
            oracle.bcsr_spmm(w.block, w.block, rp, ci, v, B, rows=rows)
    elif w.fmt in ("wcsr", "bcsr_csr"):
        row_nnz = np.diff(a["row_ptr"])
        Bf = synth_f32(B)

        def run(rows):
            oracle.csr_spmm(a["row_ptr"], a["col_idx"], a["vals"], Bf, rows=rows)
    elif w.fmt == "sddmm":
        row_nnz = np.diff(a["row_ptr"])
        # the oracle takes the operands' exact fp32 images
        Xf, Yf = (synth_f32(B[0]), synth_f32(B[1])) if w.elem == "bf16" else (
            (B[0].astype(np.float32), B[1].astype(np.float32)) if w.elem == "i8" else B)

        def run(rows):
            oracle.sddmm(a["row_ptr"], a["col_idx"], Xf, Yf, rows=rows)
    elif w.fmt == "slide":
        pruned = oracle.prune_nm(a["dense"], w.nm_group - 2, w.nm_group)
        row_nnz = np.full(w.m, w.k * (w.nm_group - 2) // w.nm_group, dtype=np.int64)

        def run(rows):
            oracle.gemm_i8(pruned[rows], B)
    elif w.fmt == "sddmm_bcsr":
        # the sample unit is a stored block (2 * 4096 * kd flop each)
        rp, ci, _ = oracle.pack_bcsr(a["dense"], w.block, w.block)
        units = len(ci)
        perm = r.permutation(units).astype(np.int64)
        count, spent = 1, 0.0
        while True:
            blocks = np.sort(perm[:count])
            t0 = time.perf_counter()
            oracle.sddmm_bcsr(w.block, w.block, rp, ci, B[0], B[1], blocks=blocks)
            spent = time.perf_counter() - t0
            if spent >= target_s or count >= units:
                break
            count = min(units, int(count * max(2.0, min(8.0, 0.9 * target_s / max(spent, 1e-3)))))
        flops = 2.0 * count * w.block * w.block * w.n
        log(f"cpu oracle: {count} blocks in {spent:.2f}s on {oracle.num_threads()} threads")
        return {"value": round(flops / spent / 1e9, 3), "unit": "GFLOP/s",
                "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                "sample": f"{count} of {units} stored blocks (uniform without replacement, "
                          f"seed 0), full inner dimension {w.n}; "
                          + ("fp64" if w.elem == "bf16" else "int64") + " accumulation"}
    elif w.fmt in ("tvw", "sp24") and w.elem == "bf16":
        # the oracle's 2:4 pruning, then its BCSR product over tiles of
        # 256 x 128 (every element of a stored tile, pruned or not, is walked)
        pruned = oracle.prune_nm(a["dense"], 2, 4)
        tm, tk = synth_tile_m(), synth_tile_k()
        rp, ci, v = oracle.pack_bcsr(pruned, tm, tk)
        row_nnz = np.repeat(np.diff(rp).astype(np.int64) * (tk // 2), tm)

        def run(rows):
            oracle.bcsr_spmm(tm, tk, rp, ci, v, B, rows=rows)
    else:
        vals, meta = oracle.pack24(a["dense"])
        # kept values per row: all k/2 for 2:4; for the tile pattern the kept
        # values of the stored tiles only (the oracle still walks every group)
        if w.fmt == "tvw":
            import sparse_dense_matrix_amd as S
            rp = S.spmm_matrix_array(d["M"], S.ARRAY_ROW_PTR).astype(np.int64)
            row_nnz = np.repeat(np.diff(rp) * (synth_tile_k() // 2), synth_tile_m())
        else:
            row_nnz = np.full(w.m, w.k // 2, dtype=np.int64)

        def run(rows):
            oracle.sp24_spmm(vals, meta, B, rows=rows)
    perm = r.permutation(w.m).astype(np.int64)
    count, spent, rows = 8, 0.0, None
    while True:
        rows = np.sort(perm[:count])
        t0 = time.perf_counter()
        run(rows)
        spent = time.perf_counter() - t0
        if spent >= target_s or count >= w.m:
            break
        grow = max(2.0, min(8.0, 0.9 * target_s / max(spent, 1e-3)))
        count = min(w.m, int(count * grow))
    flops = 2.0 * float(row_nnz[rows].sum()) * w.n
    log(f"cpu oracle: {len(rows)} rows in {spent:.2f}s on {oracle.num_threads()} threads")
    return {"value": round(flops / spent / 1e9, 3), "unit": "GFLOP/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{len(rows)} of {w.m} rows (uniform without replacement, seed 0), "
                      + ("all their stored entries" if w.fmt == "sddmm" else f"all {w.n} columns")
                      + "; fp64 accumulation"}


if __name__ == "__main__":
    main()
