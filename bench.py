"""Benchmark of the software-pipelined tiled fp16 GEMM (headline: M=N=K=4096)
and the pipelined streaming add (z = x + y over 8192 x 8192 fp32) on one
MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]

A step is one GEMM launch at 4096^3 on inputs already resident in HBM.  The
timed region is exactly K steps on one stream after W untimed warm-up
steps, bracketed by device synchronisation and timed with HIP events
recorded on that stream.  Prints one JSON line.

Order of the run.  Every input of every leg is generated and copied to the
device first, so that no host work leaves the GPU idle between the legs.
Then:
  1. cold_start: the 4096^3 GEMM, W + K launches, the first GPU work of the
     process.  MI355X runs at its 1400 W power cap under this GEMM; after
     idle its power controller first lets the clock run, then throttles
     hard for about 10 ms before it settles (per-launch durations of
     100 -> 130 -> 98 us), so a short run here times that transient.
  2. the secondary legs (streaming add at the default and at the pages'
     512 x 512 blocks, x + 1, the reduction, the other GEMM configurations,
     and torch.matmul on the GEMM operands for context),
     each after a settle phase of back-to-back launches lasting at least
     --settle-ms, then W warm-up and K timed launches of its own;
  3. the headline: W warm-up and K timed launches of the 4096^3 GEMM,
     right after the 8192^3 leg, i.e. at the sustained clock of a busy GPU.
`value` is (3); the cold figure is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOP/s (% of MFMA peak) at 4096³; streaming add GB/s (% HBM)"
# MI355X published dense figures: fp16 MFMA 2.5 PFLOP/s (256 CU x 4096 flop/clk
# x 2.4 GHz = 2516.6 TFLOP/s), HBM3E 8 TB/s.
PEAK_FP16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="back-to-back launches before each secondary leg's warm-up")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--quick", action="store_true", help="headline GEMM only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the headline oracle sample")
    ap.add_argument("--profile", action="store_true",
                    help="no timing: a 512 MiB device copy (counter calibration) followed by "
                         "launches of each kernel, for rocprofv3 runs")
    ap.add_argument("--profile-reps", type=int, default=3,
                    help="launches of each kernel in --profile mode")
    ap.add_argument("--data-dependence", action="store_true",
                    help="also time the 4096^3 and 8192^3 GEMMs on U[-1,1], normal(0,1/sqrt(K)) "
                         "and all-zero operands (same instructions, different switching power)")
    ap.add_argument("--zero-operands", action="store_true",
                    help="diagnostic: the 4096^3 legs on all-zero operands (same instructions, "
                         "no operand switching); the line then names them and is not the headline")
    ap.add_argument("--fixed-cost", action="store_true",
                    help="also time the 256x256-tile GEMM at M=N=4096 for K = 0 .. 4096 and fit "
                         "time = fixed + steps * per_step (the per-launch cost outside the K loop)")
    return ap.parse_args()


def profile_run(pg, inputs, reps):
    """Launch sequence for counter collection: one plain copy of known size
    (512 MiB read + 512 MiB written) to calibrate FETCH_SIZE / WRITE_SIZE,
    then `reps` launches each of the 4096^3 GEMM, the streaming add, x + 1,
    the (8, 4096, 4096) reduction, the 8192^3 GEMM, the 2048^2 x 32768 GEMM
    and its split-K form."""
    import torch
    src = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    A, B = inputs.gemm_inputs(4096, 4096, 4096)
    tA, tB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    tC = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
    x, y = inputs.stream_inputs((8192, 8192))
    tx, ty = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    tz = torch.empty_like(tx)
    for _ in range(reps):
        pg.pgemm_f16(tA, tB, C=tC)
    for _ in range(reps):
        pg.pstream_add(tx, ty, z=tz)
    for _ in range(reps):
        pg.pstream_add_scalar(tx, 1.0, z=tz)
    del tx, ty, tz
    xr = torch.from_numpy(inputs.uniform_f32((8, 4096, 4096), 0)).cuda()
    o = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
    for _ in range(reps):
        pg.preduce_sum_f32(xr, out=o)
    del xr, o
    for (M, N, K, dist) in [(8192, 8192, 8192, "normal"), (2048, 2048, 32768, "uniform")]:
        tA, tB, tC = gemm_operands(inputs, M, N, K, dist)
        for _ in range(reps):
            pg.pgemm_f16(tA, tB, C=tC)
    for _ in range(reps):
        pg.pgemm_f16_splitk(tA, tB, C=tC)
    torch.cuda.synchronize()
    print("profile launches done", flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiled_pgemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, src_hash):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    if there is none for this kernel or the kernel sources changed since."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def settle(fn, seconds):
    """Back-to-back launches of fn until `seconds` have passed (in batches
    of 10, synchronised); returns the number of launches."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        for i in range(10):
            fn(n + i)
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_launches(fn, steps, warmup, stream, settle_s=0.0):
    """Seconds for `steps` launches of fn after `warmup` untimed ones (and,
    before those, `settle_s` seconds of back-to-back launches)."""
    import torch
    settled = settle(fn, settle_s) if settle_s > 0 else 0
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3, settled


def gemm_operands(inputs, M, N, K, dist):
    import torch
    A, B = inputs.gemm_inputs(M, N, K, dist)
    return (torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
            torch.empty((M, N), dtype=torch.float16, device="cuda"))


def gemm_case(pg, ops, dist, steps, warmup, stream, settle_s=0.0, splitk=False):
    import torch
    tA, tB, tC = ops
    M, K = tA.shape
    N = tB.shape[1]
    rec = {"M": M, "N": N, "K": K, "dist": dist}
    if splitk:
        splits = pg.pgemm_f16_splitk_default_splits(M, N, K)
        ws = torch.empty(max(pg.pgemm_f16_splitk_workspace_bytes(M, N, K, splits) // 4, 1),
                         dtype=torch.float32, device="cuda")
        fn = lambda i: pg.pgemm_f16_splitk(tA, tB, splits, C=tC, workspace=ws)
        rec["path"] = "pgemm_f16_splitk, %d splits, %d MiB fp32 workspace" % (
            splits, ws.numel() * 4 >> 20)
    else:
        fn = lambda i: pg.pgemm_f16(tA, tB, C=tC)
        rec["path"] = "pgemm_f16 (variant %d)" % pg.pgemm_f16_choose_variant(M, N, K)
    secs, settled = time_launches(fn, steps, warmup, stream, settle_s)
    tflops = 2.0 * M * N * K * steps / secs / 1e12
    rec.update({"us_per_launch": secs / steps * 1e6, "tflops": tflops,
                "frac_of_peak": tflops / PEAK_FP16_TFLOPS, "settle_launches": settled,
                "warmup": warmup, "steps": steps})
    return rec


def vendor_case(ops, dist, steps, warmup, stream, settle_s):
    """torch.matmul on the same fp16 operands, for context."""
    import torch
    tA, tB, tC = ops
    M, K = tA.shape
    N = tB.shape[1]
    secs, _ = time_launches(lambda i: torch.matmul(tA, tB, out=tC), steps, warmup, stream, settle_s)
    tflops = 2.0 * M * N * K * steps / secs / 1e12
    return {"M": M, "N": N, "K": K, "dist": dist, "us_per_launch": round(secs / steps * 1e6, 2),
            "tflops": round(tflops, 1)}


def stream_case(pg, sets, steps, warmup, stream, settle_s, kind, block=None):
    n = sets[0][0].numel()
    if kind == "scalar":
        fn = lambda i: pg.pstream_add_scalar(sets[i % 3][0], 1.0, z=sets[i % 3][2])
        bytes_per = 8.0 * n
    elif block is not None:
        fn = lambda i: pg.pstream_add_blocked(sets[i % 3][0], sets[i % 3][1], block,
                                              z=sets[i % 3][2])
        bytes_per = 12.0 * n
    else:
        fn = lambda i: pg.pstream_add(sets[i % 3][0], sets[i % 3][1], z=sets[i % 3][2])
        bytes_per = 12.0 * n
    secs, settled = time_launches(fn, steps, warmup, stream, settle_s)
    gbs = bytes_per * steps / secs / 1e9
    return {"bytes_per_launch": bytes_per, "us_per_launch": round(secs / steps * 1e6, 2),
            "value": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "settle_launches": settled}


def reduce_case(pg, sets, out, steps, warmup, stream, settle_s):
    """The guide's section 7.2 reduction at (8, 4096, 4096) f32: 8 slices of
    64 MiB summed over the first axis; 9 * 64 MiB move per launch."""
    R, M, N = sets[0].shape
    secs, settled = time_launches(lambda i: pg.preduce_sum_f32(sets[i % 2], out=out), steps,
                                  warmup, stream, settle_s)
    bytes_per = 4.0 * (R + 1) * M * N
    gbs = bytes_per * steps / secs / 1e9
    return {"workload": "sum over axis 0 of (8, 4096, 4096) f32, U[-1,1], 2 rotating inputs",
            "value": round(gbs, 1), "unit": "GB/s", "us_per_launch": round(secs / steps * 1e6, 2),
            "settle_launches": settled,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("sum_axis0_vec_kernel", kernel_source_hash())}}


def fixed_cost(pg, inputs, stream, settle_s):
    """Per-launch time of the 4096^3 headline kernel (variant 8) at M=N=4096
    for several K, and a least-squares line time = fixed + steps * per_step
    over K >= 512 (steps = K / 32).  K = 0 runs the launch and the drain of
    a zero tile only."""
    import torch
    M = N = 4096
    A, B = inputs.gemm_inputs(M, N, 4096)
    tA, tB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    tC = torch.empty((M, N), dtype=torch.float16, device="cuda")
    pts = []
    for K in (0, 256, 512, 1024, 2048, 4096):
        a = tA[:, :K].contiguous() if K < 4096 else tA
        b = tB[:K].contiguous()
        fn = lambda i: pg.pgemm_f16_variant(a, b, 8, C=tC)
        reps = 400 if K <= 1024 else 200
        secs, _ = time_launches(fn, reps, 20, stream, settle_s)
        pts.append((K, secs / reps * 1e6))
    fit = [(K // 32, t) for K, t in pts if K >= 512]
    n = len(fit)
    sx = sum(x for x, _ in fit); sy = sum(y for _, y in fit)
    sxx = sum(x * x for x, _ in fit); sxy = sum(x * y for x, y in fit)
    slope = (n * sxy - sx * sy) / (n * sxx - sx * sx)
    icpt = (sy - slope * sx) / n
    return {"workload": "pgemm_f16_variant 8, M=N=4096, K from 0 to 4096",
            "us_per_launch": {str(K): round(t, 2) for K, t in pts},
            "fit_K_ge_512": {"fixed_us": round(icpt, 2), "us_per_K_step_of_32": round(slope, 4)}}


def data_dependence(pg, inputs, stream, settle_s, steps, warmup):
    """The same GEMM launches on three operand distributions, interleaved
    over 3 rounds (median): the kernel executes the same instructions on
    all of them, so differences come from the chip's power limit reacting
    to how much the operands switch."""
    import torch
    res = []
    for (M, N, K) in [(4096, 4096, 4096), (8192, 8192, 8192)]:
        ops = {}
        for dist in ("uniform", "normal"):
            A, B = inputs.gemm_inputs(M, N, K, dist)
            ops[dist] = (torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
        ops["zeros"] = (torch.zeros((M, K), dtype=torch.float16, device="cuda"),
                        torch.zeros((K, N), dtype=torch.float16, device="cuda"))
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        reps = max(5, steps if M == 4096 else steps // 8)
        t = {d: [] for d in ops}
        for _ in range(3):
            for d, (a, b) in ops.items():
                secs, _ = time_launches(lambda i: pg.pgemm_f16(a, b, C=C), reps, warmup, stream,
                                        settle_s)
                t[d].append(secs / reps)
        for d in ops:
            us = sorted(t[d])[1] * 1e6
            tf = 2.0 * M * N * K / us / 1e6
            res.append({"M": M, "N": N, "K": K, "operands": d, "us_per_launch": round(us, 2),
                        "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_FP16_TFLOPS, 4)})
        del ops, C
    return res


# ------------------------------------------------------------------ CPU baselines

def _oracle_points_rate(oracle, A, B, I, J):
    """(seconds, multiply-adds per second, (C, S)) of the oracle on sampled
    outputs."""
    K = A.shape[1]
    t0 = time.perf_counter()
    ref = oracle.gemm_f16_points(A, B, I, J)
    t = time.perf_counter() - t0
    return t, I.size * K / t, ref


def accuracy(workload, got, ref):
    """The GPU's outputs `got` (fp16) against the oracle's correctly rounded
    values and exact binary64 sums `ref` = (C, S) on the same outputs."""
    import numpy as np
    ref_c, ref_s = ref
    g = got.astype(np.float64)
    r = ref_c.astype(np.float64)
    err = np.abs(g - r)
    scaled = err / (np.abs(r) + 1.0)
    return {"workload": workload, "outputs": int(got.size),
            "max_abs_err": float(err.max()), "mean_abs_err": float(err.mean()),
            "max_scaled_err": float(scaled.max()),
            "frac_exact": round(float(np.mean(got.view(np.uint16) == ref_c.view(np.uint16))), 6),
            "rel_frobenius_vs_exact_sums": float(np.linalg.norm(g - ref_s) / np.linalg.norm(ref_s)),
            "tolerance": "|gpu - oracle| <= 5e-3 * (|oracle| + 1)",
            "within_tolerance": bool(scaled.max() <= 5e-3)}


def cpu_baseline(inputs, target_seconds, gpu_C=None):
    """The oracle (plain binary64 triple loop, all host threads) timed on a
    bounded sample of the headline workload: the first R full rows of the
    4096^3 product, R chosen so the run takes about `target_seconds`.
    Returns (baseline, accuracy of gpu_C on those rows or None)."""
    import numpy as np

    import oracle
    M = N = K = 4096
    A, B = inputs.gemm_inputs(M, N, K)
    cores = oracle.threads()

    def run(rows):
        I = np.repeat(np.arange(rows, dtype=np.int64), N)
        J = np.tile(np.arange(N, dtype=np.int64), rows)
        t0 = time.perf_counter()
        ref = oracle.gemm_f16_points(A, B, I, J)
        return time.perf_counter() - t0, ref

    rows = 4
    t, _ = run(rows)
    rows = int(max(4, min(M, rows * target_seconds / max(t, 1e-3))))
    t, ref = run(rows)
    flops = 2.0 * rows * N * K
    acc = None
    if gpu_C is not None:
        acc = accuracy("GEMM 4096^3 uniform (pgemm_f16), first %d rows" % rows,
                       gpu_C[:rows].reshape(-1), ref)
    return ({"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
             "sample": "first %d of 4096 rows of the 4096^3 fp16 GEMM (%.1f s, %d threads)"
                       % (rows, t, cores)}, acc)


def cpu_baselines_other(inputs, gpu_out=None):
    """The oracle on the other configurations: 256^3 in full on one thread
    and on all threads; 8192^3 and 2048^2 x 32768 on the deterministic
    output sample the parity tests use (32 rows, 32 columns, 8192 points,
    the corners of every 128-tile), extrapolated to the whole product by the
    per-output time and labelled as such; the streaming add on the full
    8192^2 workload on one thread and on all threads.  Returns (baselines,
    accuracy of the GPU outputs gpu_out[(M, N, K)] on those samples)."""
    import oracle
    allc = oracle.threads()
    out = []
    accs = []
    A, B = inputs.gemm_inputs(256, 256, 256)
    for th in (1, allc):
        oracle.set_threads(th)
        oracle.gemm_f16(A, B)  # first call builds the decode table
        t0 = time.perf_counter()
        oracle.gemm_f16(A, B)
        t = time.perf_counter() - t0
        out.append({"workload": "GEMM 256^3, full product", "value": 2.0 * 256 ** 3 / t / 1e12,
                    "unit": "TFLOP/s", "seconds": t, "cores": th, "kind": "oracle"})
    oracle.set_threads(allc)
    for (M, N, K, dist) in [(8192, 8192, 8192, "normal"), (2048, 2048, 32768, "uniform")]:
        A, B = inputs.gemm_inputs(M, N, K, dist)
        I, J = inputs.sample_points(M, N, 8192)
        t, rate, ref = _oracle_points_rate(oracle, A, B, I, J)
        if gpu_out is not None and (M, N, K) in gpu_out:
            accs.append(accuracy("GEMM %dx%dx%d %s (pgemm_f16), sampled outputs" % (M, N, K, dist),
                                 gpu_out[(M, N, K)][I, J], ref))
        full = M * N * K / rate
        out.append({"workload": "GEMM %dx%dx%d %s" % (M, N, K, dist),
                    "value": 2.0 * rate / 1e12, "unit": "TFLOP/s", "cores": allc, "kind": "oracle",
                    "sample": "%d sampled outputs in %.2f s" % (I.size, t),
                    "extrapolated_full_seconds": round(full, 1),
                    "note": "extrapolated from the sample by time per output"})
    x, y = inputs.stream_inputs((8192, 8192))
    for th in (1, allc):
        oracle.set_threads(th)
        oracle.add_f32(x, y)
        t0 = time.perf_counter()
        for _ in range(3):
            oracle.add_f32(x, y)
        t = (time.perf_counter() - t0) / 3
        out.append({"workload": "streaming add 8192^2 fp32, full", "value": round(12.0 * x.size / t / 1e9, 2),
                    "unit": "GB/s", "seconds": t, "cores": th, "kind": "oracle"})
    oracle.set_threads(allc)
    for r in out:
        for k, v in list(r.items()):
            if isinstance(v, float):
                r[k] = round(v, 6)
    return out, accs


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import software_pipelined_tiled_pgemm_amd as pg
    from software_pipelined_tiled_pgemm_amd import inputs

    if not os.path.exists(os.path.join(ROOT, "software_pipelined_tiled_pgemm_amd", "libpgemm.so")):
        from software_pipelined_tiled_pgemm_amd import build as _b
        _b.build()
    if not torch.cuda.is_available():
        print("no HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.profile:
        profile_run(pg, inputs, args.profile_reps)
        return
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    print("device: %s, %d CUs; assumed peaks: fp16 MFMA %.1f TFLOP/s, HBM %.0f GB/s"
          % (props.name, props.multi_processor_count, PEAK_FP16_TFLOPS, PEAK_HBM_GBS),
          file=sys.stderr, flush=True)
    W, K = args.warmup, args.steps
    settle_s = args.settle_ms / 1e3

    # Every input on the device before the first timed leg.
    head_ops = gemm_operands(inputs, 4096, 4096, 4096, "uniform")
    if args.zero_operands:  # diagnostic only: no oracle leg on these operands
        head_ops = (torch.zeros_like(head_ops[0]), torch.zeros_like(head_ops[1]), head_ops[2])
        args.no_cpu = True
    if not args.quick:
        x, y = inputs.stream_inputs((8192, 8192))
        sets = [(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda(),
                 torch.empty(x.size, dtype=torch.float32, device="cuda")) for _ in range(3)]
        sets = [(a.view(-1), b.view(-1), c) for a, b, c in sets]
        del x, y
        red_sets = [torch.from_numpy(inputs.uniform_f32((8, 4096, 4096), s)).cuda() for s in (0, 1)]
        red_out = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
        other_ops = [(M, N, Kk, dist, gemm_operands(inputs, M, N, Kk, dist))
                     for (M, N, Kk, dist) in [(256, 256, 256, "uniform"),
                                              (2048, 2048, 32768, "uniform"),
                                              (8192, 8192, 8192, "normal")]]
    torch.cuda.synchronize()

    cold = gemm_case(pg, head_ops, "uniform", K, W, stream)
    print("gemm 4096^3, cold start: %.1f us, %.1f TFLOP/s" % (cold["us_per_launch"], cold["tflops"]),
          file=sys.stderr, flush=True)

    out_extra = {}
    if not args.quick:
        add = stream_case(pg, sets, K, W, stream, settle_s, "add")
        add512 = stream_case(pg, sets, K, W, stream, settle_s, "add", block=512 * 512)
        addc = stream_case(pg, sets, K, W, stream, settle_s, "scalar")
        print("stream add: %.1f GB/s (512x512 blocks %.1f); x+1: %.1f GB/s"
              % (add["value"], add512["value"], addc["value"]), file=sys.stderr, flush=True)
        src_hash = kernel_source_hash()
        out_extra["streaming"] = {
            "workload": "z = x + y, fp32 8192x8192, U[-1,1], 3 rotating buffer sets",
            "value": add["value"], "unit": "GB/s", "us_per_launch": add["us_per_launch"],
            "block_elems": 4096, "settle_launches": add["settle_launches"],
            "roofline": {"bound": "hbm", "achieved": add["value"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": add["frac"],
                         "traffic": measured_traffic("add_vec_kernel", src_hash)},
            "blocks_512x512": {"value": add512["value"], "unit": "GB/s",
                               "us_per_launch": add512["us_per_launch"], "frac": add512["frac"],
                               "block_elems": 512 * 512,
                               "note": "pstream_add_blocked with the pages' 512x512 blocks"},
            "x_plus_1": {"value": addc["value"], "unit": "GB/s",
                         "us_per_launch": addc["us_per_launch"], "frac": addc["frac"]},
        }
        out_extra["reduction"] = reduce_case(pg, red_sets, red_out, K, W, stream, settle_s)
        print("reduction: %.1f GB/s" % out_extra["reduction"]["value"], file=sys.stderr, flush=True)
        del sets, red_sets, red_out
        others = []
        vendor = []
        for (M, N, Kk, dist, ops) in [(4096, 4096, 4096, "uniform", head_ops)] + other_ops[1:]:
            vendor.append(vendor_case(ops, dist, K, W, stream, settle_s))
        out_extra["vendor_context"] = {
            "note": "torch.matmul (PyTorch-ROCm's fp16 GEMM, hipBLASLt) on the same device operands, "
                    "timed the same way; context only, not part of the path",
            "runs": vendor}
        for (M, N, Kk, dist, ops) in other_ops:
            r = gemm_case(pg, ops, dist, K, W, stream, settle_s)
            print("gemm %dx%dx%d: %.1f us, %.1f TFLOP/s" % (M, N, Kk, r["us_per_launch"], r["tflops"]),
                  file=sys.stderr, flush=True)
            others.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
            if (M, N, Kk) == (2048, 2048, 32768):
                # long K through split-K (the caller provides the fp32 workspace)
                r = gemm_case(pg, ops, dist, K, W, stream, settle_s, splitk=True)
                print("gemm %dx%dx%d split-K: %.1f us, %.1f TFLOP/s"
                      % (M, N, Kk, r["us_per_launch"], r["tflops"]), file=sys.stderr, flush=True)
                others.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        out_extra["other_gemm"] = others

    head = gemm_case(pg, head_ops, "uniform", K, W, stream)
    print("gemm 4096^3: %.1f us, %.1f TFLOP/s" % (head["us_per_launch"], head["tflops"]),
          file=sys.stderr, flush=True)
    traffic = measured_traffic("gemm_f16_kernel_4096", kernel_source_hash())
    out = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["us_per_launch"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "fp16 GEMM M=N=K=4096, row-major A and B, %s inputs, "
                               "fp32 accumulate, fp16 out"
                               % ("ALL-ZERO (diagnostic)" if args.zero_operands else "U[-1,1]")},
        "roofline": {"bound": "mfma", "achieved": round(head["tflops"], 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["frac_of_peak"], 4), "traffic": traffic},
        "measured_after": ("the secondary legs (GPU busy without idle gaps)" if not args.quick
                           else "the cold-start leg"),
        "cold_start": {"value": round(cold["tflops"], 2), "unit": "TFLOP/s",
                       "us_per_launch": round(cold["us_per_launch"], 2),
                       "frac": round(cold["frac_of_peak"], 4), "warmup": W, "steps": K,
                       "note": "the first W + K launches of the process, GPU idle before: "
                               "inside the power controller's transient"},
    }
    out.update(out_extra)
    if args.data_dependence:
        out["data_dependence"] = data_dependence(pg, inputs, stream, settle_s, K, W)
        for r in out["data_dependence"]:
            print("gemm %dx%dx%d on %s operands: %.1f TFLOP/s" % (r["M"], r["N"], r["K"], r["operands"],
                                                                r["tflops"]), file=sys.stderr, flush=True)
    if args.fixed_cost:
        out["fixed_cost"] = fixed_cost(pg, inputs, stream, settle_s)
        print("fixed cost: %s" % out["fixed_cost"]["fit_K_ge_512"], file=sys.stderr, flush=True)
    if not args.no_cpu:
        # The automatic path's outputs (one more untimed launch each) for the
        # oracle leg's accuracy report.
        gpu_out = {(4096, 4096, 4096): pg.pgemm_f16(head_ops[0], head_ops[1],
                                                    C=head_ops[2]).cpu().numpy()}
        if not args.quick:
            for (M, N, Kk, dist, ops) in other_ops:
                if M * N * Kk > 256 ** 3:
                    gpu_out[(M, N, Kk)] = pg.pgemm_f16(ops[0], ops[1], C=ops[2]).cpu().numpy()
        out["cpu_baseline"], acc = cpu_baseline(inputs, args.cpu_seconds, gpu_out[(4096, 4096, 4096)])
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
        out["accuracy"] = [acc]
        if not args.quick:
            out["cpu_baseline_other"], accs = cpu_baselines_other(inputs, gpu_out)
            out["accuracy"] += accs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
