"""Benchmark of the software-pipelined tiled fp16 GEMM (headline: M=N=K=4096)
and the pipelined streaming add (z = x + y over 8192 x 8192 fp32) on one
MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]

A step is one GEMM launch at 4096^3 on inputs already resident in HBM.  The
timed region is exactly K steps on one stream, bracketed by device
synchronisation, and timed with HIP events recorded on that stream.  The
default warm-up (300 launches) lets the clock settle: throughput rises over
the first ~200 launches of a cold process and is flat afterwards.  The
streaming kernels get their own timed regions of K launches each (rotating
over three buffer sets, so no launch re-reads what the previous one left in
the caches).  Prints one JSON line.
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
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--quick", action="store_true", help="headline GEMM only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--profile", action="store_true",
                    help="no timing: a 512 MiB device copy (counter calibration) followed by "
                         "3 launches of each kernel, for rocprofv3 runs")
    return ap.parse_args()


def profile_run(pg, inputs):
    """Launch sequence for counter collection: one plain copy of known size
    (512 MiB read + 512 MiB written) to calibrate FETCH_SIZE / WRITE_SIZE,
    then 3 launches each of the 4096^3 GEMM, the streaming add, x + 1 and the
    (8, 4096, 4096) reduction."""
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
    for _ in range(3):
        pg.pgemm_f16(tA, tB, C=tC)
    for _ in range(3):
        pg.pstream_add(tx, ty, z=tz)
    for _ in range(3):
        pg.pstream_add_scalar(tx, 1.0, z=tz)
    del tx, ty, tz
    xr = torch.from_numpy(inputs.uniform_f32((8, 4096, 4096), 0)).cuda()
    o = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
    for _ in range(3):
        pg.preduce_sum_f32(xr, out=o)
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


def time_launches(fn, steps, warmup, stream):
    import torch
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
    return start.elapsed_time(end) / 1e3  # seconds


def gemm_case(pg, inputs, M, N, K, dist, steps, warmup, stream, splitk=False):
    import torch
    A, B = inputs.gemm_inputs(M, N, K, dist)
    tA = torch.from_numpy(A).cuda()
    tB = torch.from_numpy(B).cuda()
    tC = torch.empty((M, N), dtype=torch.float16, device="cuda")
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
    secs = time_launches(fn, steps, warmup, stream)
    flops = 2.0 * M * N * K
    tflops = flops * steps / secs / 1e12
    rec.update({"us_per_launch": secs / steps * 1e6, "tflops": tflops,
                "frac_of_peak": tflops / PEAK_FP16_TFLOPS})
    return rec


def stream_case(pg, inputs, steps, warmup, stream, scalar):
    import torch
    n = 8192 * 8192
    x, y = inputs.stream_inputs((8192, 8192))
    sets = []
    for _ in range(3):
        sets.append((torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda(),
                     torch.empty(n, dtype=torch.float32, device="cuda")))
    if scalar:
        fn = lambda i: pg.pstream_add_scalar(sets[i % 3][0], 1.0, z=sets[i % 3][2])
        bytes_per = 8.0 * n
    else:
        fn = lambda i: pg.pstream_add(sets[i % 3][0], sets[i % 3][1], z=sets[i % 3][2])
        bytes_per = 12.0 * n
    secs = time_launches(fn, steps, warmup, stream)
    gbs = bytes_per * steps / secs / 1e9
    return {"n": n, "bytes_per_launch": bytes_per, "us_per_launch": secs / steps * 1e6,
            "GB/s": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS}


def reduce_case(pg, inputs, steps, warmup, stream):
    """The guide's section 7.2 reduction at (8, 4096, 4096) f32: 8 slices of
    64 MiB summed over the first axis; 9 * 64 MiB move per launch."""
    import torch
    R, M, N = 8, 4096, 4096
    sets = [torch.from_numpy(inputs.uniform_f32((R, M, N), s)).cuda() for s in (0, 1)]
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    secs = time_launches(lambda i: pg.preduce_sum_f32(sets[i % 2], out=out), steps, warmup, stream)
    bytes_per = 4.0 * (R + 1) * M * N
    gbs = bytes_per * steps / secs / 1e9
    return {"workload": "sum over axis 0 of (8, 4096, 4096) f32, U[-1,1], 2 rotating inputs",
            "value": round(gbs, 1), "unit": "GB/s", "us_per_launch": round(secs / steps * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("sum_axis0_vec_kernel", kernel_source_hash())}}


def cpu_baseline(inputs, target_seconds):
    """The oracle (plain binary64 triple loop, all host threads) timed on a
    bounded sample of the headline workload: the first R full rows of the
    4096^3 product, R chosen so the run takes about `target_seconds`."""
    import numpy as np

    import oracle
    M = N = K = 4096
    A, B = inputs.gemm_inputs(M, N, K)
    cores = oracle.threads()

    def run(rows):
        I = np.repeat(np.arange(rows, dtype=np.int64), N)
        J = np.tile(np.arange(N, dtype=np.int64), rows)
        t0 = time.perf_counter()
        oracle.gemm_f16_points(A, B, I, J)
        return time.perf_counter() - t0

    rows = 4
    t = run(rows)
    rows = int(max(4, min(M, rows * target_seconds / max(t, 1e-3))))
    t = run(rows)
    flops = 2.0 * rows * N * K
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of 4096 rows of the 4096^3 fp16 GEMM (%.1f s, %d threads)"
                      % (rows, t, cores)}


def cpu_baseline_stream(inputs):
    """The oracle's elementwise add (plain loop, all host threads) on the
    same 8192 x 8192 workload, 5 calls after one untimed one, in GB/s of
    12 algorithmic bytes per element."""
    import oracle
    x, y = inputs.stream_inputs((8192, 8192))
    oracle.add_f32(x, y)
    t0 = time.perf_counter()
    for _ in range(5):
        oracle.add_f32(x, y)
    t = (time.perf_counter() - t0) / 5
    return {"value": round(12.0 * x.size / t / 1e9, 2), "unit": "GB/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": "the full 8192x8192 add, 5 calls (%.3f s each, %d threads)"
            % (t, oracle.threads())}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
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
        profile_run(pg, inputs)
        return
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    print("device: %s, %d CUs; assumed peaks: fp16 MFMA %.1f TFLOP/s, HBM %.0f GB/s"
          % (props.name, props.multi_processor_count, PEAK_FP16_TFLOPS, PEAK_HBM_GBS),
          file=sys.stderr, flush=True)

    head = gemm_case(pg, inputs, 4096, 4096, 4096, "uniform", args.steps, args.warmup, stream)
    print("gemm 4096^3: %.1f us, %.1f TFLOP/s" % (head["us_per_launch"], head["tflops"]),
          file=sys.stderr, flush=True)
    src_hash = kernel_source_hash()
    traffic = measured_traffic("gemm_f16_kernel_4096", src_hash)
    out = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_launch"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "fp16 GEMM M=N=K=4096, row-major A and B, U[-1,1] inputs, "
                               "fp32 accumulate, fp16 out"},
        "roofline": {"bound": "mfma", "achieved": round(head["tflops"], 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(head["frac_of_peak"], 4), "traffic": traffic},
    }
    if not args.quick:
        add = stream_case(pg, inputs, args.steps, args.warmup, stream, scalar=False)
        addc = stream_case(pg, inputs, args.steps, args.warmup, stream, scalar=True)
        print("stream add: %.1f GB/s; x+1: %.1f GB/s" % (add["GB/s"], addc["GB/s"]),
              file=sys.stderr, flush=True)
        out["streaming"] = {
            "workload": "z = x + y, fp32 8192x8192, U[-1,1], 3 rotating buffer sets",
            "value": round(add["GB/s"], 1), "unit": "GB/s",
            "us_per_launch": round(add["us_per_launch"], 2),
            "roofline": {"bound": "hbm", "achieved": round(add["GB/s"], 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(add["frac_of_hbm"], 4),
                         "traffic": measured_traffic("add_vec_kernel", src_hash)},
            "x_plus_1": {"value": round(addc["GB/s"], 1), "unit": "GB/s",
                         "us_per_launch": round(addc["us_per_launch"], 2),
                         "frac": round(addc["frac_of_hbm"], 4)},
        }
        out["reduction"] = reduce_case(pg, inputs, max(5, args.steps // 5), max(3, args.warmup // 5),
                                       stream)
        print("reduction: %.1f GB/s" % out["reduction"]["value"], file=sys.stderr, flush=True)
        others = []
        for (M, N, K, dist) in [(8192, 8192, 8192, "normal"), (2048, 2048, 32768, "uniform"),
                                (256, 256, 256, "uniform")]:
            r = gemm_case(pg, inputs, M, N, K, dist, max(5, args.steps // 10), max(3, args.warmup // 10),
                          stream)
            print("gemm %dx%dx%d: %.1f us, %.1f TFLOP/s" % (M, N, K, r["us_per_launch"], r["tflops"]),
                  file=sys.stderr, flush=True)
            others.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        # long K through split-K (the caller provides the fp32 workspace)
        r = gemm_case(pg, inputs, 2048, 2048, 32768, "uniform", max(5, args.steps // 10),
                      max(3, args.warmup // 10), stream, splitk=True)
        print("gemm 2048x2048x32768 split-K: %.1f us, %.1f TFLOP/s" % (r["us_per_launch"], r["tflops"]),
              file=sys.stderr, flush=True)
        others.append({k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()})
        out["other_gemm"] = others
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inputs, args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
        if "streaming" in out:
            out["streaming"]["cpu_baseline"] = cpu_baseline_stream(inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
