"""Autotuner for pgemm_f16's tile configuration.

The pages name the block size as the main knob when tuning a pipelined
kernel (software pipelining guide, section 6.1) and advise autotuning the
number of concurrent copies (Chinese quickstart, section on emit_pipeline's
key parameters).  Here the knobs are bundled into the variants of
pgemm_f16_variant (output tile 256x256 or 128x128, LDS-DMA ring of 5 stages
or register-staged 2 stages, 4 or 8 waves, 32x32x16 or 16x16x32 matrix
instruction).  This module times every variant
on a set of shapes and writes the table of every variant's rate per shape
that is compiled into libpgemm (csrc/gemm_tuned.inc).  pgemm_f16 (variant
0) then runs the fastest variant of the tuned shape nearest to the
problem, unless scaling every variant's rate there by how well its tiles
fill the CUs on the problem against on the tuned shape predicts another
variant more than 30% faster (choose() restates the library's rule).

Timing: each variant launches back to back on one stream with HIP events
around the batch; the variants of a shape are interleaved over several
rounds and the best round counts, so clock drift between variants cancels.
Variants within 1% of the fastest count as tied; the lowest id wins.
Variants of one matrix-instruction family compute bit-identical results;
the two families group each output's K sum differently and may differ in
the last bits, both within the accuracy bound.

    python -m software_pipelined_tiled_pgemm_amd.autotune --out <file.inc>
"""
from __future__ import annotations

import argparse
import math
import os
import re
import sys

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm_tuned.inc")

# Squares from one tile to several waves of tiles, long and short K, skinny
# and wide shapes, and one GPU's row block of the 4096^3, 8192^3 and
# 2048^2 x 32768 products split eight ways by rows of C.
DEFAULT_SHAPES = [
    (256, 256, 256), (512, 512, 512), (1024, 1024, 1024), (1536, 1536, 1536),
    (2048, 2048, 2048), (3072, 3072, 3072), (4096, 4096, 4096), (6144, 6144, 6144),
    (8192, 8192, 8192),
    (1024, 1024, 16384), (2048, 2048, 32768), (4096, 4096, 16384),
    (4096, 4096, 512), (8192, 8192, 1024),
    (8192, 1024, 4096), (1024, 8192, 4096), (16384, 2048, 2048),
    (512, 4096, 4096), (1024, 8192, 8192), (256, 2048, 32768),
    (2048, 2048, 8192), (4096, 4096, 2048), (1536, 1536, 8192), (3072, 3072, 12288),
    (2048, 8192, 2048), (8192, 2048, 8192), (6144, 2048, 4096), (2048, 6144, 4096),
    (12288, 12288, 4096), (16384, 16384, 1024),
]
# Plus a grid in log space, so that the nearest tuned shape of a new problem
# is never far off: M, N in 256 .. 16384 and K in 256 .. 32768 (products up
# to 2^41 flop/2).
GRID_MN = (256, 512, 1024, 2048, 4096, 8192, 16384)
GRID_K = (256, 1024, 4096, 16384, 32768)
DEFAULT_SHAPES += [(m, n, k) for m in GRID_MN for n in GRID_MN for k in GRID_K
                   if m * n * k <= 1 << 41 and (m, n, k) not in DEFAULT_SHAPES]

_ENTRY = re.compile(r"^\{\s*(\d+),\s*(\d+),\s*(\d+),\s*(\d+)\s*,\s*\{([^}]*)\}\s*\},")


def _time_batch(lib, ptrs, M, N, K, variant, n, stream):
    import torch
    a, b, c = ptrs
    h = stream.cuda_stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        rc = lib.pgemm_f16_variant(a, b, c, M, N, K, variant, h)
        if rc != 0:
            raise RuntimeError("pgemm_f16_variant(%d) failed with status %d" % (variant, rc))
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / n  # seconds per launch


def measure(shapes=None, variants=None, rounds=3, target_s=0.02, log=None):
    """Times every variant on every shape.  Returns a list of
    {"M", "N", "K", "tflops": {variant: best TFLOP/s}}."""
    import torch

    from . import lib
    L = lib()
    shapes = list(shapes or DEFAULT_SHAPES)
    variants = list(variants or range(1, L.pgemm_f16_num_variants() + 1))
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    out = []
    for (M, N, K) in shapes:
        # U[-1, 1] operands, drawn on the device (the timing depends on the
        # distribution, which sets the power draw, not on the exact values)
        tA = (torch.rand((M, K), generator=gen, device="cuda") * 2 - 1).half()
        tB = (torch.rand((K, N), generator=gen, device="cuda") * 2 - 1).half()
        tC = torch.empty((M, N), dtype=torch.float16, device="cuda")
        ptrs = (tA.data_ptr(), tB.data_ptr(), tC.data_ptr())
        # launches per batch: about target_s of GPU time per variant
        per = {}
        for v in variants:
            t = _time_batch(L, ptrs, M, N, K, v, 3, stream)
            per[v] = max(3, min(2000, int(target_s / max(t, 1e-7))))
        best = {v: 0.0 for v in variants}
        for _ in range(rounds):
            for v in variants:
                _time_batch(L, ptrs, M, N, K, v, max(2, per[v] // 4), stream)  # warm-up
                t = _time_batch(L, ptrs, M, N, K, v, per[v], stream)
                best[v] = max(best[v], 2.0 * M * N * K / t / 1e12)
        rec = {"M": M, "N": N, "K": K, "tflops": best}
        out.append(rec)
        if log:
            log("%dx%dx%d: " % (M, N, K) + "  ".join("v%d %.1f" % (v, x) for v, x in best.items())
                + "  -> v%d" % fastest(rec))
        del tA, tB, tC
    return out


# Variants within this fraction of the fastest count as tied, and the lowest
# id among them is taken: same-process repeats differ by up to about 1%, so
# a closer race would let the table flip between runs.
TIE = 0.01


def fastest(rec) -> int:
    best = max(rec["tflops"].values())
    return min(v for v, x in rec["tflops"].items() if x >= (1.0 - TIE) * best)


def render_table(records, device: str = "") -> str:
    """The table as C initialisers {M, N, K, fastest, {rate of v1, v2, ...}}.
    Rates are rounded to 0.1 TFLOP/s first; the fastest variant is taken
    from the rounded rates, which are what the library reads."""
    lines = ["// Generated by software_pipelined_tiled_pgemm_amd/autotune.py; do not edit.",
             "// {M, N, K, fastest variant, {best TFLOP/s of variant 1, 2, ...}},"]
    if device:
        lines.append("// Measured on %s." % device)
    for r in records:
        rates = {v: round(x, 1) for v, x in r["tflops"].items()}
        nv = max(rates)
        vals = ", ".join("%.1f" % rates.get(v, 0.0) for v in range(1, nv + 1))
        lines.append("{%d, %d, %d, %d, {%s}}," % (r["M"], r["N"], r["K"],
                                                 fastest({"tflops": rates}), vals))
    return "\n".join(lines) + "\n"


def parse_rates(text: str):
    """(M, N, K, fastest variant, {variant: TFLOP/s}) entries of a table."""
    out = []
    for m in map(_ENTRY.match, text.splitlines()):
        if m:
            M, N, K, v = (int(g) for g in m.groups()[:4])
            rates = {i + 1: float(x) for i, x in enumerate(m.group(5).split(","))}
            out.append((M, N, K, v, rates))
    return out


def parse_table(text: str):
    """(M, N, K, fastest variant) entries of a generated table."""
    return [e[:4] for e in parse_rates(text)]


# Tile edge of each variant of pgemm_f16_variant (the others use 128x128),
# and the variants of which two workgroups fit on one CU (the others: one).
TILE_256 = (1, 3, 5, 8, 9)
TWO_PER_CU = (2, 4, 6, 7)
# The choice leaves the nearest tuned shape's fastest variant only for an
# estimate more than this much faster.
REFILL_GAIN = 1.3


def slot_fill(M, N, b, slots):
    """Useful share of the workgroup slots of an M x N launch with b x b
    tiles: M*N / (waves * slots * b*b), waves = ceil(tiles / slots)."""
    tiles = ((M + b - 1) // b) * ((N + b - 1) // b)
    waves = (tiles + slots - 1) // slots
    return float(M) * float(N) / (float(waves) * slots * b * b)


def choose(rates_table, M, N, K, cus=256, num_variants=None) -> int:
    """The library's choice for an M x N x K problem on `cus` CUs, from
    parse_rates() entries (restated here for the tests): the nearest tuned
    shape T (sum of |log2| ratios over M, N, K; the first on ties) and its
    fastest variant v0; each variant's rate on T scaled by slot_fill on the
    problem over slot_fill on T; the best estimate (lowest id within TIE)
    replaces v0 only if it beats v0's estimate by more than REFILL_GAIN."""
    if not rates_table or M <= 0 or N <= 0:
        return 2
    if cus <= 0:
        cus = 256

    def l2(a):
        return math.log2(max(a, 1))
    lm, ln, lk = l2(M), l2(N), l2(K)
    near, near_d = None, float("inf")
    for e in rates_table:
        d = abs(lm - l2(e[0])) + abs(ln - l2(e[1])) + abs(lk - l2(e[2]))
        if d < near_d:
            near, near_d = e, d
    tm, tn, _, v0, rates = near
    nv = num_variants or max(rates)
    est = {}
    for v in range(1, nv + 1):
        b = 256 if v in TILE_256 else 128
        slots = (2 if v in TWO_PER_CU else 1) * cus
        est[v] = rates.get(v, 0.0) * slot_fill(M, N, b, slots) / slot_fill(tm, tn, b, slots)
    top = max(est.values())
    if not 1 <= v0 <= nv or top <= 0.0:
        return 2
    alt = min(v for v in est if est[v] >= (1.0 - TIE) * top)
    return alt if est[alt] > REFILL_GAIN * est[v0] else v0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=None, help="where to write the table (default: print it)")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="only 3 shapes")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("autotune needs a HIP device", file=sys.stderr)
        return 1
    shapes = DEFAULT_SHAPES[:1] + [(4096, 4096, 4096), (2048, 2048, 32768)] if args.quick else None
    recs = measure(shapes, rounds=args.rounds, log=lambda s: print(s, flush=True))
    text = render_table(recs, torch.cuda.get_device_properties(0).name)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
        print("wrote %s" % args.out, flush=True)
    else:
        sys.stdout.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
