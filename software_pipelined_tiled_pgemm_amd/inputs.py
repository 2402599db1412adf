"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check.  This module holds no arithmetic of the method: it only draws random
numbers and stores them in the input dtype.  It imports nothing from the rest
of the package and nothing from the oracle.

Recipes (numpy ``default_rng``, binary64 draws, then one round-to-nearest-even
conversion to the storage type):

* GEMM, uniform: A = U[-1,1] with seed 0, B = U[-1,1] with seed 1, stored as
  float16.  The seeds follow the key(0)/key(1) convention of the pipelined
  elementwise example of the Pallas software-pipelining guide, section 6.
* GEMM, normal: N(0, std = 1/sqrt(K)), same seeds, stored as float16.
* Streaming add: x = U[-1,1] seed 0, y = U[-1,1] seed 1, stored as float32.

For operands too large to draw on the host (several GiB), ``hashed_f16``
defines element (r, c) of a matrix by an integer hash of its indices, so any
row or column subset can be rebuilt on the host and the whole matrix drawn
on the device (``hashed_f16_torch``, the same integer steps in torch).
"""
from __future__ import annotations

import numpy as np

SEED_A = 0
SEED_B = 1


def uniform_f16(shape, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(-1.0, 1.0, size=shape).astype(np.float16)


def normal_f16(shape, std: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, size=shape).astype(np.float16)


def uniform_f32(shape, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)


def gemm_inputs(M: int, N: int, K: int, dist: str = "uniform",
                seed_a: int = SEED_A, seed_b: int = SEED_B):
    """(A [M,K] fp16, B [K,N] fp16), row-major."""
    if dist == "uniform":
        return uniform_f16((M, K), seed_a), uniform_f16((K, N), seed_b)
    if dist == "normal":
        std = 1.0 / np.sqrt(K)
        return normal_f16((M, K), std, seed_a), normal_f16((K, N), std, seed_b)
    raise ValueError("unknown distribution %r" % dist)


def stream_inputs(shape, seed_x: int = SEED_A, seed_y: int = SEED_B):
    """(x, y) float32 of the given shape, U[-1,1]."""
    return uniform_f32(shape, seed_x), uniform_f32(shape, seed_y)


def sample_points(M: int, N: int, n_points: int, seed: int = 2,
                  full_rows: int = 32, full_cols: int = 32, tile: int = 128):
    """Deterministic output sample for shapes too large for the full oracle:
    ``full_rows`` whole rows, ``full_cols`` whole columns, ``n_points`` random
    elements, and the four corners of every ``tile``-aligned block (so every
    output tile and the ragged edge are visited).  Returns (I, J) int64."""
    rng = np.random.default_rng(seed)
    rows = rng.choice(M, size=min(full_rows, M), replace=False)
    cols = rng.choice(N, size=min(full_cols, N), replace=False)
    I = [np.repeat(rows, N)]
    J = [np.tile(np.arange(N), rows.size)]
    I.append(np.tile(np.arange(M), cols.size))
    J.append(np.repeat(cols, M))
    I.append(rng.integers(0, M, size=n_points))
    J.append(rng.integers(0, N, size=n_points))
    r0 = np.arange(0, M, tile)
    c0 = np.arange(0, N, tile)
    rr = np.concatenate([r0, np.minimum(r0 + tile - 1, M - 1)])
    cc = np.concatenate([c0, np.minimum(c0 + tile - 1, N - 1)])
    gi, gj = np.meshgrid(rr, cc, indexing="ij")
    I.append(gi.ravel())
    J.append(gj.ravel())
    I = np.concatenate(I).astype(np.int64)
    J = np.concatenate(J).astype(np.int64)
    key = np.unique(I * N + J)
    return (key // N).astype(np.int64), (key % N).astype(np.int64)


def _hash_values(r, c, seed, xor, shr):
    """Integer steps of ``hashed_f16`` (non-negative int64 throughout, no
    overflow: r, c < 2**31)."""
    m31 = 2147483647  # x & m31 == x mod 2**31 for x >= 0
    h = xor((r * 2654435761) & m31, (c * 40503 + seed * 7919) & m31)
    h = (xor(h, shr(h, 15)) * 2246822519) & m31
    h = xor(h, shr(h, 13)) % 2039
    return h - 1019


def hashed_f16(rows, cols, seed: int) -> np.ndarray:
    """Matrix [len(rows), len(cols)] with element (r, c) = (hash(r, c, seed)
    - 1019) / 1024, hash in 0..2038: multiples of 2**-10 in [-1019/1024, 1019/1024],
    all exact in float16."""
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.asarray(cols, dtype=np.int64)[None, :]
    out = np.empty((r.shape[0], c.shape[1]), dtype=np.float16)
    step = max(1, (1 << 20) // max(1, c.shape[1]))  # rows per chunk: small temporaries
    for r0 in range(0, r.shape[0], step):
        v = _hash_values(r[r0:r0 + step], c, seed, np.bitwise_xor, np.right_shift)
        out[r0:r0 + step] = (v.astype(np.float64) / 1024.0).astype(np.float16)
    return out


def hashed_f16_torch(n_rows: int, n_cols: int, seed: int, device, row_chunk: int = 2048):
    """The [n_rows, n_cols] ``hashed_f16`` matrix (rows 0.., columns 0..) as a
    float16 torch tensor on ``device``, built in row chunks of at most
    ``row_chunk`` rows and 2**25 elements."""
    import torch
    row_chunk = max(1, min(row_chunk, (1 << 25) // max(1, n_cols)))
    out = torch.empty((n_rows, n_cols), dtype=torch.float16, device=device)
    c = torch.arange(n_cols, dtype=torch.int64, device=device)[None, :]
    for r0 in range(0, n_rows, row_chunk):
        r = torch.arange(r0, min(n_rows, r0 + row_chunk), dtype=torch.int64, device=device)[:, None]
        v = _hash_values(r, c, seed, torch.bitwise_xor, torch.bitwise_right_shift)
        out[r0:r0 + r.shape[0]] = (v.to(torch.float64) / 1024.0).to(torch.float16)
    return out
