"""CPU oracle for the pipelined GEMM and the streaming elementwise pipeline.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``software_pipelined_tiled_pgemm_amd``) never imports, links or calls it,
and this package never imports the product path: the two share nothing but
the seeded input generators, which live in a module of their own.

The arithmetic is in ``ref.c`` (plain C, built with gcc); this module loads
it with ctypes and converts numpy arrays.  What each function computes, and
the passage of the pages it follows:

* ``gemm_f16`` / ``gemm_f16_points`` -- C = A @ B for row-major fp16 A[M,K]
  and B[K,N]: the matmul of the Pallas "Quickstart: GPU" page, section
  "Pipelining: a matmul kernel" (fp16 in, fp32 accumulator, ``astype`` to
  fp16 out).  Written as its definition: exact fp16 products summed in
  ascending k in binary64, rounded once to binary16 (ties to even).
* ``add_f32`` / ``add_scalar_f32`` -- the pipelined elementwise add of the
  Pallas software-pipelining guide (lmnt.cn), section 6, and the "+1" loop of
  its section 4: one IEEE binary32 addition per element.
* ``fill_f32`` / ``iota_f32`` -- "Your first kernel" (42.0 everywhere) and
  "Parallel work with a grid" (0.0 .. n-1) of the quickstart.
* ``sum_axis0_f32`` -- the guide's section 7.2 reduction: the output block
  starts at zero and x[0], x[1], ... are added to it in order, in f32.
* ``f16_from_f64`` / ``f64_from_f16`` -- the binary16 rounding and decoding
  used by the GEMM oracle, exposed so tests can pin them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``ref.c`` into ``liboracle.so`` with gcc (IEEE arithmetic:
    no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_f64_from_f16.restype = ctypes.c_double
    lib.oracle_f64_from_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_from_f64.restype = ctypes.c_uint16
    lib.oracle_f16_from_f64.argtypes = [ctypes.c_double]
    lib.oracle_f16_from_f64_array.argtypes = [p, p, i64]
    lib.oracle_f64_from_f16_array.argtypes = [p, p, i64]
    lib.oracle_gemm_f16.argtypes = [p, p, p, p, i64, i64, i64]
    lib.oracle_gemm_f16_points.argtypes = [p, p, i64, i64, i64, p, p, i64, p, p]
    lib.oracle_add_f32.argtypes = [p, p, p, i64]
    lib.oracle_add_scalar_f32.argtypes = [p, ctypes.c_float, p, i64]
    lib.oracle_fill_f32.argtypes = [p, ctypes.c_float, i64]
    lib.oracle_sum_axis0_f32.argtypes = [p, p, i64, i64]
    lib.oracle_iota_f32.argtypes = [p, i64]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_f16_bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 bit patterns, got %s" % a.dtype)
    return np.ascontiguousarray(a)


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def f64_from_f16(h) -> np.ndarray:
    """Exact binary64 values of binary16 bit patterns (or float16 arrays)."""
    h = _as_f16_bits(h)
    out = np.empty(h.shape, np.float64)
    _load().oracle_f64_from_f16_array(_ptr(h), _ptr(out), h.size)
    return out


def f16_from_f64(x) -> np.ndarray:
    """Round binary64 values to binary16 (RNE, one step); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f16_from_f64_array(_ptr(x), _ptr(out), x.size)
    return out


def gemm_f16(A, B):
    """C = A @ B.  A: fp16 [M,K], B: fp16 [K,N] (row-major).

    Returns (C as float16 [M,N], S as float64 [M,N] unrounded sums)."""
    A = _as_f16_bits(A)
    B = _as_f16_bits(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("shape mismatch %s @ %s" % (A.shape, B.shape))
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.uint16)
    S = np.empty((M, N), np.float64)
    _load().oracle_gemm_f16(_ptr(A), _ptr(B), _ptr(C), _ptr(S), M, N, K)
    return C.view(np.float16), S


def gemm_f16_points(A, B, I, J):
    """Elements (I[p], J[p]) of A @ B, same arithmetic as ``gemm_f16``.

    Returns (C values as float16 [P], S float64 [P])."""
    A = _as_f16_bits(A)
    B = _as_f16_bits(B)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("shape mismatch %s @ %s" % (A.shape, B.shape))
    M, K = A.shape
    N = B.shape[1]
    I = np.ascontiguousarray(np.asarray(I, dtype=np.int64))
    J = np.ascontiguousarray(np.asarray(J, dtype=np.int64))
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D and of equal length")
    if I.size and (I.min() < 0 or I.max() >= M or J.min() < 0 or J.max() >= N):
        raise IndexError("sample point outside the output")
    C = np.empty(I.size, np.uint16)
    S = np.empty(I.size, np.float64)
    _load().oracle_gemm_f16_points(_ptr(A), _ptr(B), M, N, K, _ptr(I), _ptr(J),
                                   I.size, _ptr(C), _ptr(S))
    return C.view(np.float16), S


def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("expected float32, got %s" % a.dtype)
    return np.ascontiguousarray(a)


def add_f32(x, y) -> np.ndarray:
    """z = x + y, one binary32 addition per element."""
    x, y = _f32(x), _f32(y)
    if x.shape != y.shape:
        raise ValueError("shape mismatch")
    z = np.empty_like(x)
    _load().oracle_add_f32(_ptr(x), _ptr(y), _ptr(z), x.size)
    return z


def add_scalar_f32(x, c: float) -> np.ndarray:
    """z = x + c (c rounded to binary32 first), one addition per element."""
    x = _f32(x)
    z = np.empty_like(x)
    _load().oracle_add_scalar_f32(_ptr(x), ctypes.c_float(c), _ptr(z), x.size)
    return z


def sum_axis0_f32(x) -> np.ndarray:
    """o = x[0] + x[1] + ... + x[R-1] (first axis), f32, added in that order
    starting from +0.0.  x: float32 of shape (R, ...)."""
    x = _f32(x)
    if x.ndim < 1:
        raise ValueError("need at least one axis")
    R = x.shape[0]
    n = int(np.prod(x.shape[1:], dtype=np.int64))
    o = np.empty(x.shape[1:], np.float32)
    _load().oracle_sum_axis0_f32(_ptr(x), _ptr(o), R, n)
    return o


def fill_f32(n: int, v: float = 42.0) -> np.ndarray:
    o = np.empty(int(n), np.float32)
    _load().oracle_fill_f32(_ptr(o), ctypes.c_float(v), o.size)
    return o


def iota_f32(n: int) -> np.ndarray:
    o = np.empty(int(n), np.float32)
    _load().oracle_iota_f32(_ptr(o), o.size)
    return o
