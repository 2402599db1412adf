"""ctypes binding of libpgemm (include/pgemm.h).

Argument marshalling only: every computation runs in the HIP kernels of
libpgemm.so.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpgemm.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "pgemm.h")

PGEMM_OK = 0
PGEMM_EINVAL = -1
PGEMM_EUNSUPPORTED = -2
PGEMM_EHIP = -3
PGEMM_ESCRATCH = -4
STATIC_SCRATCH_BYTES = 64 << 20  # PGEMM_STATIC_SCRATCH_BYTES of include/pgemm.h

_lib = None


class PgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))


def _declare(lib):
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = {
        "pgemm_f16": (i32, [p, p, p, i64, i64, i64, p]),
        "pgemm_f16_variant": (i32, [p, p, p, i64, i64, i64, i32, p]),
        "pgemm_f16_num_variants": (i32, []),
        "pgemm_f16_choose_variant": (i32, [i64, i64, i64]),
        "pgemm_f16_plan": (i32, [i64, i64, i64, i32, p, p, p]),
        "pgemm_f16_splitk": (i32, [p, p, p, i64, i64, i64, i32, p, i64, p]),
        "pgemm_f16_splitk_noalloc": (i32, [p, p, p, i64, i64, i64, i32, p]),
        "pgemm_f16_splitk_workspace_bytes": (i64, [i64, i64, i64, i32]),
        "pgemm_f16_splitk_default_splits": (i32, [i64, i64, i64]),
        "pstream_add": (i32, [p, p, p, i64, p]),
        "pstream_add_blocked": (i32, [p, p, p, i64, i64, p]),
        "pstream_add_scalar": (i32, [p, ctypes.c_float, p, i64, p]),
        "preduce_sum_f32": (i32, [p, p, i64, i64, p]),
        "pgemm_test_fill_f32": (i32, [p, ctypes.c_float, i64, p]),
        "pgemm_test_iota_f32": (i32, [p, i64, p]),
        "pgemm_status_string": (ctypes.c_char_p, [i32]),
        "pgemm_last_hip_error": (i32, []),
        "pgemm_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded libpgemm (ctypes.CDLL).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpgemm.so is not built (%s); run "
                               "`python -m software_pipelined_tiled_pgemm_amd.build`" % LIB_PATH)
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return lib().pgemm_status_string(int(status)).decode()


def declared_functions() -> list:
    """Names of the functions include/pgemm.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(p\w+)\s*\(", text, flags=re.M)))
