"""libpgemm for MI355X (gfx950): software-pipelined tiled fp16 GEMM and the
pipelined streaming elementwise add, behind a plain C ABI (include/pgemm.h).

The functions below carry the C ABI's names and take torch tensors; they only
check arguments, pick the stream and pass pointers.  torch supplies device
memory and streams; all arithmetic happens in the HIP kernels.  Loading is
lazy (importing the package does not touch the GPU or the library), and a
missing library raises -- there is no CPU fallback.
"""
from __future__ import annotations

from ._lib import (PGEMM_EHIP, PGEMM_EINVAL, PGEMM_ESCRATCH, PGEMM_EUNSUPPORTED, PGEMM_OK,
                   STATIC_SCRATCH_BYTES, PgemmError, lib, status_string)

__all__ = [
    "pgemm_f16", "pgemm_f16_variant", "pgemm_f16_num_variants", "pgemm_f16_choose_variant",
    "pgemm_f16_plan",
    "pgemm_f16_splitk", "pgemm_f16_splitk_noalloc", "pgemm_f16_splitk_workspace_bytes",
    "pgemm_f16_splitk_default_splits",
    "pstream_add", "pstream_add_blocked", "pstream_add_scalar", "preduce_sum_f32",
    "pgemm_test_fill_f32", "pgemm_test_iota_f32",
    "lib", "status_string", "PgemmError",
    "PGEMM_OK", "PGEMM_EINVAL", "PGEMM_EUNSUPPORTED", "PGEMM_EHIP", "PGEMM_ESCRATCH",
    "STATIC_SCRATCH_BYTES",
]


# torch and the few of its entry points each call uses, looked up once: a
# small GEMM's kernel takes about 5 us, so the binding's own per-call work
# (argument checks, stream lookup, the ctypes call) has to stay below that.
_TORCH = None
_TENSOR = None
_F16 = None
_F32 = None
_CUR_DEVICE = None
_RAW_STREAM = None


def _torch():
    global _TORCH, _TENSOR, _F16, _F32, _CUR_DEVICE, _RAW_STREAM
    if _TORCH is None:
        import torch
        _TENSOR, _F16, _F32 = torch.Tensor, torch.float16, torch.float32
        _CUR_DEVICE = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _TORCH = torch
    return _TORCH


def _raw_stream(index, stream):
    """The hipStream_t (as an int) to launch on: `stream`'s, else the current
    stream of device `index`."""
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None:
        return _RAW_STREAM(index)
    return _torch().cuda.current_stream(index).cuda_stream


def _invoke(t, stream, fn):
    """fn(stream handle) with t's device current, switched only when it
    differs.  Device tensors exist, so the HIP runtime is initialised and the
    current device can be read directly."""
    torch = _torch()
    index = t.get_device()
    if index == _CUR_DEVICE():
        return fn(_raw_stream(index, stream))
    with torch.cuda.device(index):
        return fn(_raw_stream(index, stream))


def _check_dev(t, dtype, name, ndim=None):
    torch = _torch()
    # the common case in one expression; the branches below name the problem
    if (type(t) is _TENSOR and t.is_cuda and t.dtype is dtype
            and (ndim is None or t.dim() == ndim) and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (HIP) tensor, got %s" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major)" % name)


def _new(shape, dtype, device, stream):
    """An empty tensor for a call on `stream` (None: the current stream).
    torch's caching allocator keeps one pool per stream and orders reuse by
    that stream alone, so memory for a call on another stream is taken from
    that stream's pool: a block from the current stream's pool could still
    be in use by pending work there, and would go back to that pool, free for
    the current stream, while the call's kernels still use it."""
    torch = _torch()
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _call(rc, what):
    if rc != PGEMM_OK:
        raise PgemmError(rc, what)


def pgemm_f16(A, B, C=None, stream=None):
    """C = A @ B for fp16 row-major A [M,K], B [K,N]; returns C [M,N] fp16."""
    return pgemm_f16_variant(A, B, 0, C=C, stream=stream)


def pgemm_f16_variant(A, B, variant, C=None, stream=None):
    """pgemm_f16 with the tile configuration forced (0 = automatic)."""
    torch = _torch()
    _check_dev(A, torch.float16, "A", 2)
    _check_dev(B, torch.float16, "B", 2)
    dev_a = A.get_device()
    if dev_a != B.get_device():
        raise ValueError("A and B are on different devices")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %s @ %s" % (tuple(A.shape), tuple(B.shape)))
    if C is None:
        C = _new((M, N), torch.float16, A.device, stream)
    else:
        _check_dev(C, torch.float16, "C", 2)
        if C.shape != (M, N) or C.get_device() != dev_a:
            raise ValueError("C must be a (%d, %d) tensor on %s" % (M, N, A.device))
    f = lib().pgemm_f16_variant
    rc = _invoke(A, stream, lambda h: f(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                                        int(variant), h))
    _call(rc, "pgemm_f16")
    return C


def pgemm_f16_splitk_workspace_bytes(M, N, K, splits):
    rc = lib().pgemm_f16_splitk_workspace_bytes(int(M), int(N), int(K), int(splits))
    if rc < 0:
        raise PgemmError(int(rc), "pgemm_f16_splitk_workspace_bytes")
    return rc


def pgemm_f16_splitk_default_splits(M, N, K):
    rc = lib().pgemm_f16_splitk_default_splits(int(M), int(N), int(K))
    if rc < 0:
        raise PgemmError(rc, "pgemm_f16_splitk_default_splits")
    return rc


def pgemm_f16_splitk(A, B, splits=None, C=None, workspace=None, stream=None):
    """C = A @ B with K cut into `splits` chunks (None: the library's default
    for the shape) reduced through an fp32 workspace (allocated here with
    torch when not given)."""
    torch = _torch()
    _check_dev(A, torch.float16, "A", 2)
    _check_dev(B, torch.float16, "B", 2)
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or A.device != B.device:
        raise ValueError("inner dimensions or devices differ")
    if C is None:
        C = _new((M, N), torch.float16, A.device, stream)
    else:
        _check_dev(C, torch.float16, "C", 2)
        if tuple(C.shape) != (M, N) or C.device != A.device:
            raise ValueError("C must be a (%d, %d) tensor on %s" % (M, N, A.device))
    if splits is None:
        splits = pgemm_f16_splitk_default_splits(M, N, K)
    need = pgemm_f16_splitk_workspace_bytes(M, N, K, splits)
    if workspace is None:
        workspace = _new(max(need // 4, 1), torch.float32, A.device, stream)
    elif workspace.device != A.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % A.device)
    f = lib().pgemm_f16_splitk
    rc = _invoke(A, stream, lambda h: f(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                                        int(splits), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), h))
    _call(rc, "pgemm_f16_splitk")
    return C


def pgemm_f16_splitk_noalloc(A, B, splits=None, C=None, stream=None):
    """pgemm_f16_splitk with the partials in the library's static device
    buffer (no workspace, no allocation by the library; C is allocated here
    only when not given).  Calls that overlap on one device race on that
    buffer."""
    torch = _torch()
    _check_dev(A, torch.float16, "A", 2)
    _check_dev(B, torch.float16, "B", 2)
    M, K = A.shape
    K2, N = B.shape
    if K != K2 or A.get_device() != B.get_device():
        raise ValueError("inner dimensions or devices differ")
    if C is None:
        C = _new((M, N), torch.float16, A.device, stream)
    else:
        _check_dev(C, torch.float16, "C", 2)
        if C.shape != (M, N) or C.get_device() != A.get_device():
            raise ValueError("C must be a (%d, %d) tensor on %s" % (M, N, A.device))
    if splits is None:
        splits = pgemm_f16_splitk_default_splits(M, N, K)
    f = lib().pgemm_f16_splitk_noalloc
    rc = _invoke(A, stream, lambda h: f(A.data_ptr(), B.data_ptr(), C.data_ptr(), M, N, K,
                                        int(splits), h))
    _call(rc, "pgemm_f16_splitk_noalloc")
    return C


def pgemm_f16_num_variants():
    return lib().pgemm_f16_num_variants()


def pgemm_f16_choose_variant(M, N, K):
    """The variant pgemm_f16 runs for an M x N x K problem (host only)."""
    rc = lib().pgemm_f16_choose_variant(int(M), int(N), int(K))
    if rc < 0:
        raise PgemmError(rc, "pgemm_f16_choose_variant")
    return rc


def pgemm_f16_plan(M, N, K, cus=0):
    """(head_rows, head_variant, tail_variant): the launches pgemm_f16 makes
    for an M x N x K problem on `cus` CUs (0: the current device's count);
    tail_variant is 0 when one launch covers all M rows (host only)."""
    import ctypes
    head, hv, tv = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int()
    rc = lib().pgemm_f16_plan(int(M), int(N), int(K), int(cus), ctypes.byref(head),
                              ctypes.byref(hv), ctypes.byref(tv))
    if rc < 0:
        raise PgemmError(rc, "pgemm_f16_plan")
    return head.value, hv.value, tv.value


def _elementwise_out(x, z, stream):
    torch = _torch()
    if z is None:
        return _new(tuple(x.shape), torch.float32, x.device, stream)
    _check_dev(z, torch.float32, "z")
    if z.numel() != x.numel() or z.get_device() != x.get_device():
        raise ValueError("z must have x's size and device")
    return z


def pstream_add(x, y, z=None, stream=None):
    """z = x + y elementwise (fp32, bit-exact IEEE); z may be x or y."""
    return pstream_add_blocked(x, y, None, z=z, stream=stream)


def pstream_add_blocked(x, y, block_elems, z=None, stream=None):
    """pstream_add with the per-workgroup block size forced (None = default)."""
    torch = _torch()
    _check_dev(x, torch.float32, "x")
    _check_dev(y, torch.float32, "y")
    if x.numel() != y.numel() or x.get_device() != y.get_device():
        raise ValueError("x and y must have the same size and device")
    z = _elementwise_out(x, z, stream)
    L = lib()
    if block_elems is None:
        rc = _invoke(x, stream, lambda h: L.pstream_add(x.data_ptr(), y.data_ptr(), z.data_ptr(),
                                                        x.numel(), h))
    else:
        rc = _invoke(x, stream, lambda h: L.pstream_add_blocked(
            x.data_ptr(), y.data_ptr(), z.data_ptr(), x.numel(), int(block_elems), h))
    _call(rc, "pstream_add")
    return z


def pstream_add_scalar(x, c, z=None, stream=None):
    """z = x + c elementwise (fp32); z may be x (in place)."""
    torch = _torch()
    _check_dev(x, torch.float32, "x")
    z = _elementwise_out(x, z, stream)
    f = lib().pstream_add_scalar
    rc = _invoke(x, stream, lambda h: f(x.data_ptr(), float(c), z.data_ptr(), x.numel(), h))
    _call(rc, "pstream_add_scalar")
    return z


def preduce_sum_f32(x, out=None, stream=None):
    """Sum of a float32 tensor of shape (R, ...) over its first axis, added
    in ascending order from +0.0 (the guide's section 7.2 reduction)."""
    torch = _torch()
    _check_dev(x, torch.float32, "x")
    if x.dim() < 1:
        raise ValueError("x needs at least one dimension")
    R = x.shape[0]
    if out is None:
        out = _new(tuple(x.shape[1:]), torch.float32, x.device, stream)
    else:
        _check_dev(out, torch.float32, "out")
        if tuple(out.shape) != tuple(x.shape[1:]) or out.device != x.device:
            raise ValueError("out must have shape %s on %s" % (tuple(x.shape[1:]), x.device))
    f = lib().preduce_sum_f32
    rc = _invoke(x, stream, lambda h: f(x.data_ptr(), out.data_ptr(), R, out.numel(), h))
    _call(rc, "preduce_sum_f32")
    return out


def pgemm_test_fill_f32(n, v=42.0, device="cuda", out=None, stream=None):
    torch = _torch()
    o = out if out is not None else _new(int(n), torch.float32, device, stream)
    _check_dev(o, torch.float32, "out")
    f = lib().pgemm_test_fill_f32
    rc = _invoke(o, stream, lambda h: f(o.data_ptr(), float(v), o.numel(), h))
    _call(rc, "pgemm_test_fill_f32")
    return o


def pgemm_test_iota_f32(n, device="cuda", out=None, stream=None):
    torch = _torch()
    o = out if out is not None else _new(int(n), torch.float32, device, stream)
    _check_dev(o, torch.float32, "out")
    f = lib().pgemm_test_iota_f32
    rc = _invoke(o, stream, lambda h: f(o.data_ptr(), o.numel(), h))
    _call(rc, "pgemm_test_iota_f32")
    return o
