"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments on the host before any HIP
call (so these run on a machine without a GPU)."""
import ctypes
import os

import pytest

import software_pipelined_tiled_pgemm_amd as pg
from software_pipelined_tiled_pgemm_amd import _lib

EINVAL, EUNSUP, OK = pg.PGEMM_EINVAL, pg.PGEMM_EUNSUPPORTED, pg.PGEMM_OK


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from software_pipelined_tiled_pgemm_amd import build
        build.build()
    return pg.lib()


def test_header_declares_the_boundary():
    names = _lib.declared_functions()
    for n in ["pgemm_f16", "pgemm_f16_variant", "pgemm_f16_num_variants", "pgemm_f16_splitk",
              "pgemm_f16_splitk_noalloc",
              "pgemm_f16_splitk_workspace_bytes", "pgemm_f16_choose_variant", "pgemm_f16_plan",
              "pstream_add",
              "pstream_add_blocked", "pstream_add_scalar", "pgemm_test_fill_f32",
              "pgemm_test_iota_f32", "preduce_sum_f32", "pgemm_status_string", "pgemm_last_hip_error",
              "pgemm_version"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(L):
    for name in _lib.declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(pg.status_string(s), str) and pg.status_string(s)
    assert pg.status_string(0) == "ok"
    assert L.pgemm_last_hip_error() == 0
    assert L.pgemm_version() >= 200
    assert L.pgemm_f16_num_variants() >= 2


# Fake, never dereferenced addresses (16-byte aligned, far apart).
A, B, C = 0x10000000, 0x20000000, 0x30000000


@pytest.mark.parametrize("args,expected", [
    ((A, B, C, -1, 8, 8), EINVAL),
    ((A, B, C, 8, -8, 8), EINVAL),
    ((A, B, C, 8, 8, -8), EINVAL),
    ((0, B, C, 8, 8, 8), EINVAL),
    ((A, 0, C, 8, 8, 8), EINVAL),
    ((A, B, 0, 8, 8, 8), EINVAL),
    ((A, B, C, 8, 8, 12), EUNSUP),          # K % 8
    ((A, B, C, 8, 12, 8), EUNSUP),          # N % 8
    ((A + 2, B, C, 8, 8, 8), EUNSUP),       # alignment
    ((A, B + 8, C, 8, 8, 8), EUNSUP),
    ((A, B, C + 4, 8, 8, 8), EUNSUP),
    ((A, B, C, 8, 8, 1 << 22), EUNSUP),     # K limit
    ((A, B, C, (1 << 30) + 256, 1 << 7, 8), EUNSUP),  # M*N above 2^37: grid limit
    ((A, B, A + 16, 8, 8, 8), EINVAL),      # C overlaps A
    ((A, B, B, 8, 8, 8), EINVAL),           # C is B
    ((0, 0, 0, 0, 8, 8), OK),               # empty: nothing enqueued
    ((0, 0, 0, 8, 0, 8), OK),
])
def test_gemm_argument_checks(L, args, expected):
    assert L.pgemm_f16(*args, None) == expected


def test_splitk_workspace_bytes(L):
    wb = L.pgemm_f16_splitk_workspace_bytes
    assert wb(2048, 2048, 32768, 4) == 4 * 2048 * 2048 * 4
    assert wb(64, 64, 64, 4) == 0                  # one 64-element chunk
    assert wb(64, 64, 200, 4) == 4 * 64 * 64 * 4   # chunks of 64: 64, 64, 64, 8
    assert wb(64, 64, 136, 2) == 2 * 64 * 64 * 4   # chunks of 128: 128, 8
    assert wb(64, 64, 1000, 3) == 3 * 64 * 64 * 4  # chunks of 384
    assert wb(0, 64, 1000, 3) == 0 and wb(64, 64, 0, 3) == 0
    assert wb(-1, 8, 8, 2) == EINVAL
    assert wb(8, 8, 8, 0) == EUNSUP and wb(8, 8, 8, 65) == EUNSUP


@pytest.mark.parametrize("args,expected", [
    ((A, B, C, 64, 64, 512, 4, 0, 1 << 20), EINVAL),              # no workspace
    ((A, B, C, 64, 64, 512, 4, 0x40000000, 1000), EINVAL),        # too small
    ((A, B, C, 64, 64, 512, 4, 0x40000008, 1 << 20), EUNSUP),     # misaligned
    ((A, B, C, 64, 64, 512, 4, A, 1 << 20), EINVAL),              # overlaps A
    ((A, B, C, 64, 64, 512, 0, 0x40000000, 1 << 20), EUNSUP),     # splits out of range
    ((A, B, C, 64, 64, 512, 65, 0x40000000, 1 << 20), EUNSUP),
    ((A, B, C, 64, 12, 512, 4, 0x40000000, 1 << 20), EUNSUP),     # N % 8
    ((A, B, C, -1, 64, 512, 4, 0x40000000, 1 << 20), EINVAL),
    ((0, 0, 0, 0, 64, 512, 4, 0, 0), OK),                         # empty: nothing enqueued
])
def test_splitk_argument_checks(L, args, expected):
    assert L.pgemm_f16_splitk(*args, None) == expected


@pytest.mark.parametrize("args,expected", [
    ((A, B, C, 2048, 2048, 40960, 5), pg.PGEMM_ESCRATCH),   # 80 MiB of partials
    ((A, B, C, 64, 64, 512, 0), EUNSUP),                   # splits out of range
    ((A, B, C, 64, 12, 512, 4), EUNSUP),                   # N % 8
    ((A, B, A + 16, 64, 64, 512, 4), EINVAL),              # C overlaps A
    ((0, 0, 0, 0, 64, 512, 4), OK),                        # empty: nothing enqueued
])
def test_splitk_noalloc_argument_checks(L, args, expected):
    assert L.pgemm_f16_splitk_noalloc(*args, None) == expected


def test_splitk_default_splits(L):
    d = L.pgemm_f16_splitk_default_splits
    assert d(2048, 2048, 32768) == 4      # 64 tiles, chunks of 8192
    assert d(1024, 1024, 16384) == 4      # 16 tiles would want 16; chunks >= 4096
    assert d(2048, 2048, 2048) == 1       # short K
    assert d(4096, 4096, 16384) == 1      # 256 tiles already
    assert d(256, 256, 1 << 21) == 8      # capped at 8
    assert d(0, 8, 8) == 1
    assert d(-1, 8, 8) == EINVAL


def test_gemm_variant_range(L):
    assert L.pgemm_f16_variant(A, B, C, 8, 8, 8, -1, None) == EUNSUP
    assert L.pgemm_f16_variant(A, B, C, 8, 8, 8, L.pgemm_f16_num_variants() + 1, None) == EUNSUP


@pytest.mark.parametrize("x,y,z,n,expected", [
    (A, B, C, -1, EINVAL),
    (0, B, C, 4, EINVAL),
    (A, 0, C, 4, EINVAL),
    (A, B, 0, 4, EINVAL),
    (A, B, A + 4, 4, EINVAL),   # partial overlap with x
    (A, B, B - 4, 4, EINVAL),   # partial overlap with y
    (0, 0, 0, 0, OK),
])
def test_stream_add_argument_checks(L, x, y, z, n, expected):
    assert L.pstream_add(x, y, z, n, None) == expected


def test_stream_add_block_checks(L):
    assert L.pstream_add_blocked(A, B, C, 16, 0, None) == EUNSUP
    assert L.pstream_add_blocked(A, B, C, 16, 1000, None) == EUNSUP
    assert L.pstream_add_blocked(A, B, C, 16, (1 << 24) + 1024, None) == EUNSUP
    assert L.pstream_add_blocked(A, B, C, 0, 1024, None) == OK
    # 2^24 blocks of 256 lanes would reach 2^32 work-items in one launch
    X, Y, Z = 1 << 44, 2 << 44, 3 << 44  # far enough apart for these sizes
    assert L.pstream_add_blocked(X, Y, Z, 1024 << 24, 1024, None) == EUNSUP
    assert L.pstream_add_scalar(X, 1.0, Z, (8192 << 24) - 8191, None) == EUNSUP


def test_scalar_and_test_kernels_argument_checks(L):
    assert L.pstream_add_scalar(A, 1.0, A + 4, 4, None) == EINVAL
    assert L.pstream_add_scalar(0, 1.0, C, 4, None) == EINVAL
    assert L.pstream_add_scalar(A, 1.0, C, -2, None) == EINVAL
    assert L.pstream_add_scalar(0, 1.0, 0, 0, None) == OK
    assert L.pgemm_test_fill_f32(0, 1.0, 4, None) == EINVAL
    assert L.pgemm_test_fill_f32(0, 1.0, 0, None) == OK
    assert L.pgemm_test_iota_f32(0, 4, None) == EINVAL
    assert L.pgemm_test_iota_f32(A, -1, None) == EINVAL


def test_reduce_argument_checks(L):
    assert L.preduce_sum_f32(A, C, -1, 8, None) == EINVAL
    assert L.preduce_sum_f32(A, C, 8, -8, None) == EINVAL
    assert L.preduce_sum_f32(0, C, 8, 8, None) == EINVAL
    assert L.preduce_sum_f32(A, 0, 8, 8, None) == EINVAL
    assert L.preduce_sum_f32(A, A + 64, 8, 8, None) == EINVAL      # o inside x
    assert L.preduce_sum_f32(A, C, 8, 0, None) == OK                # nothing to do
    assert L.preduce_sum_f32(A, C, 1 << 30, 1 << 20, None) == EUNSUP
    assert L.preduce_sum_f32(A, C, 1, 1 << 36, None) == EUNSUP     # 2^24 workgroups of 4096


def test_header_compiles_as_c99_and_links(L, tmp_path):
    """include/pgemm.h is a plain C header: a C99 program that includes it
    compiles with gcc -pedantic, links against libpgemm.so and gets the
    documented statuses from the host-side checks."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(root, "include"),
                    os.path.join(root, "tests", "c_abi_check.c"),
                    "-L", libdir, "-lpgemm", "-Wl,-rpath," + libdir, "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert "c abi ok" in res.stdout


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    a = torch.zeros((8, 8), dtype=torch.float16)
    with pytest.raises(ValueError):
        pg.pgemm_f16(a, a)
    with pytest.raises(ValueError):
        pg.pstream_add(torch.zeros(4), torch.zeros(4))


def test_product_package_does_not_reference_the_oracle():
    pkg = os.path.dirname(pg.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "oracle_" not in text, f
