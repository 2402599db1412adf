"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: bit-exact for the streaming add, x + c, fill and iota; for the GEMM
|gpu - oracle| <= 5e-3 * (|oracle| + 1) per element on inputs in [-1, 1]
(and, tighter, the a-priori bound of fp32 accumulation: assert_fp32_bound),
bit-exact where the exact result is an fp16 value that fp32 accumulation
reaches exactly (identity, ones, power-of-two rank-1).  Full-size GEMMs are
checked on a deterministic sample of outputs computed one by one by the
oracle (the headline 4096^3 configuration also on every output); smaller
shapes that span several tiles and a ragged edge are checked element by
element."""
import sys

import numpy as np
import pytest

import oracle
import software_pipelined_tiled_pgemm_amd as pg
from software_pipelined_tiled_pgemm_amd import inputs
from tests import _golden
from tests._bounds import fp32_bound_violations, ulp16  # noqa: F401

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    pg.lib()  # raises if the library is missing: no fallback
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gemm(A, B, variant=0, C=None):
    say("  gemm M=%d N=%d K=%d variant=%d" % (A.shape[0], B.shape[1], A.shape[1], variant))
    tA = A if isinstance(A, torch.Tensor) else dev(A)
    tB = B if isinstance(B, torch.Tensor) else dev(B)
    return host(pg.pgemm_f16_variant(tA, tB, variant, C=C))


def assert_close(got, ref, what=""):
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    ok = np.abs(g - r) <= TOL * (np.abs(r) + 1.0)
    if not ok.all():
        idx = np.argwhere(~ok)[:8]
        detail = ", ".join("%s: gpu %r oracle %r" % (tuple(i), g[tuple(i)], r[tuple(i)]) for i in idx)
        pytest.fail("%s: %d of %d outside tolerance; first: %s" % (what, (~ok).sum(), ok.size, detail))


def assert_fp32_bound(got, ref, Sabs, K, what=""):
    bad = fp32_bound_violations(got, ref, Sabs, K)
    if bad.any():
        pytest.fail("%s: %d of %d outside the fp32 accumulation bound" % (what, bad.sum(), bad.size))


def ulp_distance16(a, b):
    """Distance in representable fp16 steps between same-shape float16
    arrays (sign-magnitude bit patterns mapped to one ordered integer line,
    so +0 and -0 coincide and values of opposite sign near zero are close)."""
    def ordered(x):
        u = np.ascontiguousarray(x).view(np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def bits_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


VARIANTS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11]
# Variants that must agree bit for bit: the same matrix instruction, so the
# same grouping of each output's K sum (32x32x16: 1-6; 16x16x32: 7-11).
FAMILIES = [[1, 2, 3, 4, 5, 6], [7, 8, 9, 10, 11]]


# ------------------------------------------------------------ worked examples

def test_fill_42_matches_pages():
    say("fill_42")
    got = host(pg.pgemm_test_fill_f32(128, 42.0))
    assert bits_equal(got, _golden.values_f32("fill_42.txt"))


def test_iota_matches_pages():
    say("iota 1024")
    got = host(pg.pgemm_test_iota_f32(1024))
    assert bits_equal(got, _golden.values_f32("iota_1024.txt"))


@pytest.mark.parametrize("n", [1, 127, 129, 3_000_001, (1 << 24) + 3])
def test_iota_large_vs_oracle(n):
    say("iota n=%d" % n)
    assert bits_equal(host(pg.pgemm_test_iota_f32(n)), oracle.iota_f32(n))


def test_iota_past_2_31_elements():
    """More elements than 2^31: the launch widens each workgroup's slice so
    that the grid stays under 2^32 work-items (with 128 elements per
    workgroup it would not launch)."""
    n = (1 << 31) + 5
    say("iota n=%d" % n)
    o = torch.empty(n, dtype=torch.float32, device="cuda:0")
    got = host(pg.pgemm_test_iota_f32(n, out=o))
    del o
    assert bits_equal(got, oracle.iota_f32(n))


def test_ones_add_512_matches_pages():
    say("ones+ones 512x512")
    g = _golden.keyed("ones_add_512.txt")
    shape = tuple(int(s) for s in g["shape"])
    x = torch.full(shape, float(g["operand"][0]), dtype=torch.float32, device="cuda:0")
    z = host(pg.pstream_add(x, x))
    assert np.all(z == np.float32(g["expected"][0]))


# ------------------------------------------------------------ streaming add

def test_stream_add_full_size_bit_exact():
    say("stream add 8192x8192 uniform[-1,1]")
    x, y = inputs.stream_inputs((8192, 8192))
    got = host(pg.pstream_add(dev(x), dev(y)))
    assert bits_equal(got, oracle.add_f32(x, y))


@pytest.mark.parametrize("bm", [128, 256, 512])
def test_stream_add_block_sizes(bm):
    # The guide's section 6.1 checks x + y at 128, 256 and 512 blocks of a
    # 4096 x 4096 array; here each workgroup block holds bm*bm elements.
    say("stream add 4096x4096 block %dx%d" % (bm, bm))
    x, y = inputs.stream_inputs((4096, 4096), 10, 11)
    got = host(pg.pstream_add_blocked(dev(x), dev(y), bm * bm))
    assert bits_equal(got, oracle.add_f32(x, y))


SPECIAL = np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-40, 1.1754942e-38, 3.4028235e38,
                    -3.4028235e38, np.inf, -np.inf, 0.5, 2.0 ** -24, 7.0], dtype=np.float32)


def test_stream_add_special_values():
    say("stream add special values")
    x = np.repeat(SPECIAL, SPECIAL.size)
    y = np.tile(SPECIAL, SPECIAL.size)
    got = host(pg.pstream_add(dev(x), dev(y)))
    assert bits_equal(got, oracle.add_f32(x, y))


@pytest.mark.parametrize("n", [1, 3, 4, 1023, 1025, 262143, 262145, 1_000_003])
def test_stream_add_ragged_lengths(n):
    say("stream add n=%d" % n)
    x, y = inputs.stream_inputs(n, 20, 21)
    got = host(pg.pstream_add(dev(x), dev(y)))
    assert bits_equal(got, oracle.add_f32(x, y))


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_stream_add_misaligned_views(offset):
    say("stream add misaligned offset %d" % offset)
    n = 100_000
    x, y = inputs.stream_inputs(n + offset, 30, 31)
    tx, ty = dev(x)[offset:], dev(y)[offset:]
    z = torch.empty(n + offset, dtype=torch.float32, device="cuda:0")[offset:]
    got = host(pg.pstream_add(tx, ty, z=z))
    assert bits_equal(got, oracle.add_f32(x[offset:], y[offset:]))


def test_stream_add_in_place():
    say("stream add in place")
    x, y = inputs.stream_inputs(1 << 20, 40, 41)
    tx, ty = dev(x), dev(y)
    pg.pstream_add(tx, ty, z=tx)
    assert bits_equal(host(tx), oracle.add_f32(x, y))
    tx2 = dev(x)
    pg.pstream_add(tx2, ty, z=ty)
    assert bits_equal(host(ty), oracle.add_f32(x, y))


def test_stream_add_poisoned_output_overwritten():
    say("stream add NaN-poisoned output")
    x, y = inputs.stream_inputs(1 << 20, 42, 43)
    z = torch.full((1 << 20,), float("nan"), device="cuda:0")
    assert bits_equal(host(pg.pstream_add(dev(x), dev(y), z=z)), oracle.add_f32(x, y))


def test_stream_add_scalar_full_size_in_place():
    say("x + 1 8192x8192, out of place and in place")
    x, _ = inputs.stream_inputs((8192, 8192))
    ref = oracle.add_scalar_f32(x, 1.0)
    tx = dev(x)
    assert bits_equal(host(pg.pstream_add_scalar(tx, 1.0)), ref)
    pg.pstream_add_scalar(tx, 1.0, z=tx)
    assert bits_equal(host(tx), ref)


@pytest.mark.parametrize("n", [1, 5, 1029, 262147])
def test_stream_add_scalar_ragged_and_specials(n):
    say("x + c n=%d" % n)
    x = np.resize(np.concatenate([SPECIAL, inputs.uniform_f32(n, 50)]), n).astype(np.float32)
    for c in (1.0, -0.0, 3.0e38):
        assert bits_equal(host(pg.pstream_add_scalar(dev(x), c)), oracle.add_scalar_f32(x, c))


# Arrays of more than 4 GiB: element offsets past 2**30 floats.  x and y come
# from the index hash (viewed as rows of 1029), y scaled by float32(0.3) so
# that the sums round; the oracle rebuilds the sampled elements on the host.
BIG_N_COLS, BIG_N_ROWS = 1029, 1043500  # n = 1 073 761 500 > 2**30


def _big_vector(seed):
    t = inputs.hashed_f16_torch(BIG_N_ROWS, BIG_N_COLS, seed, "cuda:0").view(-1).float()
    return t if seed == inputs.SEED_A else t.mul_(np.float32(0.3))


def _big_vector_at(idx, seed):
    rows, inv = np.unique(idx // BIG_N_COLS, return_inverse=True)
    v = inputs.hashed_f16(rows, np.arange(BIG_N_COLS), seed)[inv, idx % BIG_N_COLS].astype(np.float32)
    return v if seed == inputs.SEED_A else v * np.float32(0.3)


def _big_sample(n, seed=5):
    rng = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(4096), np.arange(n - 4096, n),
                           np.arange((1 << 30) - 2048, (1 << 30) + 2048)])
    return np.unique(np.concatenate([edge, rng.integers(0, n, 16384)]))


def test_streaming_beyond_4gib():
    n = BIG_N_ROWS * BIG_N_COLS
    say("stream add, x + c and reduction on %d floats (%.2f GB per array)" % (n, 4e-9 * n))
    tx, ty = _big_vector(inputs.SEED_A), _big_vector(inputs.SEED_B)
    idx = _big_sample(n)
    tidx = torch.from_numpy(idx).to("cuda:0")
    x, y = _big_vector_at(idx, inputs.SEED_A), _big_vector_at(idx, inputs.SEED_B)
    assert bits_equal(host(tx[tidx]), x) and bits_equal(host(ty[tidx]), y)
    z = torch.full_like(tx, float("nan"))
    pg.pstream_add(tx, ty, z=z)
    assert bits_equal(host(z[tidx]), oracle.add_f32(x, y))
    pg.pstream_add_scalar(ty, 1.0, z=z)
    assert bits_equal(host(z[tidx]), oracle.add_scalar_f32(y, 1.0))
    del z
    # (2, h) reductions over the first 2h elements: output j from inputs j and
    # h + j; h = n/2 (not a multiple of 4: scalar path) and a multiple of 4
    # (float4 path)
    for h in (n // 2, n // 8 * 4):
        say("  reduction (2, %d)" % h)
        o = pg.preduce_sum_f32(ty[:2 * h].view(2, h))
        j = idx[idx < h]
        pair = np.stack([_big_vector_at(j, inputs.SEED_B), _big_vector_at(j + h, inputs.SEED_B)])
        assert bits_equal(host(o[torch.from_numpy(j).to("cuda:0")]), oracle.sum_axis0_f32(pair))


def test_sum_axis0_scalar_path_past_2_32_outputs():
    """More than 2^32 outputs on the scalar path (n not a multiple of 4): the
    launch caps the grid below 2^32 work-items and each lane walks several
    outputs (grid-stride loop).  x is the index hash viewed as (2, n), the
    second slice scaled by float32(0.3) so that the sums round; the oracle
    sums the gathered columns."""
    torch.cuda.empty_cache()
    n = (1 << 32) + 3
    rows = -(-2 * n // BIG_N_COLS)
    say("sum axis 0 of (2, %d) f32 (%.1f GB of input)" % (n, 8e-9 * n))
    x = inputs.hashed_f16_torch(rows, BIG_N_COLS, inputs.SEED_A, "cuda:0").view(-1)[:2 * n].float()
    x[n:].mul_(np.float32(0.3))
    o = pg.preduce_sum_f32(x.view(2, n))
    rng = np.random.default_rng(9)
    j = np.unique(np.concatenate([np.arange(2048), np.arange(n - 2048, n),
                                  np.arange((1 << 32) - 2048, (1 << 32) + 3),
                                  rng.integers(0, n, 16384)]))
    a = _big_vector_at(j, inputs.SEED_A)
    b = _big_vector_at(j + n, inputs.SEED_A) * np.float32(0.3)
    tj = torch.from_numpy(j).to("cuda:0")
    assert bits_equal(host(x[tj]), a) and bits_equal(host(x[tj + n]), b)
    assert bits_equal(host(o[tj]), oracle.sum_axis0_f32(np.stack([a, b])))
    del x, o
    torch.cuda.empty_cache()


# ------------------------------------------------------------ GEMM, element by element

SMALL_SHAPES = [
    (256, 256, 256),   # the 256^3 config: 128x128x64 tiles -> 2x2 grid, 4 K steps
    (8, 8, 8),
    (1, 8, 8),
    (33, 40, 72),
    (128, 128, 64),
    (129, 136, 64),
    (300, 264, 520),
    (255, 248, 1000),
    (520, 776, 136),
    (64, 1024, 8),
    # K-loop structure boundaries (steps of 32; steady-state periods unrolled
    # by five, then run-time steady-state periods, then tail periods):
    (136, 264, 448),   # 14 steps: one unrolled pass, then tail periods
    (264, 136, 416),   # 13 steps: no unrolled pass, odd step count
    (256, 256, 480),   # 15 steps
    (128, 384, 832),   # 26 steps: two unrolled passes, a run-time one, tail
    # the same boundaries of the 7- and 9-slot rings (variants 10, 11: a
    # pass unrolls 2S steps and needs K/32 >= 3S - 1 steps)
    (264, 136, 608),   # 19 steps: S = 7 runs no unrolled pass
    (136, 264, 640),   # 20 steps: S = 7 one unrolled pass
    (200, 200, 800),   # 25 steps: S = 9 no unrolled pass
    (128, 256, 1184),  # 37 steps: S = 7 two passes, S = 9 one
    (72, 136, 192),    # 6 steps = S - 1 for S = 7: the steady-state prologue
    # extreme aspect ratios: one row, the narrowest C, one tile row/column
    # with long K
    (1, 8192, 4096),
    (8192, 8, 4096),
    (3, 4104, 1032),
    (4100, 24, 2056),
]


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_gemm_small_shapes_vs_full_oracle(M, N, K):
    A, B = inputs.gemm_inputs(M, N, K)
    ref, _ = oracle.gemm_f16(A, B)
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    outs = {}
    for v in VARIANTS:
        got = gemm(A, B, v)
        assert_close(got, ref, "M=%d N=%d K=%d variant %d" % (M, N, K, v))
        assert_fp32_bound(got, ref, Sabs, K, "M=%d N=%d K=%d variant %d" % (M, N, K, v))
        outs[v] = got
    # inside a family the K order of an element depends neither on the tile
    # size nor on the pipeline (LDS-DMA ring vs register staging): any
    # difference would be a race on a reused buffer
    for fam in FAMILIES:
        for v in fam[1:]:
            assert bits_equal(outs[fam[0]], outs[v]), "variants %d and %d differ" % (fam[0], v)


# Variant 9 (persistent) walks several tiles per workgroup only when there
# are more 256x256 tiles than compute units (256 on MI355X): ragged edges on
# both sides, K below the four prologue steps, K with a tail step, and four
# tiles per workgroup.  The next tile's first copies overlap the previous
# tile's drain, so a race there would show as a difference from variant 8.
@pytest.mark.parametrize("M,N,K", [(4400, 4360, 96), (4400, 4360, 200), (4136, 4616, 1048)])
def test_persistent_variant_several_tiles_vs_oracle(M, N, K):
    say("persistent %dx%dx%d" % (M, N, K))
    A, B = inputs.gemm_inputs(M, N, K, seed_a=M + K, seed_b=N + K)
    ref, _ = oracle.gemm_f16(A, B)
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    got = gemm(A, B, 9)
    assert_close(got, ref, "persistent M=%d N=%d K=%d" % (M, N, K))
    assert_fp32_bound(got, ref, Sabs, K, "persistent M=%d N=%d K=%d" % (M, N, K))
    assert bits_equal(got, gemm(A, B, 8)), "variants 8 and 9 differ"


def test_persistent_variant_four_tiles_per_workgroup():
    M = N = 8192
    K = 520
    say("persistent %dx%dx%d" % (M, N, K))
    A, B = inputs.gemm_inputs(M, N, K, seed_a=95, seed_b=96)
    tA, tB = dev(A), dev(B)
    got9 = host(pg.pgemm_f16_variant(tA, tB, 9))
    assert bits_equal(got9, host(pg.pgemm_f16_variant(tA, tB, 8))), "variants 8 and 9 differ"
    rows = np.array([0, 255, 256, 4095, 4096, 8191])
    ref, _ = oracle.gemm_f16(A[rows], B)
    assert_close(got9[rows], ref, "persistent 8192^2 x 520, sampled rows")


def test_gemm_special_values_all_variants():
    # Not part of any benchmark input, but IEEE semantics must hold: NaN
    # where the exact sum is undefined, +-inf where it overflows fp16 or
    # includes an infinite product, the rest within the bounds.
    M, N, K = 136, 144, 264
    say("gemm with NaN, +-inf and fp16-overflowing sums, %dx%dx%d" % (M, N, K))
    A, B = inputs.gemm_inputs(M, N, K, seed_a=70, seed_b=71)
    A, B = A.copy(), B.copy()
    A[3, 10] = np.inf
    A[5, 20] = np.nan
    B[30, 7] = -np.inf
    A[9, :] = 300.0   # row 9 times column 11 sums to 264 * 90000: fp16 overflow
    B[:, 11] = 300.0
    B[:, 12] = -300.0
    ref, _ = oracle.gemm_f16(A, B)
    r = ref.astype(np.float64)
    special = ~np.isfinite(r)
    assert np.isnan(r).sum() > 0 and np.isposinf(r).sum() > 0 and np.isneginf(r).sum() > 0
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    for v in VARIANTS:
        got = gemm(A, B, v).astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(r)), "variant %d: NaN positions" % v
        inf = np.isinf(r)
        assert np.array_equal(got[inf], r[inf]), "variant %d: infinities" % v
        fin = ~special
        assert_close(got[fin], r[fin], "variant %d finite part" % v)
        assert_fp32_bound(got[fin], r[fin], Sabs[fin], K, "variant %d finite part" % v)


@pytest.mark.parametrize("v", VARIANTS)
def test_gemm_k_zero_gives_zeros(v):
    say("gemm K=0")
    C = torch.full((40, 24), float("nan"), dtype=torch.float16, device="cuda:0")
    A = torch.empty((40, 0), dtype=torch.float16, device="cuda:0")
    B = torch.empty((0, 24), dtype=torch.float16, device="cuda:0")
    got = host(pg.pgemm_f16_variant(A, B, v, C=C))
    assert np.all(got.view(np.uint16) == 0)


def _finite_f16_no_negzero(rng, shape):
    h = rng.integers(0, 65536, size=shape, dtype=np.uint32).astype(np.uint16)
    h = h[((h & 0x7C00) != 0x7C00)]
    h = np.resize(h, shape)
    h[h == 0x8000] = 0
    return h.view(np.float16)


@pytest.mark.parametrize("v", VARIANTS)
@pytest.mark.parametrize("M,N", [(256, 256), (296, 136)])
def test_gemm_identity_bit_exact_with_subnormals(v, M, N):
    rng = np.random.default_rng(60)
    B = _finite_f16_no_negzero(rng, (M, N))
    I = np.eye(M, dtype=np.float16)
    ref, _ = oracle.gemm_f16(I, B)
    got = gemm(I, B, v)
    assert bits_equal(ref, B)  # the oracle's own closed form
    assert bits_equal(got, ref), "identity: first mismatches %s" % np.argwhere(got.view(np.uint16) != ref.view(np.uint16))[:8]


@pytest.mark.parametrize("v", VARIANTS)
def test_gemm_permutation_bit_exact(v):
    rng = np.random.default_rng(61)
    M, N = 264, 200
    perm = rng.permutation(M)
    P = np.zeros((M, M), np.float16)
    P[np.arange(M), perm] = 1
    B = inputs.uniform_f16((M, N), 62)
    got = gemm(P, B, v)
    ref, _ = oracle.gemm_f16(P, B)
    assert bits_equal(got, ref)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (2048, 2048, 32768), (8192, 8192, 8192)])
def test_gemm_ones_full_size_exact(M, N, K):
    say("gemm ones %dx%dx%d" % (M, N, K))
    A = torch.ones((M, K), dtype=torch.float16, device="cuda:0")
    B = torch.ones((K, N), dtype=torch.float16, device="cuda:0")
    C = pg.pgemm_f16(A, B)
    torch.cuda.synchronize()
    assert bool((C == K).all().item())
    # the oracle's closed form at the same K (a few elements)
    ref, _ = oracle.gemm_f16(np.ones((2, K), np.float16), np.ones((K, 3), np.float16))
    assert np.all(ref.astype(np.float64) == K)


@pytest.mark.parametrize("K", [4096, 32768])
def test_gemm_rank1_powers_of_two_exact(K):
    say("gemm rank-1 K=%d" % K)
    rng = np.random.default_rng(K + 1)
    M, N = 264, 520
    u = rng.choice([-1.0, -0.5, 0.5, 1.0], M)
    v = rng.choice([-1.0, -0.5, 0.5, 1.0], N)
    A = np.repeat(u[:, None], K, axis=1).astype(np.float16)
    B = np.repeat(v[None, :], K, axis=0).astype(np.float16)
    got = gemm(A, B)
    assert np.array_equal(got.astype(np.float64), K * np.outer(u, v))


@pytest.mark.parametrize("v", VARIANTS)
def test_gemm_poisoned_output_overwritten(v):
    A, B = inputs.gemm_inputs(300, 264, 136, seed_a=70, seed_b=71)
    C = torch.full((300, 264), float("nan"), dtype=torch.float16, device="cuda:0")
    got = gemm(A, B, v, C=C)
    ref, _ = oracle.gemm_f16(A, B)
    assert_close(got, ref, "poisoned C")


def test_gemm_repeat_and_stream_determinism():
    A, B = inputs.gemm_inputs(1024, 1024, 1024, seed_a=80, seed_b=81)
    tA, tB = dev(A), dev(B)
    first = host(pg.pgemm_f16(tA, tB))
    for _ in range(3):
        assert bits_equal(host(pg.pgemm_f16(tA, tB)), first)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = pg.pgemm_f16(tA, tB)
    s.synchronize()
    assert bits_equal(C.cpu().numpy(), first)


def test_gemm_row_subset_consistency():
    # Rows of a 256-row product equal the same rows of a 4096-row product
    # made with the same tile configuration.
    A, B = inputs.gemm_inputs(4096, 1024, 512, seed_a=90, seed_b=91)
    for v in VARIANTS:
        full = gemm(A, B, v)
        part = gemm(A[:256], B, v)
        assert bits_equal(full[:256], part)


def test_gemm_device_pointer_checks():
    say("gemm argument checks with device pointers")
    L = pg.lib()
    buf = torch.zeros(1 << 16, dtype=torch.float16, device="cuda:0")
    p = buf.data_ptr()
    s = None
    assert L.pgemm_f16(p + 2, p + 4096, p + 8192, 8, 8, 8, s) == pg.PGEMM_EUNSUPPORTED
    assert L.pgemm_f16(p, p + 4096, p + 64, 8, 8, 8, s) == pg.PGEMM_EINVAL
    torch.cuda.synchronize()


# ------------------------------------------------------------ GEMM at full size (sampled)

FULL_CONFIGS = [
    ("4096^3 uniform", 4096, 4096, 4096, "uniform"),
    ("8192^3 normal(0,1/sqrt(K))", 8192, 8192, 8192, "normal"),
    ("2048x2048x32768 uniform (long K)", 2048, 2048, 32768, "uniform"),
]


@pytest.mark.parametrize("name,M,N,K,dist", FULL_CONFIGS, ids=[c[0] for c in FULL_CONFIGS])
def test_gemm_full_size_sampled(name, M, N, K, dist):
    say("gemm full size %s" % name)
    A, B = inputs.gemm_inputs(M, N, K, dist)
    got = gemm(A, B)  # automatic variant: what the benchmark times
    I, J = inputs.sample_points(M, N, 8192)
    ref, S = oracle.gemm_f16_points(A, B, I, J)
    assert_close(got[I, J], ref, name)
    # diagnostics on the sample: error in fp16 ulps of the oracle value
    d = ulp_distance16(got[I, J], ref)
    say("  sample %d points: max |ulp diff| %d, frac exact %.4f" % (I.size, d.max(), np.mean(d == 0)))
    g = got[I, J].astype(np.float64)
    say("  relative Frobenius error against the exact sums: %.3e" % (np.linalg.norm(g - S) / np.linalg.norm(S)))
    _, Sabs = oracle.gemm_f16_points(np.abs(A), np.abs(B), I, J)
    assert_fp32_bound(got[I, J], ref, Sabs, K, name)


def _random_auto_shapes(seed, n):
    """Seeded ragged shapes across tile and wave boundaries (M any size;
    N and K multiples of 8), at most 2e11 multiply-adds each."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(0, 48)) * 128 + int(rng.choice([1, 8, 72, 128, 136]))
        N = int(rng.integers(0, 48)) * 128 + int(rng.choice([8, 64, 120, 128]))
        K = int(rng.choice([8, 56, 256, 1032, 4096, 8200]))
        if M * N * K <= 2e11:
            out.append((M, N, K))
    return out


def test_gemm_auto_random_shapes_sampled():
    """The automatic path (the variant the tuned table and the fill rule
    pick, and the row split) on random ragged shapes: every tile's corners,
    four whole rows and columns and random outputs against the oracle."""
    chosen = set()
    for (M, N, K) in _random_auto_shapes(23, 30):
        head, hv, tv = pg.pgemm_f16_plan(M, N, K, 0)
        chosen.add(hv)
        say("  auto %dx%dx%d: variant %d%s" % (M, N, K, hv,
                                              " + %d rows on %d" % (M - head, tv) if tv else ""))
        A, B = inputs.gemm_inputs(M, N, K, seed_a=M + 1, seed_b=N + 2)
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
        got = host(pg.pgemm_f16(dev(A), dev(B), C=C))
        I, J = inputs.sample_points(M, N, 1024, full_rows=4, full_cols=4, tile=128)
        ref, _ = oracle.gemm_f16_points(A, B, I, J)
        what = "auto %dx%dx%d" % (M, N, K)
        assert_close(got[I, J], ref, what)
        _, Sabs = oracle.gemm_f16_points(np.abs(A), np.abs(B), I, J)
        assert_fp32_bound(got[I, J], ref, Sabs, K, what)
    say("  variants chosen: %s" % sorted(chosen))


def test_gemm_every_variant_at_4096_families_bit_identical():
    """All variants at the headline size: bit-identical inside each
    matrix-instruction family (the same K grouping at 256 tiles of 256x256
    or 1024 of 128x128, one or two workgroups per CU, persistent or not,
    5-, 7- or 9-slot rings), and each family within the bounds on the
    full-size sample."""
    M = N = K = 4096
    A, B = inputs.gemm_inputs(M, N, K)
    tA, tB = dev(A), dev(B)
    I, J = inputs.sample_points(M, N, 8192)
    ref, _ = oracle.gemm_f16_points(A, B, I, J)
    _, Sabs = oracle.gemm_f16_points(np.abs(A), np.abs(B), I, J)
    for fam in FAMILIES:
        first = None
        for v in fam:
            C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
            got = gemm(tA, tB, v, C=C)
            if first is None:
                first = got
                assert_close(got[I, J], ref, "variant %d at 4096^3" % v)
                assert_fp32_bound(got[I, J], ref, Sabs, K, "variant %d at 4096^3" % v)
            else:
                assert bits_equal(got, first), "variant %d differs from variant %d at 4096^3" % (v, fam[0])


def test_gemm_4096_every_output_vs_oracle():
    """The headline configuration (4096^3, U[-1,1]) on every one of its
    16,777,216 outputs: the whole result against the oracle, as the
    quickstart's matmul example checks its whole result against a @ b.
    Automatic variant (what the benchmark times), C poisoned with NaN first."""
    M = N = K = 4096
    say("gemm 4096^3 uniform, every output against the oracle (%d oracle threads)" % oracle.threads())
    A, B = inputs.gemm_inputs(M, N, K, "uniform")
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda:0")
    got = gemm(A, B, C=C)
    assert not np.isnan(got).any(), "NaN left in C"
    ref, S = oracle.gemm_f16(A, B)
    assert_close(got, ref, "4096^3 every output")
    d = ulp_distance16(got, ref)
    say("  max |ulp diff| %d, frac exact %.4f, relative Frobenius error against the exact sums %.3e"
        % (d.max(), np.mean(d == 0), np.linalg.norm(got.astype(np.float64) - S) / np.linalg.norm(S)))
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    assert_fp32_bound(got, ref, Sabs, K, "4096^3 every output")


# ------------------------------------------------------------ automatic row split

# Shapes whose 256x256 tiles leave most of the last wave idle: pgemm_f16 runs
# the head rows with the 256x256 variant and the rest with the 128x128
# variant of the same family.  The result must be bit-identical to the
# 256x256 variant over all rows, and within the bound of the oracle.
ROW_SPLIT_CASES = [(4392, 4352, 4096), (6144, 6144, 6144)]


@pytest.mark.parametrize("M,N,K", ROW_SPLIT_CASES)
def test_gemm_auto_row_split(M, N, K):
    head, hv, tv = pg.pgemm_f16_plan(M, N, K)
    say("gemm auto %dx%dx%d: head %d rows on variant %d, tail on variant %d" % (M, N, K, head, hv, tv))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert 0 < head < M and tv != 0, "the split should be taken on 256 CUs"
    A, B = inputs.gemm_inputs(M, N, K)
    tA, tB = dev(A), dev(B)
    auto = gemm(tA, tB)
    assert bits_equal(auto, gemm(tA, tB, hv))
    I, J = inputs.sample_points(M, N, 4096, seed=6, full_rows=8, full_cols=8)
    ref, _ = oracle.gemm_f16_points(A, B, I, J)
    assert_close(auto[I, J], ref, "auto %dx%dx%d" % (M, N, K))


# ------------------------------------------------------------ one GPU's row shard

# Split G ways by rows of C, GPU g computes A's row block g times all of B
# (output tiles are independent).  One GPU's share of each product below is
# its (M/8) x N x K block: checked against the oracle with the variant chosen
# for the shard shape, and, run with the variant of the whole product,
# bit-identical to the same rows of the whole product.
SHARD_CASES = [(4096, 4096, 4096, "uniform"), (2048, 2048, 32768, "uniform")]


@pytest.mark.parametrize("M,N,K,dist", SHARD_CASES, ids=["%dx%dx%d" % c[:3] for c in SHARD_CASES])
def test_gemm_row_shards(M, N, K, dist):
    G = 8
    L = pg.lib()
    A, B = inputs.gemm_inputs(M, N, K, dist)
    tA, tB = dev(A), dev(B)
    v_full = L.pgemm_f16_choose_variant(M, N, K)
    full = gemm(tA, tB, v_full)
    m = M // G
    say("gemm %d-way row shards of %dx%dx%d: shard variant %d, whole-product variant %d"
        % (G, M, N, K, L.pgemm_f16_choose_variant(m, N, K), v_full))
    for g in (0, 3, G - 1):
        rows = slice(g * m, (g + 1) * m)
        shard = gemm(tA[rows], tB)  # automatic variant at the shard shape
        I, J = inputs.sample_points(m, N, 2048, seed=10 + g, full_rows=8, full_cols=8)
        ref, _ = oracle.gemm_f16_points(A[rows], B, I, J)
        assert_close(shard[I, J], ref, "shard %d of %dx%dx%d" % (g, M, N, K))
        same = gemm(tA[rows], tB, v_full)
        assert np.array_equal(same.view(np.uint16), full[rows].view(np.uint16)), "shard %d" % g


# ------------------------------------------------------------ operands beyond 4 GiB

# One operand of more than 4 GiB per case, so byte offsets into A, B or C pass
# 32 bits (every variant).  Elements come from the index hash, so the oracle
# rebuilds only the rows of A and columns of B that the sampled outputs need.
BIG_CASES = [("A", 135000, 264, 16384), ("B", 136, 1048584, 2048), ("C", 65600, 32776, 64)]
BIG_SPLITS = {"A": 4, "B": 2, "C": None}  # split-K too where K has several chunks


@pytest.mark.parametrize("which,M,N,K", BIG_CASES, ids=["%s over 4 GiB" % c[0] for c in BIG_CASES])
def test_gemm_operand_beyond_4gib(which, M, N, K):
    say("gemm with %s over 4 GiB: M=%d N=%d K=%d" % (which, M, N, K))
    tA = inputs.hashed_f16_torch(M, K, inputs.SEED_A, "cuda:0")
    tB = inputs.hashed_f16_torch(K, N, inputs.SEED_B, "cuda:0")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    assert {"A": tA, "B": tB, "C": C}[which].numel() * 2 > 1 << 32
    I, J = inputs.sample_points(M, N, 2048, seed=3, full_rows=0, full_cols=0)
    rows, Iu = np.unique(I, return_inverse=True)
    cols, Ju = np.unique(J, return_inverse=True)
    ref, _ = oracle.gemm_f16_points(inputs.hashed_f16(rows, np.arange(K), inputs.SEED_A),
                                    inputs.hashed_f16(np.arange(K), cols, inputs.SEED_B), Iu, Ju)
    tI, tJ = torch.from_numpy(I).to("cuda:0"), torch.from_numpy(J).to("cuda:0")
    for v in [0] + VARIANTS:
        say("  variant %d" % v)
        C.fill_(float("nan"))
        pg.pgemm_f16_variant(tA, tB, v, C=C)
        assert_close(host(C[tI, tJ]), ref, "%s over 4 GiB, variant %d" % (which, v))
    if BIG_SPLITS[which]:
        say("  split-K, %d splits" % BIG_SPLITS[which])
        C.fill_(float("nan"))
        pg.pgemm_f16_splitk(tA, tB, BIG_SPLITS[which], C=C)
        assert_close(host(C[tI, tJ]), ref, "%s over 4 GiB, split-K" % which)


# ------------------------------------------------------------ split-K GEMM

def splitk(A, B, splits):
    say("  gemm split-K M=%d N=%d K=%d splits=%d" % (A.shape[0], B.shape[1], A.shape[1], splits))
    tA = A if isinstance(A, torch.Tensor) else dev(A)
    tB = B if isinstance(B, torch.Tensor) else dev(B)
    return host(pg.pgemm_f16_splitk(tA, tB, splits))


# (M, N, K, splits): several tiles, ragged edges, K not a multiple of the
# 64-element chunk granule, more splits than chunks, an odd number of steps
# per chunk, and both tile sizes of the split path (few and many tiles).
SPLITK_CASES = [(64, 64, 512, 2), (200, 136, 1000, 3), (256, 256, 4096, 4), (300, 264, 2056, 7),
                (520, 776, 136, 2), (128, 128, 64, 4), (96, 520, 1088, 5), (1024, 1024, 2048, 2)]


@pytest.mark.parametrize("M,N,K,splits", SPLITK_CASES)
def test_gemm_splitk_vs_full_oracle(M, N, K, splits):
    A, B = inputs.gemm_inputs(M, N, K)
    ref, _ = oracle.gemm_f16(A, B)
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    got = splitk(A, B, splits)
    assert_close(got, ref, "split-K %dx%dx%d/%d" % (M, N, K, splits))
    assert_fp32_bound(got, ref, Sabs, K, "split-K %dx%dx%d/%d" % (M, N, K, splits))
    assert bits_equal(got, splitk(A, B, splits)), "split-K is not deterministic"


def test_gemm_splitk_one_chunk_is_pgemm():
    A, B = inputs.gemm_inputs(256, 264, 64)
    assert pg.pgemm_f16_splitk_workspace_bytes(256, 264, 64, 4) == 0
    assert bits_equal(splitk(A, B, 4), gemm(A, B))
    A, B = inputs.gemm_inputs(128, 128, 1024)
    assert bits_equal(splitk(A, B, 1), gemm(A, B))


def test_gemm_splitk_identity_and_ones_exact():
    # identity: each output has one non-zero product, in one chunk -> exact,
    # subnormals included (no -0: sums start from +0, so -0 comes out +0 on
    # every path, the oracle's included)
    rng = np.random.default_rng(9)
    Bm = _finite_f16_no_negzero(rng, (512, 264))
    I = np.eye(512, dtype=np.float16)
    ref, _ = oracle.gemm_f16(I, Bm)
    assert bits_equal(ref, Bm)
    got = splitk(I, Bm, 4)
    assert bits_equal(got, ref), "split-K identity: first mismatches %s" % np.argwhere(
        got.view(np.uint16) != ref.view(np.uint16))[:8]
    # ones: every partial is an integer below 2^24 -> C = K exactly
    M, N, K = 2048, 2048, 32768
    ones = torch.ones((M, K), dtype=torch.float16, device="cuda:0")
    onesb = torch.ones((K, N), dtype=torch.float16, device="cuda:0")
    got = host(pg.pgemm_f16_splitk(ones, onesb, 4))
    assert np.all(got == np.float16(K))


def test_gemm_splitk_full_size_sampled():
    M, N, K = 2048, 2048, 32768
    say("gemm split-K full size %dx%dx%d" % (M, N, K))
    A, B = inputs.gemm_inputs(M, N, K)
    got = splitk(A, B, 4)
    I, J = inputs.sample_points(M, N, 8192)
    ref, _ = oracle.gemm_f16_points(A, B, I, J)
    assert_close(got[I, J], ref, "split-K long K")
    _, Sabs = oracle.gemm_f16_points(np.abs(A), np.abs(B), I, J)
    assert_fp32_bound(got[I, J], ref, Sabs, K, "split-K long K")


def test_gemm_splitk_on_a_side_stream_keeps_its_workspace():
    # The binding allocates the split-K workspace and C for a call with
    # stream=side. That memory must not be free for the current stream while
    # the side stream still runs the call: blocks of the workspace's size,
    # taken and filled with NaN on the current stream over the whole call,
    # must never be the workspace (or C).
    M, N, K = 2048, 2048, 32768
    say("gemm split-K on a side stream %dx%dx%d" % (M, N, K))
    A, B = inputs.gemm_inputs(M, N, K, seed_a=61, seed_b=62)
    tA, tB = dev(A), dev(B)
    ref = host(pg.pgemm_f16_splitk(tA, tB, 4))
    need = pg.pgemm_f16_splitk_workspace_bytes(M, N, K, 4)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(pg.pgemm_f16_splitk(tA, tB, 4, stream=side))
        for _ in range(24):  # about 24 x 15 us, longer than the call
            junk = torch.empty(need // 4, dtype=torch.float32, device="cuda:0")
            junk.fill_(float("nan"))
            del junk
    torch.cuda.synchronize()
    for i, C in enumerate(outs):
        assert bits_equal(C.cpu().numpy(), ref), "side-stream call %d differs" % i


def test_gemm_splitk_device_argument_checks():
    L = pg.lib()
    buf = torch.zeros(1 << 20, dtype=torch.float16, device="cuda:0")
    p = buf.data_ptr()
    A, B, C, W = p, p + (1 << 18), p + (2 << 18), p + (3 << 18)
    M = N = 64
    K = 512
    need = L.pgemm_f16_splitk_workspace_bytes(M, N, K, 4)
    assert need == 4 * M * N * 4
    s = None
    assert L.pgemm_f16_splitk(A, B, C, M, N, K, 4, 0, need, s) == pg.PGEMM_EINVAL
    assert L.pgemm_f16_splitk(A, B, C, M, N, K, 4, W, need - 16, s) == pg.PGEMM_EINVAL
    assert L.pgemm_f16_splitk(A, B, C, M, N, K, 4, W + 8, need, s) == pg.PGEMM_EUNSUPPORTED
    assert L.pgemm_f16_splitk(A, B, C, M, N, K, 4, C, need, s) == pg.PGEMM_EINVAL  # overlaps C
    assert L.pgemm_f16_splitk(A, B, C, M, N, K, 0, W, need, s) == pg.PGEMM_EUNSUPPORTED
    torch.cuda.synchronize()


# ------------------------------------------------------------ reduction (guide 7.2)

def test_sum_axis0_pages_worked_example():
    say("sum over axis 0 of ones (8, 1024, 1024)")
    g = _golden.keyed("sum_ones_8x1024x1024.txt")
    shape = tuple(int(s) for s in g["shape"])
    x = torch.full(shape, float(g["operand"][0]), dtype=torch.float32, device="cuda:0")
    o = torch.full(shape[1:], float("nan"), dtype=torch.float32, device="cuda:0")
    got = host(pg.preduce_sum_f32(x, out=o))
    assert np.all(got == np.float32(g["expected"][0]))


@pytest.mark.parametrize("R,shape", [(8, (1024, 1024)), (1, (100,)), (3, (64, 33)), (9, (4096,)),
                                     (17, (255, 4)), (1000, (64,)), (2, (1,)), (13, (7, 3)),
                                     # 3 full blocks of 1024 float4 + a block with 300
                                     (5, (3 * 4096 + 1200,)),
                                     # the shape bench.py times
                                     (8, (4096, 4096))])
def test_sum_axis0_bit_exact_vs_oracle(R, shape):
    say("sum axis 0 R=%d shape=%s" % (R, shape))
    x = inputs.uniform_f32((R,) + shape, 60 + R)
    got = host(pg.preduce_sum_f32(dev(x)))
    assert bits_equal(got, oracle.sum_axis0_f32(x))


def test_sum_axis0_order_and_empty():
    e = 2.0 ** -24
    x = np.array([[1.0] * 8, [e] * 8, [e] * 8, [e] * 8, [e] * 8], np.float32)
    got = host(pg.preduce_sum_f32(dev(x)))
    assert np.all(got == np.float32(1.0))  # ascending order from +0: stays 1.0
    o = torch.full((8,), float("nan"), dtype=torch.float32, device="cuda:0")
    z = host(pg.preduce_sum_f32(torch.empty((0, 8), dtype=torch.float32, device="cuda:0"), out=o))
    assert np.array_equal(z.view(np.uint32), np.zeros(8, np.uint32))


@pytest.mark.parametrize("n", [1024, 1022])  # float4 path, scalar path
def test_sum_axis0_special_values(n):
    # ordered triples of the special values down the reduction axis:
    # signed zeros, subnormals, infinities (inf + -inf = NaN), NaN, overflow
    say("sum axis 0 special values, n=%d" % n)
    sp = SPECIAL.astype(np.float32)
    trip = np.array(np.meshgrid(sp, sp, sp, indexing="ij")).reshape(3, -1)  # 3 x 3375
    x = np.ascontiguousarray(trip[:, np.random.default_rng(5).permutation(trip.shape[1])[:n]])
    got = host(pg.preduce_sum_f32(dev(x)))
    ref = oracle.sum_axis0_f32(x)
    nan = np.isnan(ref)
    assert nan.any() and np.array_equal(np.isnan(got), nan)
    assert bits_equal(got[~nan], ref[~nan])


def test_sum_axis0_misaligned_view_scalar_path():
    say("sum axis 0 misaligned")
    R, n = 5, 1001
    flat = inputs.uniform_f32(R * n + 1, 77)
    tx = dev(flat)[1:].view(R, n)
    got = host(pg.preduce_sum_f32(tx))
    assert bits_equal(got, oracle.sum_axis0_f32(flat[1:].reshape(R, n)))


# ------------------------------------------------------------ autotuner on the device

def test_autotune_measures_every_variant():
    from software_pipelined_tiled_pgemm_amd import autotune
    say("autotune: 256^3, variants 1 and 2, one round")
    recs = autotune.measure([(256, 256, 256)], variants=[1, 2], rounds=1, target_s=0.002)
    assert len(recs) == 1 and set(recs[0]["tflops"]) == {1, 2}
    assert all(x > 0 for x in recs[0]["tflops"].values())
    table = autotune.parse_table(autotune.render_table(recs, "test"))
    assert table == [(256, 256, 256, autotune.fastest(recs[0]))]


# ------------------------------------------------------------ HIP graph capture

def test_graph_capture_and_replay():
    # Every call only enqueues kernels on the caller's stream (no allocation,
    # no synchronisation, no memset), so a captured sequence replays.  Each
    # replay follows eager work that poisons the outputs and is checked
    # against the eager results.
    say("graph capture: gemm (auto, row split; persistent; 9-slot ring), split-K, stream add, "
        "x + c, reduction")
    A, B = inputs.gemm_inputs(4392, 4352, 4096)
    tA, tB = dev(A), dev(B)
    A2, B2 = inputs.gemm_inputs(256, 264, 8192, seed_a=60, seed_b=61)
    tA2, tB2 = dev(A2), dev(B2)
    x, y = inputs.stream_inputs(1 << 22, 62, 63)
    tx, ty = dev(x), dev(y)
    r = dev(inputs.uniform_f32((6, 1 << 18), 64))
    C = torch.empty((4392, 4352), dtype=torch.float16, device="cuda:0")
    C2 = torch.empty((256, 264), dtype=torch.float16, device="cuda:0")
    C9 = torch.empty((4392, 4352), dtype=torch.float16, device="cuda:0")
    C11 = torch.empty((256, 264), dtype=torch.float16, device="cuda:0")
    W = torch.empty(pg.pgemm_f16_splitk_workspace_bytes(256, 264, 8192, 4) // 4, device="cuda:0")
    z = torch.empty_like(tx)
    z1 = torch.empty_like(tx)
    o = torch.empty(1 << 18, device="cuda:0")

    def work():
        pg.pgemm_f16(tA, tB, C=C)
        pg.pgemm_f16_variant(tA, tB, 9, C=C9)
        pg.pgemm_f16_variant(tA2, tB2, 11, C=C11)
        pg.pgemm_f16_splitk(tA2, tB2, 4, C=C2, workspace=W)
        pg.pstream_add(tx, ty, z=z)
        pg.pstream_add_scalar(tx, 1.0, z=z1)
        pg.preduce_sum_f32(r, out=o)

    outs = (C, C2, z, z1, o, C9, C11)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # eager run on a side stream (also the warm-up before capture)
    torch.cuda.current_stream().wait_stream(s)
    eager = [host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for t, e in zip(outs, eager):
            assert bits_equal(host(t), e), "replay %d" % rep
    assert bits_equal(eager[2], oracle.add_f32(x, y))
    # the persistent variant gives the automatic path's bits (same family)
    assert bits_equal(eager[5], eager[0])
