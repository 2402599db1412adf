"""Pins for the CPU oracle: every check compares it with something other than
itself -- numpy's IEEE conversions and additions (library routines), exact
rational arithmetic on tiny inputs, closed forms, and the values the pages
print.  A last group plants typical mistakes in calls to the oracle and shows
that the pins catch them."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import _golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- binary16

ALL_H = np.arange(65536, dtype=np.uint16)
FINITE_H = ALL_H[(ALL_H & 0x7C00) != 0x7C00]


def test_f16_decode_exhaustive():
    got = oracle.f64_from_f16(ALL_H)
    ref = ALL_H.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))


def test_f16_encode_roundtrip_all_finite():
    vals = FINITE_H.view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.f16_from_f64(vals), FINITE_H)


def _positive_finite_sorted():
    v = FINITE_H.view(np.float16).astype(np.float64)
    v = np.unique(v[v >= 0])
    return v


def test_f16_encode_midpoints_and_neighbours():
    v = _positive_finite_sorted()
    # add the first value past the largest finite binary16 (2^16) so the
    # overflow midpoint 65520 is included
    v = np.append(v, 65536.0)
    mid = (v[:-1] + v[1:]) / 2  # exact in binary64
    xs = np.concatenate([mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])
    xs = np.concatenate([xs, -xs])
    got = oracle.f16_from_f64(xs)
    ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_encode_random_against_numpy():
    rng = np.random.default_rng(123)
    n = 1_000_000
    x = rng.uniform(1.0, 2.0, n) * np.exp2(rng.integers(-30, 18, n)) * rng.choice([-1.0, 1.0], n)
    got = oracle.f16_from_f64(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("x,expected", [
    (65504.0, 0x7BFF),             # largest finite
    (65519.99, 0x7BFF),            # just below the overflow midpoint
    (65520.0, 0x7C00),             # overflow midpoint ties to even -> inf
    (2.0 ** -25, 0x0000),          # half the smallest subnormal: tie to even 0
    (3 * 2.0 ** -26, 0x0001),      # 0.75 ulp -> smallest subnormal
    (2.0 ** -24, 0x0001),
    (2.0 ** -14 - 2.0 ** -25, 0x0400),  # rounds up into the normal range
    (1.0 + 2.0 ** -11, 0x3C00),    # tie between 1 and 1+2^-10 -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),  # tie -> even (1+2^-9)
    (-0.0, 0x8000),
    (float("inf"), 0x7C00),
    (float("-inf"), 0xFC00),
])
def test_f16_hand_cases(x, expected):
    assert int(oracle.f16_from_f64([x])[0]) == expected


def test_f16_nan():
    h = oracle.f16_from_f64([float("nan")])
    assert np.isnan(h.view(np.float16)[0])


# ---------------------------------------------------------------- GEMM pins

def _round_f16_exact(fr: Fraction) -> np.float16:
    """Nearest binary16 to an exact rational, ties to even, found by comparing
    exact distances to the neighbouring binary16 values (independent of any
    binary64 rounding)."""
    c = np.float16(float(fr))
    cands = {c, np.nextafter(c, np.float16(np.inf)), np.nextafter(c, np.float16(-np.inf))}
    cands = [h for h in cands if np.isfinite(h)]
    best = min(abs(Fraction(float(h)) - fr) for h in cands)
    ties = [h for h in cands if abs(Fraction(float(h)) - fr) == best]
    if len(ties) > 1:
        ties = [h for h in ties if (int(np.array(h).view(np.uint16)) & 1) == 0]
    return ties[0]


def _exact_product_f16(A, B):
    A64 = A.astype(np.float64)
    B64 = B.astype(np.float64)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float16)
    for i in range(M):
        for j in range(N):
            s = sum((Fraction(float(A64[i, k])) * Fraction(float(B64[k, j])) for k in range(K)),
                    Fraction(0))
            C[i, j] = _round_f16_exact(s)
    return C


def _tiny_exact_regime(rng, shape):
    """fp16 normals with |x| in [2^-8, 1] and random sign: for K <= 8 the
    binary64 sum of products is exact, so the oracle must equal the exact
    rational result rounded once."""
    mag = rng.uniform(2.0 ** -8, 1.0, shape)
    sign = rng.choice([-1.0, 1.0], shape)
    return (mag * sign).astype(np.float16)


TINY_SHAPES = [(1, 1, 1), (1, 5, 3), (4, 1, 7), (3, 7, 8), (8, 8, 8), (5, 2, 6), (7, 3, 1), (2, 8, 5)]


def _passes_bruteforce(gemm_fn, seed=7) -> bool:
    rng = np.random.default_rng(seed)
    for (M, N, K) in TINY_SHAPES:
        A = _tiny_exact_regime(rng, (M, K))
        B = _tiny_exact_regime(rng, (K, N))
        C = np.asarray(gemm_fn(A, B))
        if C.shape != (M, N):
            return False
        if not np.array_equal(C.view(np.uint16), _exact_product_f16(A, B).view(np.uint16)):
            return False
    return True


def _oracle_c(A, B):
    return oracle.gemm_f16(A, B)[0]


def test_gemm_bruteforce_exact_rational():
    assert _passes_bruteforce(_oracle_c)


def _all_finite_f16_no_negzero(rng, shape):
    h = rng.choice(FINITE_H, size=shape)
    h[h == 0x8000] = 0
    return h.view(np.float16)


def test_gemm_identity_left_and_right():
    rng = np.random.default_rng(11)
    for (M, N) in [(1, 1), (5, 9), (64, 33), (130, 70)]:
        B = _all_finite_f16_no_negzero(rng, (M, N))   # includes subnormals and 65504
        C, S = oracle.gemm_f16(np.eye(M, dtype=np.float16), B)
        assert np.array_equal(C.view(np.uint16), B.view(np.uint16))
        C2, _ = oracle.gemm_f16(B, np.eye(N, dtype=np.float16))
        assert np.array_equal(C2.view(np.uint16), B.view(np.uint16))


def test_gemm_permutation():
    rng = np.random.default_rng(12)
    M, N = 97, 45
    perm = rng.permutation(M)
    P = np.zeros((M, M), np.float16)
    P[np.arange(M), perm] = 1
    B = _all_finite_f16_no_negzero(rng, (M, N))
    C, _ = oracle.gemm_f16(P, B)
    assert np.array_equal(C.view(np.uint16), B[perm].view(np.uint16))


def test_gemm_rank1_integer_closed_form():
    rng = np.random.default_rng(13)
    for (M, N, K) in [(3, 4, 5), (31, 17, 64), (40, 24, 256)]:
        u = rng.integers(-4, 5, M).astype(np.float64)
        v = rng.integers(-4, 5, N).astype(np.float64)
        A = np.repeat(u[:, None], K, axis=1).astype(np.float16)
        B = np.repeat(v[None, :], K, axis=0).astype(np.float16)
        C, S = oracle.gemm_f16(A, B)
        expect = K * np.outer(u, v)
        assert np.array_equal(S, expect)
        assert np.array_equal(C.astype(np.float64), expect)


@pytest.mark.parametrize("K", [4096, 8192, 32768])
def test_gemm_rank1_powers_of_two_long_k(K):
    rng = np.random.default_rng(K)
    u = rng.choice([-1.0, -0.5, 0.5, 1.0], 6)
    v = rng.choice([-1.0, -0.5, 0.5, 1.0], 5)
    A = np.repeat(u[:, None], K, axis=1).astype(np.float16)
    B = np.repeat(v[None, :], K, axis=0).astype(np.float16)
    C, _ = oracle.gemm_f16(A, B)
    assert np.array_equal(C.astype(np.float64), K * np.outer(u, v))


@pytest.mark.parametrize("K", [256, 4096, 32768])
def test_gemm_ones(K):
    A = np.ones((3, K), np.float16)
    B = np.ones((K, 4), np.float16)
    C, _ = oracle.gemm_f16(A, B)
    assert np.all(C.astype(np.float64) == K)


def test_gemm_scaling_invariant():
    A, B = [np.random.default_rng(s).uniform(-1, 1, sh).astype(np.float16)
            for s, sh in ((20, (33, 70)), (21, (70, 29)))]
    C1, S1 = oracle.gemm_f16(A, B)
    C2, S2 = oracle.gemm_f16((A.astype(np.float64) * 2).astype(np.float16), B)
    assert np.array_equal(S2, 2 * S1)
    assert np.array_equal(C2.astype(np.float64), 2 * C1.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (129, 65, 200), (256, 256, 256), (300, 190, 520)])
def test_gemm_numpy_crosscheck(M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float16)
    C, S = oracle.gemm_f16(A, B)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    ref = A64 @ B64                                # BLAS, other summation order
    bound = K * 2.0 ** -52 * (np.abs(A64) @ np.abs(B64))
    assert np.all(np.abs(S - ref) <= bound)
    # rounding of nearly equal binary64 sums can differ by at most one ulp
    d = np.abs(C.view(np.uint16).astype(np.int32) - ref.astype(np.float16).view(np.uint16).astype(np.int32))
    assert d.max() <= 1
    assert np.mean(d == 0) > 0.999


def test_gemm_points_match_full():
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, (150, 96)).astype(np.float16)
    B = rng.uniform(-1, 1, (96, 170)).astype(np.float16)
    C, S = oracle.gemm_f16(A, B)
    from software_pipelined_tiled_pgemm_amd import inputs
    I, J = inputs.sample_points(150, 170, 500, full_rows=3, full_cols=3, tile=64)
    Cp, Sp = oracle.gemm_f16_points(A, B, I, J)
    assert np.array_equal(Cp.view(np.uint16), C[I, J].view(np.uint16))
    assert np.array_equal(Sp, S[I, J])


def test_gemm_empty_k_is_zero():
    C, S = oracle.gemm_f16(np.zeros((3, 0), np.float16), np.zeros((0, 5), np.float16))
    assert np.all(S == 0) and np.all(C.view(np.uint16) == 0)


# Planted mistakes: each would be a plausible bug inside the oracle; the
# brute-force pin must reject every one of them.
MUTANTS = {
    "dropped_last_k_term": lambda A, B: oracle.gemm_f16(A[:, :-1], B[:-1, :])[0] if A.shape[1] > 1
    else np.zeros((A.shape[0], B.shape[1]), np.float16),
    "transposed_B": lambda A, B: oracle.gemm_f16(A, np.ascontiguousarray(B.T))[0]
    if B.shape[0] == B.shape[1] else oracle.gemm_f16(A, B)[0].T,
    "wrong_sign": lambda A, B: -oracle.gemm_f16(A, B)[0],
    "k_index_shifted": lambda A, B: oracle.gemm_f16(A, np.roll(B, 1, axis=0))[0],
    "rounded_through_f32": lambda A, B: (A.astype(np.float32) @ B.astype(np.float32)).astype(np.float16)
    if A.shape[1] > 4 else oracle.gemm_f16(A, B)[0] + np.float16(2.0 ** -10),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bruteforce_pin_rejects_planted_mistake(name):
    assert not _passes_bruteforce(MUTANTS[name])


# ---------------------------------------------------------------- streaming

SPECIAL_F32 = np.array([0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1e-40, 1.1754942e-38,
                        3.4028235e38, -3.4028235e38, np.inf, -np.inf, np.nan, 0.5, 2.0 ** -24],
                       dtype=np.float32)


def _bits_equal_f32(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


def test_add_random_against_numpy():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-140, 120, 1_000_000))).astype(np.float32)
    y = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-140, 120, 1_000_000))).astype(np.float32)
    assert _bits_equal_f32(oracle.add_f32(x, y), np.add(x, y))


def test_add_special_values_all_pairs():
    x = np.repeat(SPECIAL_F32, SPECIAL_F32.size)
    y = np.tile(SPECIAL_F32, SPECIAL_F32.size)
    z = oracle.add_f32(x, y)
    assert _bits_equal_f32(z, np.add(x, y))
    # IEEE facts that do not depend on numpy
    neg0 = oracle.add_f32(np.array([-0.0], np.float32), np.array([-0.0], np.float32))
    pos0 = oracle.add_f32(np.array([0.0], np.float32), np.array([-0.0], np.float32))
    assert neg0.view(np.uint32)[0] == 0x80000000 and pos0.view(np.uint32)[0] == 0
    big = oracle.add_f32(np.array([3.4028235e38], np.float32), np.array([3.4028235e38], np.float32))
    assert np.isposinf(big[0])
    sub = oracle.add_f32(np.array([1e-45], np.float32), np.array([1e-45], np.float32))
    assert sub.view(np.uint32)[0] == 2  # subnormals are not flushed


def test_add_pages_worked_example_ones():
    g = _golden.keyed("ones_add_512.txt")
    shape = tuple(int(s) for s in g["shape"])
    x = np.full(shape, float(g["operand"][0]), np.float32)
    z = oracle.add_f32(x, x)
    assert np.all(z == np.float32(g["expected"][0]))


def test_add_scalar_plus_one():
    rng = np.random.default_rng(6)
    x = rng.uniform(-1, 1, 100_000).astype(np.float32)
    x = np.concatenate([x, SPECIAL_F32])
    assert _bits_equal_f32(oracle.add_scalar_f32(x, 1.0), x + np.float32(1.0))
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: even -> 1.0
    assert oracle.add_scalar_f32(np.array([2.0 ** -24], np.float32), 1.0)[0] == 1.0


def test_fill_pages_worked_example():
    assert _bits_equal_f32(oracle.fill_f32(128, 42.0), _golden.values_f32("fill_42.txt"))


def test_iota_pages_worked_example():
    assert _bits_equal_f32(oracle.iota_f32(1024), _golden.values_f32("iota_1024.txt"))


# ---------------------------------------------------------------- reduction (guide 7.2)

def test_sum_axis0_pages_worked_example():
    g = _golden.keyed("sum_ones_8x1024x1024.txt")
    shape = tuple(int(s) for s in g["shape"])
    x = np.full(shape, float(g["operand"][0]), np.float32)
    o = oracle.sum_axis0_f32(x)
    assert o.shape == shape[1:]
    assert np.all(o == np.float32(g["expected"][0]))


def test_sum_axis0_order_is_ascending_sequential():
    # 1 + 2^-24 rounds to 1 (tie to even), so adding two 2^-24 after the 1
    # leaves 1.0; adding them first gives 2^-23, and 1 + 2^-23 is exact.
    e = 2.0 ** -24
    x = np.array([[1.0], [e], [e]], np.float32)
    assert oracle.sum_axis0_f32(x)[0] == np.float32(1.0)
    y = np.array([[e], [e], [1.0]], np.float32)
    assert oracle.sum_axis0_f32(y)[0] == np.float32(1.0 + 2.0 ** -23)


def test_sum_axis0_exact_integer_sums_and_signed_zero():
    rng = np.random.default_rng(70)
    x = rng.integers(-1000, 1000, size=(37, 5, 7)).astype(np.float32)
    assert np.array_equal(oracle.sum_axis0_f32(x), x.astype(np.int64).sum(axis=0).astype(np.float32))
    z = oracle.sum_axis0_f32(np.array([[-0.0, 0.0]], np.float32))
    assert z.view(np.uint32)[0] == 0 and z.view(np.uint32)[1] == 0  # +0 start: -0 + ... -> +0
    empty = oracle.sum_axis0_f32(np.zeros((0, 3), np.float32))
    assert np.array_equal(empty.view(np.uint32), np.zeros(3, np.uint32))


def test_sum_axis0_error_bound_random():
    rng = np.random.default_rng(71)
    x = rng.uniform(-1, 1, size=(64, 1000)).astype(np.float32)
    o = oracle.sum_axis0_f32(x).astype(np.float64)
    exact = x.astype(np.float64).sum(axis=0)
    bound = 64 * 2.0 ** -24 * np.abs(x.astype(np.float64)).sum(axis=0)
    assert np.all(np.abs(o - exact) <= bound)


def _sum_reversed(x):
    s = np.zeros(x.shape[1:], np.float32)
    for i in range(x.shape[0] - 1, -1, -1):
        s = (s + x[i]).astype(np.float32)
    return s


def _sum_pairwise(x):
    parts = [x[i] for i in range(x.shape[0])]
    while len(parts) > 1:
        nxt = [(parts[k] + parts[k + 1]).astype(np.float32) for k in range(0, len(parts) - 1, 2)]
        if len(parts) % 2:
            nxt.append(parts[-1])
        parts = nxt
    return parts[0]


@pytest.mark.parametrize("mutant", [_sum_reversed, _sum_pairwise])
def test_sum_axis0_order_pin_rejects_other_orders(mutant):
    # Plausible wrong oracles: the reduction axis walked backwards, or a
    # pairwise tree.  On 1 followed by four 2^-24 the ascending sum is 1.0
    # and both of these differ.
    e = 2.0 ** -24
    x = np.array([[1.0], [e], [e], [e], [e]], np.float32)
    assert oracle.sum_axis0_f32(x)[0] == np.float32(1.0)
    assert mutant(x)[0] != np.float32(1.0)


# ------------------------------------------------------------ the fp32 accumulation bound

def _fp32_sums(A, B, order):
    """fp16 GEMM with fp32 accumulation in a given order, simulated on the host."""
    P = A.astype(np.float32)[:, :, None] * B.astype(np.float32)[None, :, :]  # exact products
    if order == "ascending":
        return np.cumsum(P, axis=1, dtype=np.float32)[:, -1, :]
    if order == "descending":
        return np.cumsum(P[:, ::-1, :], axis=1, dtype=np.float32)[:, -1, :]
    # blocks of 32 products summed pairwise, blocks added in ascending order
    K = P.shape[1]
    blocks = np.add.reduce(P.reshape(P.shape[0], K // 32, 32, P.shape[2]), axis=2, dtype=np.float32)
    return np.cumsum(blocks, axis=1, dtype=np.float32)[:, -1, :]


@pytest.mark.parametrize("K", [64, 1024, 4096])
def test_fp32_bound_holds_for_any_order_and_catches_mistakes(K):
    from software_pipelined_tiled_pgemm_amd import inputs
    from tests._bounds import fp32_bound_violations
    A, B = inputs.gemm_inputs(48, 40, K, seed_a=30, seed_b=31)
    ref, _ = oracle.gemm_f16(A, B)
    _, Sabs = oracle.gemm_f16(np.abs(A), np.abs(B))
    for order in ("ascending", "descending", "blocks"):
        got = _fp32_sums(A, B, order).astype(np.float16)
        assert not fp32_bound_violations(got, ref, Sabs, K).any(), order
    # plausible kernel mistakes must fall outside it for most outputs; the
    # bound grows like K * 2**-24 * K/4, so one dropped term (|ab| ~ 1/4)
    # stands out only up to K of about a thousand
    if K <= 1024:
        dropped = _fp32_sums(A[:, 1:], B[1:, :], "ascending")
        assert fp32_bound_violations(dropped.astype(np.float16), ref, Sabs, K).mean() > 0.5
    half_k = _fp32_sums(A[:, : K // 2], B[: K // 2, :], "ascending")
    assert fp32_bound_violations(half_k.astype(np.float16), ref, Sabs, K).mean() > 0.9
    transposed_b = _fp32_sums(A[:, :40], B[:40, :].T.copy(), "ascending") if K == 64 else None
    if transposed_b is not None:
        ref40, _ = oracle.gemm_f16(A[:, :40], B[:40, :])
        _, Sabs40 = oracle.gemm_f16(np.abs(A[:, :40]), np.abs(B[:40, :]))
        assert fp32_bound_violations(transposed_b.astype(np.float16), ref40, Sabs40, 40).mean() > 0.9
