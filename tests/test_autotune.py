"""Host-side checks of the autotuner's table and the library's automatic
variant choice (no GPU needed: pgemm_f16_choose_variant is a host function)."""
import itertools
import os
import random

import pytest

import software_pipelined_tiled_pgemm_amd as pg
from software_pipelined_tiled_pgemm_amd import _lib, autotune


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from software_pipelined_tiled_pgemm_amd import build
        build.build()
    return pg.lib()


def committed_table():
    with open(autotune.TABLE_PATH) as f:
        return autotune.parse_table(f.read())


def committed_rates():
    with open(autotune.TABLE_PATH) as f:
        return autotune.parse_rates(f.read())


def test_committed_table_is_well_formed(L):
    table = committed_table()
    assert table, "empty tuned table"
    nv = L.pgemm_f16_num_variants()
    for (M, N, K, v) in table:
        assert M > 0 and N > 0 and K > 0 and 1 <= v <= nv
    assert len({t[:3] for t in table}) == len(table), "duplicate shapes"
    for (M, N, K, v, rates) in committed_rates():
        assert sorted(rates) == list(range(1, nv + 1)), (M, N, K)
        assert all(x > 0 for x in rates.values()), (M, N, K)
        assert autotune.fastest({"tflops": rates}) == v, (M, N, K)


def test_tuned_shapes_get_their_variant(L):
    for (M, N, K, v) in committed_table():
        assert pg.pgemm_f16_choose_variant(M, N, K) == v, (M, N, K)


def test_library_applies_the_choice_rule(L):
    # no device here: the library assumes 256 CUs, as does choose()
    rates = committed_rates()
    nv = L.pgemm_f16_num_variants()
    rng = random.Random(7)
    shapes = [(rng.choice([8, 64, 200, 256, 1000, 2048, 3000, 4096, 9000, 20000]),
               rng.choice([8, 128, 256, 1024, 4096, 8192, 16384]),
               rng.choice([8, 32, 512, 4096, 32768, 100000])) for _ in range(300)]
    shapes += [(0, 8, 8), (8, 0, 8), (8, 8, 0), (1, 1, 1)]
    for (M, N, K) in shapes:
        got = pg.pgemm_f16_choose_variant(M, N, K)
        assert 1 <= got <= nv
        assert got == autotune.choose(rates, M, N, K, 256, nv), (M, N, K)


def test_choose_variant_rejects_negative_sizes(L):
    for args in [(-1, 8, 8), (8, -1, 8), (8, 8, -1)]:
        assert L.pgemm_f16_choose_variant(*args) == pg.PGEMM_EINVAL
    with pytest.raises(pg.PgemmError):
        pg.pgemm_f16_choose_variant(-1, 8, 8)


def test_render_parse_round_trip():
    recs = [{"M": 256, "N": 512, "K": 1024, "tflops": {1: 10.0, 2: 30.0, 5: 20.0}},
            {"M": 4096, "N": 4096, "K": 4096, "tflops": {1: 1200.0, 2: 1000.0, 5: 1250.54}}]
    text = autotune.render_table(recs, "test device")
    assert autotune.parse_table(text) == [(256, 512, 1024, 2), (4096, 4096, 4096, 5)]
    assert autotune.parse_rates(text)[1][4] == {1: 1200.0, 2: 1000.0, 3: 0.0, 4: 0.0, 5: 1250.5}
    assert "test device" in text
    # the stored fastest variant comes from the rounded rates
    text = autotune.render_table([{"M": 8, "N": 8, "K": 8, "tflops": {1: 100.0, 2: 101.0104}}])
    assert autotune.parse_table(text) == [(8, 8, 8, 1)]


def test_fastest_prefers_lowest_id_on_ties():
    assert autotune.fastest({"tflops": {3: 5.0, 1: 5.0, 2: 4.0}}) == 1


def test_choice_rule_examples():
    def e(M, N, K, rates):
        return (M, N, K, autotune.fastest({"tflops": rates}), rates)
    table = [e(256, 256, 256, {2: 7.0, 5: 3.0}), e(4096, 4096, 4096, {2: 1000.0, 5: 1250.0}),
             e(2048, 2048, 32768, {2: 1000.0, 5: 600.0})]
    assert autotune.choose(table, 4096, 4096, 4096) == 5
    assert autotune.choose(table, 300, 300, 300) == 2
    assert autotune.choose(table, 2048, 2048, 65536) == 2
    assert autotune.choose(table, 8192, 8192, 8192) == 5
    assert autotune.choose([], 1, 1, 1) == 2
    # 1024 x 8200 next to a tuned 1024 x 8192: the 128x128 tiles (two per
    # CU) go from exactly 512 to 520, a second wave for 8 of them (fill 1.0
    # -> 0.50), while the 132 256x256 tiles still take one (0.50 -> 0.50):
    # variant 8's estimate is 1.84 times variant 7's
    t = [e(1024, 8192, 4096, {7: 1076.6, 8: 989.0})]
    assert autotune.choose(t, 1024, 8192, 4096) == 7
    assert autotune.choose(t, 1024, 8200, 4096) == 8
    assert autotune.slot_fill(1024, 8200, 128, 512) == 1024 * 8200 / (2 * 512 * 16384)
    assert autotune.slot_fill(1024, 8200, 256, 256) == 1024 * 8200 / (256 * 65536)
    # 2184 x 4096 next to a tuned 2048 x 2048: variant 8's estimate leads by
    # 4.5% only (fill 0.25 -> 0.53 against 0.50 -> 0.53), below the 30% the
    # rule asks before it leaves the tuned shape's choice
    t = [e(2048, 2048, 8192, {7: 1053.0, 8: 550.0})]
    assert autotune.choose(t, 2184, 4096, 8192) == 7
    # fewer CUs: the same tiles take more waves
    assert autotune.slot_fill(2048, 2048, 128, 64) == 1.0


# ------------------------------------------------------------ row split of pgemm_f16

SMALL_PARTNER = {1: 2, 5: 2, 8: 7, 9: 7}  # 256x256 variant -> 128x128 variant of its family


def _waves(tiles, cus):
    return -(-tiles // cus)


def test_plan_examples(L):
    # the head variant is the tuned table's 256x256 choice on the
    # 16x16x32 instruction (one-tile 8 or persistent 9); its partner is 7
    assert pg.pgemm_f16_plan(4096, 4096, 4096, 256) == (4096, 8, 0)  # exactly one wave
    head, hv, tv = pg.pgemm_f16_plan(8192, 8192, 8192, 256)  # exactly four waves
    assert head == 8192 and hv in (8, 9) and tv == 0
    # 6144^3: 576 tiles of 256x256 = 2.25 waves; 21 tile rows (504 tiles, 2
    # waves) plus 768 rows as 288 tiles of 128x128 (2 waves at 0.35)
    head, hv, tv = pg.pgemm_f16_plan(6144, 6144, 6144, 256)
    assert head == 5376 and hv in (8, 9) and tv == 7
    assert pg.pgemm_f16_plan(1024, 1024, 1024, 256)[2] == 0  # too small to split


def test_plan_properties_on_random_shapes(L):
    rates = committed_rates()
    nv = L.pgemm_f16_num_variants()
    rng = random.Random(7)
    for _ in range(400):
        M, N, K = (rng.choice([8, 128, 256]) * rng.randint(1, 64) for _ in range(3))
        cus = rng.choice([0, 64, 256, 304])
        head, hv, tv = pg.pgemm_f16_plan(M, N, K, cus)
        assert hv == autotune.choose(rates, M, N, K, cus or 256, nv), (M, N, K, cus)
        if tv == 0:
            assert head == M
            continue
        c = cus or 256
        assert tv == SMALL_PARTNER[hv] and 0 < head < M and head % 256 == 0
        assert M * N * K >= 1e10
        # the split beats one launch by the margin in the library's model
        whole = _waves(-(-M // 256) * -(-N // 256), c)
        split = _waves((head // 256) * -(-N // 256), c) + 0.35 * _waves(-(-(M - head) // 128) * -(-N // 128), c)
        assert split < 0.95 * whole, (M, N, K, cus, head)


def test_plan_argument_errors(L):
    import ctypes
    h, a, b = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int()
    assert L.pgemm_f16_plan(-1, 8, 8, 256, ctypes.byref(h), ctypes.byref(a), ctypes.byref(b)) == pg.PGEMM_EINVAL
    assert L.pgemm_f16_plan(8, 8, 8, 256, None, ctypes.byref(a), ctypes.byref(b)) == pg.PGEMM_EINVAL


def test_fastest_takes_the_lowest_id_among_ties():
    rec = {"tflops": {1: 90.0, 8: 1438.5, 9: 1441.3}}
    assert autotune.fastest(rec) == 8      # 0.2% apart: tied
    rec = {"tflops": {7: 952.6, 8: 1069.3, 9: 1089.9}}
    assert autotune.fastest(rec) == 9      # 1.9% faster
    rec = {"tflops": {2: 5.0, 3: 5.0}}
    assert autotune.fastest(rec) == 2
