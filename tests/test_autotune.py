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


def test_committed_table_is_well_formed(L):
    table = committed_table()
    assert table, "empty tuned table"
    nv = L.pgemm_f16_num_variants()
    for (M, N, K, v) in table:
        assert M > 0 and N > 0 and K > 0 and 1 <= v <= nv
    assert len({t[:3] for t in table}) == len(table), "duplicate shapes"


def test_tuned_shapes_get_their_variant(L):
    for (M, N, K, v) in committed_table():
        assert pg.pgemm_f16_choose_variant(M, N, K) == v, (M, N, K)


def test_library_applies_the_nearest_rule(L):
    table = committed_table()
    rng = random.Random(7)
    shapes = [(rng.choice([8, 64, 200, 256, 1000, 2048, 3000, 4096, 9000, 20000]),
               rng.choice([8, 128, 256, 1024, 4096, 8192, 16384]),
               rng.choice([8, 32, 512, 4096, 32768, 100000])) for _ in range(300)]
    shapes += [(0, 8, 8), (8, 0, 8), (8, 8, 0), (1, 1, 1)]
    for (M, N, K) in shapes:
        got = pg.pgemm_f16_choose_variant(M, N, K)
        assert 1 <= got <= L.pgemm_f16_num_variants()
        # ties can resolve differently only if two tuned shapes are at the
        # same distance; the table has none at these points
        assert got == autotune.nearest(table, M, N, K), (M, N, K)


def test_choose_variant_rejects_negative_sizes(L):
    for args in [(-1, 8, 8), (8, -1, 8), (8, 8, -1)]:
        assert L.pgemm_f16_choose_variant(*args) == pg.PGEMM_EINVAL
    with pytest.raises(pg.PgemmError):
        pg.pgemm_f16_choose_variant(-1, 8, 8)


def test_render_parse_round_trip():
    recs = [{"M": 256, "N": 512, "K": 1024, "tflops": {1: 10.0, 2: 30.0, 5: 20.0}},
            {"M": 4096, "N": 4096, "K": 4096, "tflops": {1: 1200.0, 2: 1000.0, 5: 1250.5}}]
    text = autotune.render_table(recs, "test device")
    assert autotune.parse_table(text) == [(256, 512, 1024, 2), (4096, 4096, 4096, 5)]
    assert "test device" in text


def test_fastest_prefers_lowest_id_on_ties():
    assert autotune.fastest({"tflops": {3: 5.0, 1: 5.0, 2: 4.0}}) == 1


def test_nearest_rule_examples():
    table = [(256, 256, 256, 2), (4096, 4096, 4096, 5), (2048, 2048, 32768, 2)]
    assert autotune.nearest(table, 4096, 4096, 4096) == 5
    assert autotune.nearest(table, 300, 300, 300) == 2
    assert autotune.nearest(table, 2048, 2048, 65536) == 2
    assert autotune.nearest(table, 8192, 8192, 8192) == 5
    assert autotune.nearest([], 1, 1, 1) == 2


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
    rng = random.Random(7)
    for _ in range(400):
        M, N, K = (rng.choice([8, 128, 256]) * rng.randint(1, 64) for _ in range(3))
        cus = rng.choice([0, 64, 256, 304])
        head, hv, tv = pg.pgemm_f16_plan(M, N, K, cus)
        assert hv == pg.pgemm_f16_choose_variant(M, N, K)
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
