"""Host checks of the shared input generators (no GPU)."""
import numpy as np
import torch

from software_pipelined_tiled_pgemm_amd import inputs


def test_hashed_numpy_and_torch_agree():
    a = inputs.hashed_f16(np.arange(300), np.arange(520), 0)
    b = inputs.hashed_f16_torch(300, 520, 0, "cpu", row_chunk=128).numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_hashed_subsets_and_seeds():
    full = inputs.hashed_f16(np.arange(64), np.arange(96), 1)
    r, c = np.array([63, 0, 17, 17]), np.array([95, 3, 0])
    assert np.array_equal(inputs.hashed_f16(r, c, 1), full[np.ix_(r, c)])
    assert not np.array_equal(full, inputs.hashed_f16(np.arange(64), np.arange(96), 0))


def test_hashed_values_exact_and_spread():
    a = inputs.hashed_f16(np.arange(512), np.arange(512), 0).astype(np.float64)
    assert np.all(a * 1024 == np.round(a * 1024))  # multiples of 2**-10: exact in fp16
    assert a.min() >= -1019 / 1024 and a.max() <= 1019 / 1024
    assert np.unique(a).size == 2039
    assert abs(a.mean()) < 0.01 and abs(a.std() - 0.577) < 0.01


def test_hashed_large_indices_do_not_overflow():
    # row and column indices at the GEMM size limits
    r = np.array([2**31 - 257, 140000])
    c = np.array([2**23 - 8, 7])
    v = inputs.hashed_f16(r, c, 1)
    t = inputs.hashed_f16_torch(1, 8, 1, "cpu").numpy()
    assert np.all(np.abs(v.astype(np.float64)) <= 1019 / 1024)
    assert np.array_equal(inputs.hashed_f16(np.array([0]), np.arange(8), 1), t)
