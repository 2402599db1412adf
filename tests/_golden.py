"""Readers for the fixtures under tests/golden (values the pages print)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def values_f32(name) -> np.ndarray:
    return np.array([float(v) for v in _lines(name)], dtype=np.float32)


def keyed(name) -> dict:
    out = {}
    for ln in _lines(name):
        k, *v = ln.split()
        out[k] = v
    return out
