"""The layout kernel computes a token's rank set with rank(e) = e / m taken as
trunc(fmaf(e, fl(1/m), fl(1/m)/2)) instead of an integer division. Check that
identity for every expert id e < E and every experts-per-rank count m the
library accepts (E <= 1024, so m <= 1024 and e <= 1023): 1024 * 1024 pairs.

The fused multiply-add is evaluated exactly: e * c + c/2 with c = fl(1/m) is
a sum of two products of small integers and floats, exact in float64 (c has a
24-bit significand, e < 2^10), then rounded once to float32 as the hardware
instruction rounds it; the C library's correctly rounded fmaf checks a sample
of the same values."""
import ctypes
import ctypes.util

import numpy as np

libm = ctypes.CDLL(ctypes.util.find_library("m"))
libm.fmaf.restype = ctypes.c_float
libm.fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]


def fused_rank(e: np.ndarray, m: np.ndarray) -> np.ndarray:
    c = (1.0 / m.astype(np.float64)).astype(np.float32)         # fl(1/m)
    half = (np.float32(0.5) * c).astype(np.float32)              # exact (a power of two)
    exact = e.astype(np.float64) * c.astype(np.float64) + half.astype(np.float64)
    return np.trunc(exact.astype(np.float32)).astype(np.int64)  # one rounding, then trunc


def test_float_rank_division_is_exact_for_every_pair():
    m = np.arange(1, 1025, dtype=np.int64)[:, None]
    e = np.arange(0, 1024, dtype=np.int64)[None, :]
    got = fused_rank(np.broadcast_to(e, (1024, 1024)), np.broadcast_to(m, (1024, 1024)))
    want = e // m
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(int(m[i, 0]), int(e[0, j])) for i, j in bad[:5]]


def test_exact_evaluation_matches_the_c_fmaf():
    rng = np.random.default_rng(0)
    ms = rng.integers(1, 1025, 4000)
    es = rng.integers(0, 1024, 4000)
    model = fused_rank(es, ms)
    for e, m, r in zip(es, ms, model):
        inv = float(np.float32(1.0 / m))
        half = float(np.float32(0.5) * np.float32(inv))
        assert int(libm.fmaf(float(e), inv, half)) == r, (e, m)
