"""The layout kernel computes a token's rank set with rank(e) = e / m taken as
trunc(fmaf(e, fl(1/m), fl(1/m)/2)) instead of an integer division. Check that
identity exhaustively for every expert id and every experts-per-rank count the
library accepts (E <= 1024), with the C library's correctly rounded fmaf."""
import ctypes
import ctypes.util

import numpy as np

libm = ctypes.CDLL(ctypes.util.find_library("m"))
libm.fmaf.restype = ctypes.c_float
libm.fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]


def test_float_rank_division_is_exact():
    bad = []
    for m in range(1, 1025):
        inv = float(np.float32(1.0 / m))
        half = float(np.float32(0.5) * np.float32(inv))
        for e in range(0, 1024, 1 if m < 64 or m % 7 == 0 else 3):
            r = int(libm.fmaf(float(e), inv, half))
            if r != e // m:
                bad.append((m, e, r))
    assert not bad, bad[:5]
