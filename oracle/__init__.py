"""ctypes wrapper over the C oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the plain, slow, single-threaded CPU definition of
MoE dispatch (layout, pack, permute) and combine that the GPU library is
checked against. Only the tests, the smoke check and the benchmark's CPU
baseline may import this package. It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

ERR_BAD_ID = 1
ERR_RANK_CAP = 2
ERR_EXPERT_CAP = 4

class _Lib:
    """Typed handle on one build of the oracle library (the default build, or a
    test's deliberately altered copy)."""

    def __init__(self, path: str):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_layout.restype = ctypes.c_int
        lib.oracle_layout.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_pack.argtypes = [i32, i32, i32, vp, vp, vp, vp, i64]
        lib.oracle_permute.restype = ctypes.c_int
        lib.oracle_permute.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                       i64, vp, vp, i64]
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_combine.argtypes = [i32, i32, i32, vp, vp, vp, i64, vp, vp]
        lib.oracle_combine_f64.restype = ctypes.c_int
        lib.oracle_combine_f64.argtypes = [i32, i32, i32, vp, vp, vp, i64, vp]
        lib.oracle_combine_rank_partial.restype = ctypes.c_int
        lib.oracle_combine_rank_partial.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, vp, vp,
                                                    vp, vp, i64, vp, vp]
        lib.oracle_combine_ranks.restype = ctypes.c_int
        lib.oracle_combine_ranks.argtypes = [i32, i32, i32, vp, i64, vp, vp, vp]
        lib.oracle_quantize_mxfp8.restype = None
        lib.oracle_quantize_mxfp8.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_quantize_mxfp4.restype = None
        lib.oracle_quantize_mxfp4.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_quantize_nvfp4.restype = None
        lib.oracle_quantize_nvfp4.argtypes = [i64, i32, vp, vp, vp]
        self.lib = lib


_default = None
_override = None


def _load():
    global _default
    if _override is not None:
        return _override.lib
    if _default is None:
        _default = _Lib(LIB_PATH)
    return _default.lib


class use_library:
    """Context manager: route this module's functions to another build of the
    oracle (used by the test that checks the pins catch planted mistakes)."""

    def __init__(self, path: str):
        self.handle = _Lib(path)

    def __enter__(self):
        global _override
        self.prev = _override
        _override = self.handle
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def layout(topk_ids: np.ndarray, E: int, R: int, align: int = 1, block: int = 0) -> dict:
    """Counts, offsets and rows of the layout. align > 1 pads every expert's
    run to a multiple of align rows; block > 0 gives every expert a fixed
    block of rows instead (masked). The result records align and block."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    assert E % R == 0 and align >= 1 and block >= 0 and (block == 0 or align == 1)
    res = dict(
        rank_counts=np.zeros(R, np.int32),
        rank_offsets=np.zeros(R + 1, np.int32),
        expert_counts=np.zeros(E, np.int32),
        expert_offsets=np.zeros(E + 1, np.int32),
        token_rank_slot=np.zeros((T, R), np.int32),
        pair_row=np.zeros((T, k), np.int32),
    )
    res["err"] = _load().oracle_layout(
        T, E, R, k, align, block, _p(ids), _p(res["rank_counts"]), _p(res["rank_offsets"]),
        _p(res["expert_counts"]), _p(res["expert_offsets"]), _p(res["token_rank_slot"]),
        _p(res["pair_row"]))
    res["align"], res["block"] = align, block
    return res


def pack(hidden: np.ndarray, token_rank_slot: np.ndarray, cap_rank: int,
         rank_buf: np.ndarray | None = None, rank_src_token: np.ndarray | None = None):
    hid = _c(hidden, np.uint16)
    slots = _c(token_rank_slot, np.int32)
    T, H = hid.shape
    R = slots.shape[1]
    if rank_buf is None:
        rank_buf = np.zeros((cap_rank, H), np.uint16)
    if rank_src_token is None:
        rank_src_token = np.full(cap_rank, -1, np.int32)
    err = _load().oracle_pack(T, H, R, _p(hid), _p(slots), _p(rank_buf), _p(rank_src_token),
                              cap_rank)
    return rank_buf, rank_src_token, err


def permute(rank_buf, rank_src_token, lay: dict, topk_ids, E: int, cap_expert: int,
            expert_buf=None, expert_src_pair=None):
    """Regroup the rank-buffer rows by expert, at the rows the layout `lay`
    (from layout()) assigned, and mark its padding rows -1."""
    rb = _c(rank_buf, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    R = len(lay["rank_offsets"]) - 1
    H = rb.shape[1]
    if expert_buf is None:
        expert_buf = np.zeros((cap_expert, H), np.uint16)
    if expert_src_pair is None:
        expert_src_pair = np.full(cap_expert, -2, np.int32)
    err = _load().oracle_permute(
        T, H, E, R, k, lay.get("block", 0), _p(rb), _p(_c(rank_src_token, np.int32)),
        _p(_c(lay["rank_offsets"], np.int32)), _p(ids), _p(_c(lay["pair_row"], np.int32)),
        _p(_c(lay["expert_counts"], np.int32)), _p(_c(lay["expert_offsets"], np.int32)),
        rb.shape[0], _p(expert_buf), _p(expert_src_pair), cap_expert)
    return expert_buf, expert_src_pair, err


def combine(expert_out, pair_row, topk_weights, want_f32: bool = True):
    eo = _c(expert_out, np.uint16)
    pr = _c(pair_row, np.int32)
    w = _c(topk_weights, np.float32)
    T, k = pr.shape
    H = eo.shape[1]
    out = np.zeros((T, H), np.uint16)
    out32 = np.zeros((T, H), np.float32) if want_f32 else None
    err = _load().oracle_combine(T, H, k, _p(eo), _p(pr), _p(w), eo.shape[0], _p(out), _p(out32))
    return out, out32, err


def combine_f64(expert_out, pair_row, topk_weights):
    eo = _c(expert_out, np.uint16)
    pr = _c(pair_row, np.int32)
    w = _c(topk_weights, np.float32)
    T, k = pr.shape
    H = eo.shape[1]
    out = np.zeros((T, H), np.float64)
    err = _load().oracle_combine_f64(T, H, k, _p(eo), _p(pr), _p(w), eo.shape[0], _p(out))
    return out, err


def combine_rank_partial(expert_out, rank_src_token, rank_offsets, topk_ids, pair_row,
                         topk_weights, E: int, cap_rank: int, want_f32: bool = True):
    """First stage of the two-stage combine: one partial row per rank-buffer
    row (bf16, and the float32 accumulator if want_f32). Rows past the last
    segment stay zero."""
    eo = _c(expert_out, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    R = len(rank_offsets) - 1
    H = eo.shape[1]
    part = np.zeros((cap_rank, H), np.uint16)
    part32 = np.zeros((cap_rank, H), np.float32) if want_f32 else None
    err = _load().oracle_combine_rank_partial(
        T, H, E, R, k, _p(eo), eo.shape[0], _p(_c(rank_src_token, np.int32)),
        _p(_c(rank_offsets, np.int32)), _p(ids), _p(_c(pair_row, np.int32)),
        _p(_c(topk_weights, np.float32)), cap_rank, _p(part), _p(part32))
    return part, part32, err


def combine_ranks(partial, token_rank_slot, want_f32: bool = True):
    """Second stage of the two-stage combine: per token, the sum over ranks of
    its partial rows, in float32, rounded to bf16."""
    part = _c(partial, np.uint16)
    slots = _c(token_rank_slot, np.int32)
    T, R = slots.shape
    H = part.shape[1]
    out = np.zeros((T, H), np.uint16)
    out32 = np.zeros((T, H), np.float32) if want_f32 else None
    err = _load().oracle_combine_ranks(T, H, R, _p(part), part.shape[0], _p(slots), _p(out),
                                       _p(out32))
    return out, out32, err


def quantize_mxfp8(x):
    """bf16 rows [rows, H] (H a multiple of 32) -> (q [rows, H] uint8 e4m3 codes,
    scale [rows, H/32] uint8 E8M0 exponents)."""
    xb = _c(x, np.uint16)
    rows, H = xb.shape
    assert H % 32 == 0
    q = np.zeros((rows, H), np.uint8)
    sc = np.zeros((rows, H // 32), np.uint8)
    _load().oracle_quantize_mxfp8(rows, H, _p(xb), _p(q), _p(sc))
    return q, sc


def pack_mxfp8(hidden, token_rank_slot, cap_rank: int):
    """Quantise every hidden row once, then pack the codes and the scales once
    per distinct rank (the rows are plain byte copies, as in pack())."""
    q, sc = quantize_mxfp8(hidden)
    T, H = q.shape
    rq, src, err = pack(q.view(np.uint16), token_rank_slot, cap_rank)
    rs, _, _ = pack(sc.view(np.uint16), token_rank_slot, cap_rank)
    return rq.view(np.uint8), rs.view(np.uint8), src, err


def permute_mxfp8(rank_q, rank_scale, rank_src_token, lay: dict, topk_ids, E: int,
                  cap_expert: int):
    """Regroup quantised rows by expert: the codes and the scales each move as
    permute() moves bf16 rows."""
    eq, esrc, err = permute(np.ascontiguousarray(rank_q).view(np.uint16), rank_src_token, lay,
                            topk_ids, E, cap_expert)
    es, _, _ = permute(np.ascontiguousarray(rank_scale).view(np.uint16), rank_src_token, lay,
                       topk_ids, E, cap_expert)
    return eq.view(np.uint8), es.view(np.uint8), esrc, err


def quantize_mxfp4(x):
    """bf16 rows [rows, H] (H a multiple of 32) -> (q [rows, H/2] uint8, two e2m1
    codes per byte, even value in the low nibble; scale [rows, H/32] uint8)."""
    xb = _c(x, np.uint16)
    rows, H = xb.shape
    assert H % 32 == 0
    q = np.zeros((rows, H // 2), np.uint8)
    sc = np.zeros((rows, H // 32), np.uint8)
    _load().oracle_quantize_mxfp4(rows, H, _p(xb), _p(q), _p(sc))
    return q, sc


def pack_mxfp4(hidden, token_rank_slot, cap_rank: int):
    """Quantise every hidden row once to MXFP4, then pack codes and scales once
    per distinct rank (plain byte copies, as in pack())."""
    q, sc = quantize_mxfp4(hidden)
    rq, src, err = pack(q.view(np.uint16), token_rank_slot, cap_rank)
    rs, _, _ = pack(sc.view(np.uint16), token_rank_slot, cap_rank)
    return rq.view(np.uint8), rs.view(np.uint8), src, err


def permute_mxfp4(rank_q, rank_scale, rank_src_token, lay: dict, topk_ids, E: int,
                  cap_expert: int):
    """Regroup MXFP4 rows by expert: codes and scales move as bytes, exactly as
    permute_mxfp8 moves them."""
    return permute_mxfp8(rank_q, rank_scale, rank_src_token, lay, topk_ids, E, cap_expert)


def quantize_nvfp4(x):
    """bf16 rows [rows, H] (H a multiple of 16) -> (q [rows, H/2] uint8, two
    e2m1 codes per byte, even value in the low nibble; scale [rows, H/16] uint8
    E4M3 codes): the pages' 4-bit row, one scale byte per 16 values."""
    xb = _c(x, np.uint16)
    rows, H = xb.shape
    assert H % 16 == 0
    q = np.zeros((rows, H // 2), np.uint8)
    sc = np.zeros((rows, H // 16), np.uint8)
    _load().oracle_quantize_nvfp4(rows, H, _p(xb), _p(q), _p(sc))
    return q, sc


def pack_nvfp4(hidden, token_rank_slot, cap_rank: int):
    """Quantise every hidden row once to the 16-value-block 4-bit row, then
    pack codes and scales once per distinct rank (plain byte copies)."""
    q, sc = quantize_nvfp4(hidden)
    rq, src, err = pack(q.view(np.uint16), token_rank_slot, cap_rank)
    rs, _, _ = pack(sc.view(np.uint16), token_rank_slot, cap_rank)
    return rq.view(np.uint8), rs.view(np.uint8), src, err


def permute_nvfp4(rank_q, rank_scale, rank_src_token, lay: dict, topk_ids, E: int,
                  cap_expert: int):
    """Regroup 16-value-block 4-bit rows by expert: codes and scales move as
    bytes, exactly as permute_mxfp8 moves them."""
    return permute_mxfp8(rank_q, rank_scale, rank_src_token, lay, topk_ids, E, cap_expert)


def place_slots(y_slots: np.ndarray, pair_row: np.ndarray, rows: int) -> np.ndarray:
    """Scatter per-(token, slot) rows [T, k, H] to their expert-grouped rows,
    as an expert kernel that writes its output in input order would."""
    T, k, H = y_slots.shape
    out = np.zeros((rows, H), np.uint16)
    pr = np.asarray(pair_row).reshape(-1)
    ok = (pr >= 0) & (pr < rows)
    out[pr[ok]] = y_slots.reshape(T * k, H)[ok]
    return out


def dispatch_combine(hidden, topk_ids, topk_weights, E: int, R: int, expert_out_slots=None):
    """One full pass of the path: layout, pack, permute, then combine of either the
    given expert outputs (in token-slot order) or, if None, the identity experts."""
    T, k = np.asarray(topk_ids).shape
    lay = layout(topk_ids, E, R)
    cap_rank = T * min(k, R)
    cap_expert = T * k
    rank_buf, src, e1 = pack(hidden, lay["token_rank_slot"], cap_rank)
    expert_buf, src_pair, e2 = permute(rank_buf, src, lay, topk_ids, E, cap_expert)
    if expert_out_slots is None:
        eo = expert_buf
    else:
        eo = place_slots(expert_out_slots, lay["pair_row"], cap_expert)
    out, out32, e3 = combine(eo, lay["pair_row"], topk_weights)
    return dict(layout=lay, rank_buf=rank_buf, rank_src_token=src, expert_buf=expert_buf,
                expert_src_pair=src_pair, expert_out=eo, out=out, out_f32=out32,
                err=lay["err"] | e1 | e2 | e3)
