"""Python binding of libmoe_dispatch.so (MoE token dispatch and combine on
MI355X / gfx950).

Argument marshalling only: every step runs in the library's HIP kernels on the
caller's current torch stream. Torch tensors supply device memory; bf16 rows
may be passed as torch.bfloat16, torch.int16 or torch.uint16 tensors (the bits
are what matter). There is no CPU fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loads the HIP runtime the library binds to; must come first

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_dispatch.so")

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_HIP = -2
ERRBIT_BAD_ID = 1
ERRBIT_RANK_CAP = 2
ERRBIT_EXPERT_CAP = 4

EXPORTS = ("moe_abi_version", "moe_status_string", "moe_dispatch_layout",
           "moe_dispatch_layout_noalloc", "moe_layout_workspace_bytes", "moe_dispatch_pack",
           "moe_permute_by_expert", "moe_combine", "moe_combine_rank_partial",
           "moe_combine_ranks", "moe_dispatch_pack_mxfp8", "moe_permute_by_expert_mxfp8",
           "moe_dispatch_pack_mxfp4", "moe_permute_by_expert_mxfp4",
           "moe_dispatch_pack_nvfp4", "moe_permute_by_expert_nvfp4",
           "moe_dispatch", "moe_dispatch_quantised", "moe_testing_set_layout_form",
           "moe_testing_set_layout_match",
           "moe_testing_set_dispatch_fused", "moe_testing_time_next_launch")


ABI_VERSION = 9

# Quantised wire formats: name -> (code bits per value, values per scale byte).
WIRE_FORMATS = {"mxfp8": (8, 32), "mxfp4": (4, 32), "nvfp4": (4, 16)}
WIRE_CODES = {"mxfp8": 1, "mxfp4": 2, "nvfp4": 3}  # moe_dispatch_quantised's format


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("R", ctypes.c_int32), ("k", ctypes.c_int32), ("align", ctypes.c_int32),
                ("block", ctypes.c_int32)]

    def __init__(self, T=0, H=8, E=1, R=1, k=1, align=1, block=0):
        super().__init__(T, H, E, R, k, align, block)


class MoeError(RuntimeError):
    pass


_lib = None


def lib():
    """Load the library (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    for name in EXPORTS:
        if not hasattr(L, name):
            raise MoeError(f"{LIB_PATH} does not export {name}")
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    shp = ctypes.POINTER(MoeShape)
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_dispatch_layout.restype = ctypes.c_int
    L.moe_dispatch_layout.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp,
                                      vp]
    L.moe_dispatch_layout_noalloc.restype = ctypes.c_int
    L.moe_dispatch_layout_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_layout_workspace_bytes.restype = ctypes.c_size_t
    L.moe_layout_workspace_bytes.argtypes = [shp]
    L.moe_dispatch_pack.restype = ctypes.c_int
    L.moe_dispatch_pack.argtypes = [shp, vp, vp, vp, vp, i64, vp, vp]
    L.moe_permute_by_expert.restype = ctypes.c_int
    L.moe_permute_by_expert.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64, vp,
                                        vp]
    L.moe_combine.restype = ctypes.c_int
    L.moe_combine.argtypes = [shp, vp, vp, vp, i64, vp, vp, vp, vp]
    L.moe_combine_rank_partial.restype = ctypes.c_int
    L.moe_combine_rank_partial.argtypes = [shp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp]
    L.moe_combine_ranks.restype = ctypes.c_int
    L.moe_combine_ranks.argtypes = [shp, vp, vp, i64, vp, vp, vp, vp]
    L.moe_dispatch_pack_mxfp8.restype = ctypes.c_int
    L.moe_dispatch_pack_mxfp8.argtypes = [shp, vp, vp, vp, vp, vp, i64, vp, vp]
    L.moe_permute_by_expert_mxfp8.restype = ctypes.c_int
    L.moe_permute_by_expert_mxfp8.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp,
                                              vp, i64, vp, vp]
    L.moe_dispatch_pack_mxfp4.restype = ctypes.c_int
    L.moe_dispatch_pack_mxfp4.argtypes = L.moe_dispatch_pack_mxfp8.argtypes
    L.moe_permute_by_expert_mxfp4.restype = ctypes.c_int
    L.moe_permute_by_expert_mxfp4.argtypes = L.moe_permute_by_expert_mxfp8.argtypes
    L.moe_dispatch_pack_nvfp4.restype = ctypes.c_int
    L.moe_dispatch_pack_nvfp4.argtypes = L.moe_dispatch_pack_mxfp8.argtypes
    L.moe_permute_by_expert_nvfp4.restype = ctypes.c_int
    L.moe_permute_by_expert_nvfp4.argtypes = L.moe_permute_by_expert_mxfp8.argtypes
    L.moe_dispatch.restype = ctypes.c_int
    L.moe_dispatch.argtypes = [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64,
                               vp, ctypes.c_size_t, vp, vp]
    L.moe_dispatch_quantised.restype = ctypes.c_int
    L.moe_dispatch_quantised.argtypes = [shp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, i64, vp, vp, vp, i64, vp, ctypes.c_size_t, vp,
                                         vp]
    L.moe_testing_set_dispatch_fused.restype = ctypes.c_int
    L.moe_testing_set_dispatch_fused.argtypes = [ctypes.c_int]
    L.moe_testing_set_layout_form.restype = ctypes.c_int
    L.moe_testing_set_layout_form.argtypes = [ctypes.c_int]
    L.moe_testing_set_layout_match.restype = ctypes.c_int
    L.moe_testing_set_layout_match.argtypes = [ctypes.c_int]
    L.moe_testing_time_next_launch.restype = ctypes.c_int
    L.moe_testing_time_next_launch.argtypes = [vp, vp]
    if L.moe_abi_version() != ABI_VERSION:
        raise MoeError(f"{LIB_PATH} has ABI version {L.moe_abi_version()}, this binding "
                       f"expects {ABI_VERSION}: rebuild with __graft_entry__.build()")
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        msg = lib().moe_status_string(status).decode()
        raise MoeError(f"{what} failed: {msg} ({status})")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise MoeError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor | None, name: str, shape: tuple | None = None,
          min_numel: int | None = None) -> None:
    """Checks a tensor against the shape of the call before its pointer goes to
    the library, which cannot see buffer lengths: `shape` exactly, or at least
    `min_numel` elements. Raises MoeError."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name} has shape {tuple(t.shape)}, the call needs {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise MoeError(f"{name} has {t.numel()} elements, the call needs at least {min_numel}")


def _rows(t: torch.Tensor, name: str, width: int) -> int:
    """Rows of a row buffer [rows, width]; raises MoeError on another width."""
    if t.dim() != 2 or t.shape[1] != width:
        raise MoeError(f"{name} has shape {tuple(t.shape)}, the call needs [rows, {width}]")
    return t.shape[0]


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _i32(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise MoeError(f"expected int32, got {t.dtype}")
    return t


def _check_err(t: torch.Tensor | None) -> None:
    """The device error word: None, or an int32 tensor of at least one element
    (the kernels OR 4 bytes into its first element)."""
    if t is not None and (t.dtype != torch.int32 or t.numel() < 1):
        raise MoeError(f"err must be an int32 tensor of at least 1 element, got {t.dtype} "
                       f"with {t.numel()}")


def _err(t: torch.Tensor | None):
    _check_err(t)
    return _ptr(t)


def _rows16(t: torch.Tensor) -> torch.Tensor:
    if t.element_size() != 2:
        raise MoeError(f"expected a 16-bit row tensor, got {t.dtype}")
    return t


@dataclass
class Shape:
    T: int
    H: int
    E: int
    R: int
    k: int
    align: int = 1  # expert runs padded to a multiple of align rows
    block: int = 0  # > 0: a fixed block of rows per expert (masked layout)

    def c(self) -> MoeShape:
        return MoeShape(self.T, self.H, self.E, self.R, self.k, self.align, self.block)

    @property
    def cap_rank(self) -> int:
        """Worst-case rank-buffer rows: T * min(k, R)."""
        return self.T * min(self.k, self.R)

    @property
    def cap_expert(self) -> int:
        """Worst-case expert-buffer rows: T*k + E*(align-1), or E*block."""
        if self.block > 0:
            return self.E * self.block
        return self.T * self.k + self.E * (self.align - 1)


def layout_workspace_bytes(shape: "Shape") -> int:
    """moe_layout_workspace_bytes: scratch the two-launch layout needs (0: none)."""
    return int(lib().moe_layout_workspace_bytes(ctypes.byref(shape.c())))


def layout(topk_ids: torch.Tensor, E: int, R: int, H: int = 8, *, align: int = 1,
           block: int = 0, err=None, out: dict | None = None,
           workspace: torch.Tensor | None = None) -> dict:
    """moe_dispatch_layout: counts, offsets, token_rank_slot [T,R], pair_row [T,k].
    `workspace` (a device tensor of at least layout_workspace_bytes bytes)
    selects the two-launch layout; without it every workgroup counts all ids."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    shape = Shape(T, H, E, R, k, align, block)
    _check_err(err)
    if out is not None:
        for key, want in (("rank_counts", (R,)), ("rank_offsets", (R + 1,)),
                          ("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                          ("token_rank_slot", (T, R)), ("pair_row", (T, k))):
            _need(out[key], key, want)
            if out[key].dtype != torch.int32:
                raise MoeError(f"{key} must be int32, got {out[key].dtype}")
    if out is None:
        out = dict(
            rank_counts=torch.empty(R, dtype=torch.int32, device=dev),
            rank_offsets=torch.empty(R + 1, dtype=torch.int32, device=dev),
            expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
            expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            token_rank_slot=torch.empty((T, R), dtype=torch.int32, device=dev),
            pair_row=torch.empty((T, k), dtype=torch.int32, device=dev),
        )
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().moe_dispatch_layout(
        ctypes.byref(shape.c()), _ptr(_i32(topk_ids)), _ptr(_i32(out["rank_counts"])),
        _ptr(_i32(out["rank_offsets"])), _ptr(_i32(out["expert_counts"])),
        _ptr(_i32(out["expert_offsets"])), _ptr(_i32(out["token_rank_slot"])),
        _ptr(_i32(out["pair_row"])), _ptr(workspace), ws_bytes,
        _err(err), _stream(dev))
    _check(st, "moe_dispatch_layout")
    return out


def layout_noalloc(topk_ids: torch.Tensor, E: int, R: int, H: int = 8, *, align: int = 1,
                   block: int = 0, err=None, out: dict) -> dict:
    """moe_dispatch_layout_noalloc: the layout into caller-provided `out`
    tensors (the same keys as layout()), its workspace the library's static
    array on the current device; this call allocates nothing."""
    T, k = topk_ids.shape
    shape = Shape(T, H, E, R, k, align, block)
    _check_err(err)
    for key, want in (("rank_counts", (R,)), ("rank_offsets", (R + 1,)),
                      ("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                      ("token_rank_slot", (T, R)), ("pair_row", (T, k))):
        _need(out[key], key, want)
        if out[key].dtype != torch.int32:
            raise MoeError(f"{key} must be int32, got {out[key].dtype}")
    st = lib().moe_dispatch_layout_noalloc(
        ctypes.byref(shape.c()), _ptr(_i32(topk_ids)), _ptr(out["rank_counts"]),
        _ptr(out["rank_offsets"]), _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
        _ptr(out["token_rank_slot"]), _ptr(out["pair_row"]), _err(err),
        _stream(topk_ids.device))
    _check(st, "moe_dispatch_layout_noalloc")
    return out


def pack(hidden: torch.Tensor, token_rank_slot: torch.Tensor, E: int, k: int, rank_buf,
         rank_src_token, *, err=None) -> None:
    """moe_dispatch_pack into caller-provided rank_buf [cap_rank, H] and
    rank_src_token [cap_rank]."""
    _check_err(err)
    T, H = hidden.shape
    R = token_rank_slot.shape[1]
    _need(token_rank_slot, "token_rank_slot", (T, R))
    cap = _rows(rank_buf, "rank_buf", H)
    _need(rank_src_token, "rank_src_token", min_numel=cap)
    shape = Shape(T, H, E, R, k)
    st = lib().moe_dispatch_pack(
        ctypes.byref(shape.c()), _ptr(_rows16(hidden)), _ptr(_i32(token_rank_slot)),
        _ptr(_rows16(rank_buf)), _ptr(_i32(rank_src_token)), rank_buf.shape[0], _err(err),
        _stream(hidden.device))
    _check(st, "moe_dispatch_pack")


def permute(rank_buf, rank_src_token, rank_offsets, topk_ids, pair_row, E: int, expert_buf,
            expert_src_pair, *, expert_counts=None, expert_offsets=None, align: int = 1,
            block: int = 0, err=None) -> None:
    """moe_permute_by_expert into caller-provided expert_buf [cap_expert, H].
    A padded (align > 1) or blocked (block > 0) layout needs the layout's
    expert_counts and expert_offsets, to mark its padding rows."""
    _check_err(err)
    T, k = topk_ids.shape
    H = rank_buf.shape[1]
    R = rank_offsets.shape[0] - 1
    _need(pair_row, "pair_row", (T, k))
    cap_r = _rows(rank_buf, "rank_buf", H)
    _need(rank_src_token, "rank_src_token", min_numel=cap_r)
    cap_e = _rows(expert_buf, "expert_buf", H)
    _need(expert_src_pair, "expert_src_pair", min_numel=cap_e)
    _need(expert_counts, "expert_counts", (E,))
    _need(expert_offsets, "expert_offsets", (E + 1,))
    shape = Shape(T, H, E, R, k, align, block)
    st = lib().moe_permute_by_expert(
        ctypes.byref(shape.c()), _ptr(_rows16(rank_buf)), _ptr(_i32(rank_src_token)),
        _ptr(_i32(rank_offsets)), _ptr(_i32(topk_ids)), _ptr(_i32(pair_row)),
        _ptr(None if expert_counts is None else _i32(expert_counts)),
        _ptr(None if expert_offsets is None else _i32(expert_offsets)),
        rank_buf.shape[0], _ptr(_rows16(expert_buf)), _ptr(_i32(expert_src_pair)),
        expert_buf.shape[0], _err(err), _stream(rank_buf.device))
    _check(st, "moe_permute_by_expert")


def dispatch_all(hidden, topk_ids, E: int, R: int, out: dict, rank_buf, rank_src_token,
                 expert_buf, expert_src_pair, *, align: int = 1, block: int = 0,
                 workspace: torch.Tensor | None = None, err=None) -> None:
    """moe_dispatch: layout, pack and permute in one call (one kernel launch
    for up to 256 tokens with k in {1, 2, 4, 6, 8}, up to 64
    for another k; else the layout and one pack-and-permute kernel), into
    the caller's tensors: `out`
    holds the layout's outputs (the keys of layout()), rank_buf [cap_rank, H],
    rank_src_token [cap_rank], expert_buf [cap_expert, H], expert_src_pair
    [cap_expert]."""
    _check_err(err)
    T, k = topk_ids.shape
    H = hidden.shape[1]
    _need(hidden, "hidden", (T, H))
    for key, want in (("rank_counts", (R,)), ("rank_offsets", (R + 1,)),
                      ("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                      ("token_rank_slot", (T, R)), ("pair_row", (T, k))):
        _need(out[key], key, want)
        _i32(out[key])
    cap_r = _rows(rank_buf, "rank_buf", H)
    _need(rank_src_token, "rank_src_token", min_numel=cap_r)
    cap_e = _rows(expert_buf, "expert_buf", H)
    _need(expert_src_pair, "expert_src_pair", min_numel=cap_e)
    shape = Shape(T, H, E, R, k, align, block)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().moe_dispatch(
        ctypes.byref(shape.c()), _ptr(_rows16(hidden)), _ptr(_i32(topk_ids)),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["expert_counts"]),
        _ptr(out["expert_offsets"]), _ptr(out["token_rank_slot"]), _ptr(out["pair_row"]),
        _ptr(_rows16(rank_buf)), _ptr(_i32(rank_src_token)), rank_buf.shape[0],
        _ptr(_rows16(expert_buf)), _ptr(_i32(expert_src_pair)), expert_buf.shape[0],
        _ptr(workspace), ws_bytes, _err(err), _stream(hidden.device))
    _check(st, "moe_dispatch")


def _bytes(t: torch.Tensor) -> torch.Tensor:
    if t.element_size() != 1 or not t.is_contiguous():
        raise MoeError(f"expected a contiguous 8-bit tensor, got {t.dtype}")
    return t


def _wire(fmt) -> tuple:
    """A wire format name (or the bits 8 / 4 of an MX format) -> (name, code
    bits per value, values per scale byte)."""
    name = {8: "mxfp8", 4: "mxfp4"}.get(fmt, fmt)
    if name not in WIRE_FORMATS:
        raise MoeError(f"unknown wire format {fmt!r}: one of {sorted(WIRE_FORMATS)}")
    return (name,) + WIRE_FORMATS[name]


def pack_mx(fmt, hidden: torch.Tensor, token_rank_slot: torch.Tensor, E: int, k: int,
            rank_q, rank_scale, rank_src_token, *, err=None) -> None:
    """moe_dispatch_pack_mxfp8 / _mxfp4 / _nvfp4 (fmt "mxfp8", "mxfp4",
    "nvfp4", or the bits 8 / 4 of an MX format): quantise each hidden row once
    and pack it once per distinct rank into rank_q [cap_rank, H*bits/8] (uint8
    codes) and rank_scale [cap_rank, H/block] (uint8 scales)."""
    name, bits, blk = _wire(fmt)
    _check_err(err)
    T, H = hidden.shape
    R = token_rank_slot.shape[1]
    _need(token_rank_slot, "token_rank_slot", (T, R))
    cap = _rows(rank_q, "rank_q", H * bits // 8)
    _need(rank_scale, "rank_scale", (cap, H // blk))
    _need(rank_src_token, "rank_src_token", min_numel=cap)
    shape = Shape(T, H, E, R, k)
    fn = getattr(lib(), f"moe_dispatch_pack_{name}")
    st = fn(ctypes.byref(shape.c()), _ptr(_rows16(hidden)), _ptr(_i32(token_rank_slot)),
            _ptr(_bytes(rank_q)), _ptr(_bytes(rank_scale)), _ptr(_i32(rank_src_token)),
            rank_q.shape[0], _err(err), _stream(hidden.device))
    _check(st, f"moe_dispatch_pack_{name}")


def dispatch_all_mx(fmt, hidden, topk_ids, E: int, R: int, out: dict, rank_q, rank_scale,
                    rank_src_token, expert_q, expert_scale, expert_src_pair, *, align: int = 1,
                    block: int = 0, workspace: torch.Tensor | None = None, err=None) -> None:
    """moe_dispatch_quantised: layout, quantise-and-pack and permute of the
    quantised rows in one call (one kernel launch for a decode-sized batch, else
    the layout and one quantise-pack-and-permute kernel, as dispatch_all), into
    the caller's tensors: `out` holds the layout's outputs,
    rank_q [cap_rank, H*bits/8] and rank_scale [cap_rank, H/block] (uint8),
    rank_src_token [cap_rank], expert_q / expert_scale / expert_src_pair
    likewise with cap_expert rows."""
    name, bits, blk = _wire(fmt)
    _check_err(err)
    T, k = topk_ids.shape
    H = hidden.shape[1]
    _need(hidden, "hidden", (T, H))
    for key, want in (("rank_counts", (R,)), ("rank_offsets", (R + 1,)),
                      ("expert_counts", (E,)), ("expert_offsets", (E + 1,)),
                      ("token_rank_slot", (T, R)), ("pair_row", (T, k))):
        _need(out[key], key, want)
        _i32(out[key])
    cap_r = _rows(rank_q, "rank_q", H * bits // 8)
    _need(rank_scale, "rank_scale", (cap_r, H // blk))
    _need(rank_src_token, "rank_src_token", min_numel=cap_r)
    cap_e = _rows(expert_q, "expert_q", H * bits // 8)
    _need(expert_scale, "expert_scale", (cap_e, H // blk))
    _need(expert_src_pair, "expert_src_pair", min_numel=cap_e)
    shape = Shape(T, H, E, R, k, align, block)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().moe_dispatch_quantised(
        ctypes.byref(shape.c()), WIRE_CODES[name], _ptr(_rows16(hidden)), _ptr(_i32(topk_ids)),
        _ptr(out["rank_counts"]), _ptr(out["rank_offsets"]), _ptr(out["expert_counts"]),
        _ptr(out["expert_offsets"]), _ptr(out["token_rank_slot"]), _ptr(out["pair_row"]),
        _ptr(_bytes(rank_q)), _ptr(_bytes(rank_scale)), _ptr(_i32(rank_src_token)),
        rank_q.shape[0], _ptr(_bytes(expert_q)), _ptr(_bytes(expert_scale)),
        _ptr(_i32(expert_src_pair)), expert_q.shape[0], _ptr(workspace), ws_bytes, _err(err),
        _stream(hidden.device))
    _check(st, "moe_dispatch_quantised")


def pack_mxfp8(*args, **kw) -> None:
    pack_mx("mxfp8", *args, **kw)


def pack_mxfp4(*args, **kw) -> None:
    pack_mx("mxfp4", *args, **kw)


def pack_nvfp4(*args, **kw) -> None:
    pack_mx("nvfp4", *args, **kw)


def permute_mx(fmt, rank_q, rank_scale, rank_src_token, rank_offsets, topk_ids, pair_row,
               E: int, expert_q, expert_scale, expert_src_pair, *, expert_counts=None,
               expert_offsets=None, align: int = 1, block: int = 0, err=None) -> None:
    """moe_permute_by_expert_mxfp8 / _mxfp4 / _nvfp4: the codes and scales of
    each rank-buffer row to the rows of its token's experts on that rank."""
    name, bits, blk = _wire(fmt)
    _check_err(err)
    T, k = topk_ids.shape
    H = rank_q.shape[1] * 8 // bits
    R = rank_offsets.shape[0] - 1
    _need(pair_row, "pair_row", (T, k))
    cap_r = rank_q.shape[0]
    _need(rank_scale, "rank_scale", (cap_r, H // blk))
    _need(rank_src_token, "rank_src_token", min_numel=cap_r)
    cap_e = _rows(expert_q, "expert_q", rank_q.shape[1])
    _need(expert_scale, "expert_scale", (cap_e, H // blk))
    _need(expert_src_pair, "expert_src_pair", min_numel=cap_e)
    _need(expert_counts, "expert_counts", (E,))
    _need(expert_offsets, "expert_offsets", (E + 1,))
    shape = Shape(T, H, E, R, k, align, block)
    fn = getattr(lib(), f"moe_permute_by_expert_{name}")
    st = fn(ctypes.byref(shape.c()), _ptr(_bytes(rank_q)), _ptr(_bytes(rank_scale)),
            _ptr(_i32(rank_src_token)), _ptr(_i32(rank_offsets)), _ptr(_i32(topk_ids)),
            _ptr(_i32(pair_row)), _ptr(None if expert_counts is None else _i32(expert_counts)),
            _ptr(None if expert_offsets is None else _i32(expert_offsets)), rank_q.shape[0],
            _ptr(_bytes(expert_q)), _ptr(_bytes(expert_scale)), _ptr(_i32(expert_src_pair)),
            expert_q.shape[0], _err(err), _stream(rank_q.device))
    _check(st, f"moe_permute_by_expert_{name}")


def permute_mxfp8(*args, **kw) -> None:
    permute_mx("mxfp8", *args, **kw)


def permute_mxfp4(*args, **kw) -> None:
    permute_mx("mxfp4", *args, **kw)


def permute_nvfp4(*args, **kw) -> None:
    permute_mx("nvfp4", *args, **kw)


def combine(expert_out, pair_row, topk_weights, E: int, R: int, out, *, out_f32=None,
            err=None) -> None:
    """moe_combine: out [T, H] bf16 (and optionally out_f32 [T, H] float32)."""
    _check_err(err)
    T, k = pair_row.shape
    H = out.shape[1]
    if topk_weights.dtype != torch.float32:
        raise MoeError("topk_weights must be float32")
    if out_f32 is not None and out_f32.dtype != torch.float32:
        raise MoeError("out_f32 must be float32")
    _need(topk_weights, "topk_weights", (T, k))
    _need(out, "out", (T, H))
    _need(out_f32, "out_f32", (T, H))
    _rows(expert_out, "expert_out", H)
    shape = Shape(T, H, E, R, k)
    st = lib().moe_combine(
        ctypes.byref(shape.c()), _ptr(_rows16(expert_out)), _ptr(_i32(pair_row)),
        _ptr(topk_weights), expert_out.shape[0], _ptr(_rows16(out)), _ptr(out_f32), _err(err),
        _stream(out.device))
    _check(st, "moe_combine")


def combine_rank_partial(expert_out, rank_src_token, rank_offsets, topk_ids, pair_row,
                         topk_weights, E: int, partial, *, partial_f32=None, err=None) -> None:
    """moe_combine_rank_partial: one bf16 partial row per rank-buffer row into
    caller-provided partial [cap_rank, H] (and optionally partial_f32)."""
    _check_err(err)
    T, k = topk_ids.shape
    H = partial.shape[1]
    R = rank_offsets.shape[0] - 1
    if topk_weights.dtype != torch.float32:
        raise MoeError("topk_weights must be float32")
    if partial_f32 is not None and partial_f32.dtype != torch.float32:
        raise MoeError("partial_f32 must be float32")
    _need(pair_row, "pair_row", (T, k))
    _need(topk_weights, "topk_weights", (T, k))
    cap_r = _rows(partial, "partial", H)
    _need(partial_f32, "partial_f32", (cap_r, H))
    _need(rank_src_token, "rank_src_token", min_numel=cap_r)
    _rows(expert_out, "expert_out", H)
    shape = Shape(T, H, E, R, k)
    st = lib().moe_combine_rank_partial(
        ctypes.byref(shape.c()), _ptr(_rows16(expert_out)), _ptr(_i32(rank_src_token)),
        _ptr(_i32(rank_offsets)), _ptr(_i32(topk_ids)), _ptr(_i32(pair_row)),
        _ptr(topk_weights), expert_out.shape[0], partial.shape[0], _ptr(_rows16(partial)),
        _ptr(partial_f32), _err(err), _stream(partial.device))
    _check(st, "moe_combine_rank_partial")


def combine_ranks(partial, token_rank_slot, E: int, k: int, out, *, out_f32=None,
                  err=None) -> None:
    """moe_combine_ranks: out [T, H] = sum over ranks of the token's partial rows."""
    _check_err(err)
    T, R = token_rank_slot.shape
    H = out.shape[1]
    if out_f32 is not None and out_f32.dtype != torch.float32:
        raise MoeError("out_f32 must be float32")
    _need(out, "out", (T, H))
    _need(out_f32, "out_f32", (T, H))
    _rows(partial, "partial", H)
    shape = Shape(T, H, E, R, k)
    st = lib().moe_combine_ranks(
        ctypes.byref(shape.c()), _ptr(_rows16(partial)), _ptr(_i32(token_rank_slot)),
        partial.shape[0], _ptr(_rows16(out)), _ptr(out_f32), _err(err), _stream(out.device))
    _check(st, "moe_combine_ranks")


def time_next_launch(start: "torch.cuda.Event | None", stop: "torch.cuda.Event | None") -> None:
    """moe_testing_time_next_launch: the library's next kernel launch records
    `start` as it begins and `stop` as it ends (a measurement hook; both events
    must have been recorded once, so that they exist). None, None disarms."""
    if (start is None) != (stop is None):
        raise MoeError("give both events or neither")
    if start is not None and not (start.cuda_event and stop.cuda_event):
        raise MoeError("record both events once before arming them")
    st = lib().moe_testing_time_next_launch(
        None if start is None else ctypes.c_void_p(start.cuda_event),
        None if stop is None else ctypes.c_void_p(stop.cuda_event))
    _check(st, "moe_testing_time_next_launch")


class Buffers:
    """Every buffer of one dispatch + combine pass, allocated once for a shape
    at worst-case size (Shape.cap_rank and Shape.cap_expert rows)."""

    def __init__(self, shape: Shape, device, row_dtype=torch.bfloat16, want_f32: bool = False):
        T, H, E, R, k = shape.T, shape.H, shape.E, shape.R, shape.k
        d = device
        i32 = torch.int32
        self.shape = shape
        self.rank_counts = torch.empty(R, dtype=i32, device=d)
        self.rank_offsets = torch.empty(R + 1, dtype=i32, device=d)
        self.expert_counts = torch.empty(E, dtype=i32, device=d)
        self.expert_offsets = torch.empty(E + 1, dtype=i32, device=d)
        self.token_rank_slot = torch.empty((T, R), dtype=i32, device=d)
        self.pair_row = torch.empty((T, k), dtype=i32, device=d)
        self.rank_buf = torch.empty((shape.cap_rank, H), dtype=row_dtype, device=d)
        self.rank_src_token = torch.empty(shape.cap_rank, dtype=i32, device=d)
        self.expert_buf = torch.empty((shape.cap_expert, H), dtype=row_dtype, device=d)
        self.expert_src_pair = torch.empty(shape.cap_expert, dtype=i32, device=d)
        self.out = torch.empty((T, H), dtype=row_dtype, device=d)
        self.out_f32 = torch.empty((T, H), dtype=torch.float32, device=d) if want_f32 else None
        self.err = torch.zeros(1, dtype=i32, device=d)
        ws = layout_workspace_bytes(shape)
        self.workspace = torch.empty(max(ws, 4) // 4, dtype=i32, device=d) if ws else None

    def layout_dict(self) -> dict:
        return dict(rank_counts=self.rank_counts, rank_offsets=self.rank_offsets,
                    expert_counts=self.expert_counts, expert_offsets=self.expert_offsets,
                    token_rank_slot=self.token_rank_slot, pair_row=self.pair_row)


def dispatch(buf: Buffers, hidden, topk_ids) -> None:
    """Layout, pack and permute into `buf` (three library calls, no host sync)."""
    s = buf.shape
    layout(topk_ids, s.E, s.R, s.H, align=s.align, block=s.block, err=buf.err,
           out=buf.layout_dict(), workspace=buf.workspace)
    pack(hidden, buf.token_rank_slot, s.E, s.k, buf.rank_buf, buf.rank_src_token, err=buf.err)
    permute(buf.rank_buf, buf.rank_src_token, buf.rank_offsets, topk_ids, buf.pair_row, s.E,
            buf.expert_buf, buf.expert_src_pair, expert_counts=buf.expert_counts,
            expert_offsets=buf.expert_offsets, align=s.align, block=s.block, err=buf.err)


def combine_into(buf: Buffers, expert_out, topk_weights) -> None:
    s = buf.shape
    combine(expert_out, buf.pair_row, topk_weights, s.E, s.R, buf.out, out_f32=buf.out_f32,
            err=buf.err)
