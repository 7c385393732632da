"""Seeded synthetic inputs for MoE token dispatch and combine.

Shared by the oracle side and the GPU side of every test and of the benchmark.
It holds none of the dispatch/combine arithmetic: it only draws hidden states,
router logits (top-k ids and renormalised softmax weights) and expert outputs.
The heavy lifting is in ``synth.c`` (counter-based splitmix64 + Box-Muller).

Workloads follow the shapes the pages discuss: DeepSeek-V4.1-Flash dims for
decode and prefill (hidden 5,120, 384 experts, top-6, 8 GPUs with 48 experts
each; "A2A backends" page, sections 1.1 and 1.3), GLM-5.3 dims for the skewed
case (hidden 6,144, 256 experts, top-8; "How GPUs Talk to Each Other", section
7) and DeepSeek-V3 dims for the adversarial case (hidden 7,168, 256 experts,
top-8; "Beyond One GPU", section on MoE parallelism).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

STREAM_HIDDEN = 0
STREAM_LOGITS = 1
STREAM_EXPERT = 2
STREAM_PERM = 3


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    R: int
    k: int
    seed: int
    routing: str = "uniform"  # "uniform" | "zipf" | "adversarial"
    zipf_s: float = 1.2
    adv_frac: float = 0.1
    notes: str = field(default="", compare=False)

    @property
    def m(self) -> int:
        return self.E // self.R

    def describe(self) -> str:
        return (f"{self.name} T={self.T} H={self.H} E={self.E} R={self.R} "
                f"top-{self.k} ({self.routing})")


WORKLOADS = {
    "tiny": Workload("tiny", 256, 512, 16, 4, 2, 10),
    "decode": Workload("decode", 64, 5120, 384, 8, 6, 20),
    "prefill": Workload("prefill", 4096, 5120, 384, 8, 6, 30),
    "skew": Workload("skew", 8192, 6144, 256, 8, 8, 40, routing="zipf"),
    "adv": Workload("adv", 16384, 7168, 256, 8, 8, 50, routing="adversarial"),
}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32
    vp = ctypes.c_void_p
    lib.synth_hash.restype = u64
    lib.synth_hash.argtypes = [u64, u64, u64]
    lib.synth_normal.restype = ctypes.c_double
    lib.synth_normal.argtypes = [u64, u64, u64]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_permutation.argtypes = [u64, u64, u64, i32, vp]
    lib.synth_router.argtypes = [u64, i32, i32, i32, vp, vp, i32, ctypes.c_float, vp, vp]
    lib.synth_expert_out_slots.argtypes = [u64, i32, i32, i32, i32, vp, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def normal_bf16(seed: int, stream: int, n: int, base: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(seed, stream, base, n, _ptr(out))
    return out


def normal_f32(seed: int, stream: int, n: int, base: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_normal_f32(seed, stream, base, n, _ptr(out))
    return out


def permutation(seed: int, stream: int, n: int, salt: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    if n:
        _load().synth_permutation(seed, stream, salt, n, _ptr(out))
    return out


def hidden(w: Workload) -> np.ndarray:
    """bf16 bit patterns [T, H], N(0,1)."""
    return normal_bf16(w.seed, STREAM_HIDDEN, w.T * w.H).reshape(w.T, w.H)


def router_bias(w: Workload) -> np.ndarray | None:
    """Per-expert logit bias: log of a Zipf(s) popularity, hot experts placed by
    a seeded permutation (rank rho(e) = position of e in the permutation + 1)."""
    if w.routing != "zipf":
        return None
    order = permutation(w.seed, STREAM_PERM, w.E)
    rho = np.empty(w.E, dtype=np.float64)
    rho[order] = np.arange(1, w.E + 1, dtype=np.float64)
    return (-w.zipf_s * np.log(rho)).astype(np.float32)


def forced_tokens(w: Workload) -> np.ndarray | None:
    """Adversarial case: exactly floor(adv_frac*T) tokens, picked by a seeded
    shuffle, have every expert outside rank 0 pushed down by 1e4."""
    if w.routing != "adversarial":
        return None
    n = int(math.floor(w.adv_frac * w.T))
    order = permutation(w.seed, STREAM_PERM, w.T, salt=1 << 40)
    force = np.zeros(w.T, dtype=np.uint8)
    force[order[:n]] = 1
    return force


def routing(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    return router(w.seed, w.T, w.E, w.k, bias=router_bias(w), force=forced_tokens(w),
                  force_below=w.m)


def router(seed: int, T: int, E: int, k: int, bias=None, force=None, force_below: int = 0,
           force_offset: float = -1.0e4) -> tuple[np.ndarray, np.ndarray]:
    """Top-k ids [T,k] int32 and renormalised softmax weights [T,k] float32."""
    assert 1 <= k <= E
    ids = np.empty((T, k), dtype=np.int32)
    wts = np.empty((T, k), dtype=np.float32)
    if T == 0:
        return ids, wts
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    f = None if force is None else np.ascontiguousarray(force, dtype=np.uint8)
    _load().synth_router(seed, T, E, k, None if b is None else _ptr(b),
                         None if f is None else _ptr(f), force_below,
                         ctypes.c_float(force_offset), _ptr(ids), _ptr(wts))
    return ids, wts


def expert_out_slots(seed: int, E: int, H: int, ids: np.ndarray) -> np.ndarray:
    """Synthetic expert outputs in (token, slot) order, bf16 bits [T, k, H].
    Value at (t, j, h) depends only on (t, ids[t,j], h); invalid ids give zeros."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    y = np.empty((T, k, H), dtype=np.uint16)
    if T * k * H:
        _load().synth_expert_out_slots(seed, T, E, k, H, _ptr(ids), _ptr(y))
    return y
