"""Seeded random shapes through the whole path, against the oracle: the
layout (in the form forced for the case), pack, permute and combine with plain,
padded and masked expert layouts, the two-stage combine, and the MXFP8 / MXFP4
dispatch, and the one-call moe_dispatch. Every shape parameter is drawn (T around the 256-token tile size and
up to a few thousand, H any multiple of 8, R from 1 to 64, E up to 1024, k up
to 16, -1 / duplicate / out-of-range ids), so the cases reach corners that
the hand-picked shapes do not name. Sizes stay small enough for the oracle to
finish each case in about a second. The bar is the same as everywhere:
bit-exact layout, rows, codes and sums, identical error words."""
import sys

import numpy as np
import pytest
import torch

import combine_topk_ids_02_amd as moe
import pins
import synth
from gpu_path import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

ROW_BUDGET = 48 << 20  # bytes of expert rows per case (canary copies on both sides)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests must run on an MI355X")
    moe.lib()


def draw(seed: int, mx: bool = False) -> dict:
    """One random case; mx: H a multiple of 512 (the MX row quantum)."""
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32, 64]))
    E = R * int(rng.integers(1, 1024 // R + 1))
    k = int(rng.integers(1, min(16, E) + 1))
    T = int(rng.choice([0, 1, 255, 256, 257, 511, 513, 1024, 1025,
                        int(rng.integers(2, 256)), int(rng.integers(256, 6000))]))
    H = 512 * int(rng.integers(1, 5)) if mx else 8 * int(rng.integers(1, 257))
    kind = str(rng.choice(["plain", "plain", "align", "block"]))
    align = int(rng.choice([2, 16, 128])) if kind == "align" else 1
    block = int(rng.integers(1, 3 * max(1, T * k // E) + 2)) if kind == "block" else 0
    shape = moe.Shape(T, H, E, R, k, align, block)
    while shape.cap_expert * H * 2 > ROW_BUDGET and H > (512 if mx else 8):
        H = H // 2 // (512 if mx else 8) * (512 if mx else 8) or (512 if mx else 8)
        shape = moe.Shape(T, H, E, R, k, align, block)
    if shape.cap_expert * H * 2 > ROW_BUDGET:  # still too large: no padding
        align, block = 1, 0
    p_neg = float(rng.choice([0.0, 0.05, 0.3]))
    p_dup = float(rng.choice([0.0, 0.0, 0.1])) if k > 1 else 0.0
    p_bad = float(rng.choice([0.0, 0.0, 0.0, 0.02]))
    form = int(rng.choice([-1, 0, 1]))
    match = int(rng.choice([0, 1, 1]))  # 0: the layout matches equal experts with ballots only
    return dict(seed=seed, T=T, H=H, E=E, R=R, k=k, align=align, block=block, p_neg=p_neg,
                p_dup=p_dup, p_bad=p_bad, form=form, match=match)


def inputs(c: dict):
    rng = np.random.default_rng(9000 + c["seed"])
    ids = pins.rand_ids(rng, c["T"], c["E"], c["k"], p_neg=c["p_neg"], p_dup=c["p_dup"],
                        p_bad=c["p_bad"])
    wts = rng.random((c["T"], c["k"])).astype(np.float32)
    hid = synth.normal_bf16(c["seed"], 0, c["T"] * c["H"]).reshape(c["T"], c["H"])
    return ids, wts, hid


class layout_form:
    """Forces the layout form (-1: chosen by size) and its way of matching
    equal experts (1: LDS tables where they fit, 0: ballots) for the duration."""

    def __init__(self, form: int, match: int = 1):
        self.form = form
        self.match = match

    def __enter__(self):
        self.old = moe.lib().moe_testing_set_layout_form(self.form)
        self.old_match = moe.lib().moe_testing_set_layout_match(self.match)

    def __exit__(self, *exc):
        moe.lib().moe_testing_set_layout_form(self.old)
        moe.lib().moe_testing_set_layout_match(self.old_match)


CASES = [draw(s) for s in range(192)]


@pytest.mark.parametrize("c", CASES, ids=[f"s{c['seed']}" for c in CASES])
def test_random_shape_one_stage(c):
    say(f"[random] {c}")
    ids, wts, hid = inputs(c)
    y = synth.expert_out_slots(c["seed"], c["E"], c["H"], ids)
    with layout_form(c["form"], c["match"]):
        gpu = run_gpu(hid, ids, wts, c["E"], c["R"], y, align=c["align"], block=c["block"])
    ref = run_oracle(hid, ids, wts, c["E"], c["R"], y, gpu["cap_rank"], gpu["cap_expert"],
                     align=c["align"], block=c["block"])
    compare(gpu, ref, f"random {c}")


@pytest.mark.parametrize("c", CASES, ids=[f"s{c['seed']}" for c in CASES])
def test_random_shape_dispatch(c):
    """The same cases with layout, pack and permute through the one call
    moe_dispatch (one launch up to 256 tokens, else the layout and one
    pack-and-permute kernel)."""
    say(f"[random moe_dispatch] {c}")
    ids, wts, hid = inputs(c)
    y = synth.expert_out_slots(c["seed"], c["E"], c["H"], ids)
    with layout_form(c["form"], c["match"]):
        gpu = run_gpu(hid, ids, wts, c["E"], c["R"], y, align=c["align"], block=c["block"],
                      whole_dispatch=True)
    ref = run_oracle(hid, ids, wts, c["E"], c["R"], y, gpu["cap_rank"], gpu["cap_expert"],
                     align=c["align"], block=c["block"])
    compare(gpu, ref, f"random moe_dispatch {c}")


TWO_STAGE = [c for c in CASES if c["align"] == 1 and c["block"] == 0][:48]


@pytest.mark.parametrize("c", TWO_STAGE, ids=[f"s{c['seed']}" for c in TWO_STAGE])
def test_random_shape_two_stage(c):
    from test_two_stage_gpu import check
    say(f"[random two-stage] {c}")
    ids, wts, hid = inputs(c)
    y = synth.expert_out_slots(c["seed"], c["E"], c["H"], ids)
    with layout_form(c["form"], c["match"]):
        check(hid, ids, wts, c["E"], c["R"], y, f"random two-stage {c}")


MX_CASES = [draw(200 + s, mx=True) for s in range(24)]


@pytest.mark.parametrize("c", MX_CASES, ids=[f"s{c['seed']}" for c in MX_CASES])
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_random_shape_mx(c, fmt):
    from test_mx_dispatch_gpu import check
    say(f"[random {fmt}] {c}")
    ids, _, hid = inputs(c)
    with layout_form(c["form"], c["match"]):
        check(hid, ids, c["E"], c["R"], f"random {fmt} {c}", fmt=fmt, align=c["align"],
              block=c["block"])


@pytest.mark.parametrize("c", MX_CASES, ids=[f"s{c['seed']}" for c in MX_CASES])
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_random_shape_mx_dispatch(c, fmt):
    """The same cases through the one call moe_dispatch_quantised."""
    from test_mx_dispatch_gpu import check
    say(f"[random {fmt} moe_dispatch_quantised] {c}")
    ids, _, hid = inputs(c)
    with layout_form(c["form"], c["match"]):
        check(hid, ids, c["E"], c["R"], f"random {fmt} one call {c}", fmt=fmt,
              align=c["align"], block=c["block"], whole_dispatch=True)
