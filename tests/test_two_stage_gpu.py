"""GPU parity of the two-stage combine (per-rank bf16 partial rows, then the
home sum over ranks) against the oracle, through the C ABI. The bar is the
same as for the one-stage combine: partial rows and outputs bit-exact in bf16
and in float32 (both sides take the same fused multiply-adds and additions in
the same order); the float32 result is also checked against the exact sum
within the bound that the bf16 partial rows allow."""
import sys

import numpy as np
import pytest
import torch

import oracle
import pins
import synth
from gpu_path import compare_two_stage, run_gpu_two_stage, run_oracle_two_stage
from test_parity_gpu import EDGE

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests must run on an MI355X")
    import combine_topk_ids_02_amd as moe
    moe.lib()


def check(hid, ids, wts, E, R, y, what, cap_rank=None, cap_expert=None, spare_rows=4):
    gpu = run_gpu_two_stage(hid, ids, wts, E, R, y, cap_rank, cap_expert, spare_rows)
    ref = run_oracle_two_stage(hid, ids, wts, E, R, y, gpu["cap_rank"], gpu["cap_expert"])
    compare_two_stage(gpu, ref, what)
    return gpu, ref


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "adv"])
def test_two_stage_workload_parity(name):
    w = synth.WORKLOADS[name]
    say(f"[two-stage] {w.describe()}")
    hid = synth.hidden(w)
    ids, wts = synth.routing(w)
    y = synth.expert_out_slots(w.seed, w.E, w.H, ids)
    gpu, ref = check(hid, ids, wts, w.E, w.R, y, name)
    assert ref["err"] == 0
    if name in ("tiny", "decode"):
        # against the exact sum: a fused chain per rank, one bf16 rounding of each
        # partial row (2^-8 relative), a chain of float32 adds over the ranks
        exact, _ = oracle.combine_f64(ref["expert_out"], ref["layout"]["pair_row"], wts)
        mag, _ = oracle.combine_f64(ref["expert_out"] & np.uint16(0x7FFF),
                                    ref["layout"]["pair_row"], np.abs(wts))
        bound = ((w.k + w.R) * 2.0 ** -24 + 2.0 ** -8) * 1.01 * mag
        assert np.all(np.abs(gpu["out_f32"].astype(np.float64) - exact) <= bound)


@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}_H{c[1]}_E{c[2]}_R{c[3]}_k{c[4]}" for c in EDGE])
def test_two_stage_edge_shapes(case):
    T, H, E, R, k, pn, pd, seed = case
    say(f"[two-stage edge] T={T} H={H} E={E} R={R} k={k}")
    rng = np.random.default_rng(seed)
    ids = pins.rand_ids(rng, T, E, k, p_neg=pn, p_dup=pd)
    wts = rng.standard_normal((T, k)).astype(np.float32)
    hid = synth.normal_bf16(seed, 0, T * H).reshape(T, H)
    y = synth.expert_out_slots(seed, E, H, ids)
    check(hid, ids, wts, E, R, y, f"edge {case}")


def test_two_stage_bad_ids_and_undersized_buffers():
    T, H, E, R, k = 600, 256, 32, 4, 4
    rng = np.random.default_rng(24)
    ids = pins.rand_ids(rng, T, E, k, p_neg=0.1, p_bad=0.05)
    wts = rng.random((T, k)).astype(np.float32)
    hid = synth.normal_bf16(24, 0, T * H).reshape(T, H)
    y = synth.expert_out_slots(24, E, H, ids)
    _, ref = check(hid, ids, wts, E, R, y, "bad ids")
    assert ref["err"] == 1
    C = int(ref["layout"]["rank_offsets"][-1])
    P = int(ref["layout"]["expert_offsets"][-1])
    _, ref2 = check(hid, ids, wts, E, R, y, "undersized", cap_rank=C - 29, cap_expert=P - 41,
                    spare_rows=64)
    assert ref2["err"] == 1 | 2 | 4
