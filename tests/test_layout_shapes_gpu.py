"""GPU parity of the padded and masked expert layouts (runs padded to a
multiple of `align` rows; fixed blocks of `block` rows per expert) against the
oracle, through the C ABI: layout, pack, permute (with its padding marks) and
combine, bit for bit. The row buffers carry canary rows and indices so that
writes outside what the oracle writes are seen."""
import sys

import numpy as np
import pytest
import torch

import pins
import synth
from gpu_path import compare, run_gpu, run_oracle

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


def check(hid, ids, wts, E, R, y, what, align=1, block=0, **kw):
    gpu = run_gpu(hid, ids, wts, E, R, y, align=align, block=block, **kw)
    ref = run_oracle(hid, ids, wts, E, R, y, gpu["cap_rank"], gpu["cap_expert"], align=align,
                     block=block)
    compare(gpu, ref, what)
    return gpu, ref


WORKLOAD_SHAPES = [("prefill", 128, 0), ("skew", 128, 0), ("decode", 1, 128), ("tiny", 1, 64),
                   ("adv", 128, 0)]


@pytest.mark.parametrize("name,align,block", WORKLOAD_SHAPES,
                         ids=[f"{n}_align{a}_block{b}" for n, a, b in WORKLOAD_SHAPES])
def test_workload_layout_shapes(name, align, block):
    w = synth.WORKLOADS[name]
    say(f"[shapes] {w.describe()} align={align} block={block}")
    hid = synth.hidden(w)
    ids, wts = synth.routing(w)
    y = synth.expert_out_slots(w.seed, w.E, w.H, ids)
    _, ref = check(hid, ids, wts, w.E, w.R, y, name, align=align, block=block)
    assert ref["err"] == 0
    offs = ref["layout"]["expert_offsets"]
    if block:
        assert np.array_equal(offs, np.arange(w.E + 1) * block)
    else:
        assert np.all(offs % align == 0)


EDGE_SHAPES = [
    # (T, H, E, R, k, p_neg, p_dup, seed, align, block)
    (0, 512, 16, 4, 2, 0.0, 0.0, 31, 128, 0),
    (0, 512, 16, 4, 2, 0.0, 0.0, 32, 1, 16),
    (1, 8, 2, 1, 1, 0.0, 0.0, 33, 2, 0),
    (257, 512, 16, 4, 2, 0.1, 0.0, 34, 3, 0),
    (1000, 1024, 64, 8, 4, 0.05, 0.1, 35, 128, 0),
    (2000, 64, 1024, 64, 16, 0.02, 0.02, 36, 128, 0),     # largest E, R, k
    (70000, 16, 64, 8, 5, 0.05, 0.0, 37, 64, 0),          # several sub-tiles per workgroup
    (300, 520, 32, 4, 4, 0.0, 0.0, 38, 1, 1),             # one row per expert block
    (3000, 64, 64, 8, 6, 0.0, 0.0, 39, 1, 200),           # blocks overflow (about 281 per expert)
    (513, 2880, 384, 8, 6, 0.0, 0.0, 40, 1, 16),          # blocks overflow, tail columns
    (700, 256, 96, 1, 5, 0.1, 0.0, 41, 7, 0),             # one rank
]


@pytest.mark.parametrize("case", EDGE_SHAPES,
                         ids=[f"T{c[0]}_E{c[2]}_R{c[3]}_k{c[4]}_a{c[8]}_b{c[9]}" for c in EDGE_SHAPES])
def test_edge_layout_shapes(case):
    T, H, E, R, k, pn, pd, seed, align, block = case
    say(f"[shapes edge] T={T} H={H} E={E} R={R} k={k} align={align} block={block}")
    rng = np.random.default_rng(seed)
    ids = pins.rand_ids(rng, T, E, k, p_neg=pn, p_dup=pd)
    wts = rng.random((T, k)).astype(np.float32)
    hid = synth.normal_bf16(seed, 0, T * H).reshape(T, H)
    y = synth.expert_out_slots(seed, E, H, ids)
    _, ref = check(hid, ids, wts, E, R, y, f"shapes {case}", align=align, block=block)
    if block and T and int(ref["layout"]["expert_counts"].max()) > block:
        assert ref["err"] & 4


def test_masked_layout_with_undersized_buffers():
    """Blocks of 8 rows, a rank buffer 37 rows short and an expert buffer that
    stops in the middle of a block."""
    w = synth.WORKLOADS["tiny"]
    hid = synth.hidden(w)
    ids, wts = synth.routing(w)
    y = synth.expert_out_slots(w.seed, w.E, w.H, ids)
    lay = run_oracle(hid, ids, wts, w.E, w.R, None, w.T * 2, w.T * 2, block=8)["layout"]
    C = int(lay["rank_offsets"][-1])
    _, ref = check(hid, ids, wts, w.E, w.R, y, "masked undersized", block=8, cap_rank=C - 37,
                   cap_expert=w.E * 8 - 13, spare_rows=64)
    assert ref["err"] == 2 | 4
