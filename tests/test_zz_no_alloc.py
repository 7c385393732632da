"""The allocation-free layout (moe_dispatch_layout_noalloc, its workspace the
library's static device array) against the layout with a caller workspace
(moe_dispatch_layout), through the C ABI: every count, offset, slot and pair
row and the error word identical, on calls in a row on the same GPU, each
later one smaller than the one before (the static array then still holds the
previous call's tile counts, which must not matter), in both forms (two
launches through the array; one launch), padded and masked runs included."""
import sys

import numpy as np
import pytest
import torch

import combine_topk_ids_02_amd as moe
import pins

pytestmark = pytest.mark.gpu

KEYS = ("rank_counts", "rank_offsets", "expert_counts", "expert_offsets", "token_rank_slot",
        "pair_row")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests must run on an MI355X")
    moe.lib()


def outputs(T, E, R, k, dev):
    i32 = torch.int32
    return dict(rank_counts=torch.full((R,), -9, dtype=i32, device=dev),
                rank_offsets=torch.full((R + 1,), -9, dtype=i32, device=dev),
                expert_counts=torch.full((E,), -9, dtype=i32, device=dev),
                expert_offsets=torch.full((E + 1,), -9, dtype=i32, device=dev),
                token_rank_slot=torch.full((T, R), -9, dtype=i32, device=dev),
                pair_row=torch.full((T, k), -9, dtype=i32, device=dev))


# (T, E, R, k, align, block, p_neg, p_bad): calls in this order, each smaller
SEQUENCES = [
    [(20000, 1024, 64, 8, 1, 0, 0.05, 0.01), (7000, 256, 8, 8, 1, 0, 0.0, 0.0),
     (300, 384, 8, 6, 1, 0, 0.0, 0.0)],
    [(16385, 384, 8, 6, 128, 0, 0.1, 0.0), (12000, 64, 4, 5, 1, 40, 0.0, 0.02),
     (64, 384, 8, 6, 1, 0, 0.0, 0.0)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_layout_matches_the_caller_workspace_layout(seq):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(77 + seq)
    for call, (T, E, R, k, align, block, p_neg, p_bad) in enumerate(SEQUENCES[seq]):
        say(f"[no-alloc layout] sequence {seq} call {call}: T={T} E={E} R={R} k={k} "
            f"align={align} block={block}")
        ids = pins.rand_ids(rng, T, E, k, p_neg=p_neg, p_bad=p_bad)
        ids_d = torch.from_numpy(ids).to(dev)
        shape = moe.Shape(T, 8, E, R, k, align, block)
        ws = moe.layout_workspace_bytes(shape)
        workspace = torch.full(((ws + 15) // 16 * 4,), 0x5A5A5A5A, dtype=torch.int32,
                               device=dev) if ws else None
        err_a = torch.zeros(1, dtype=torch.int32, device=dev)
        err_b = torch.zeros(1, dtype=torch.int32, device=dev)
        want = moe.layout(ids_d, E, R, 8, align=align, block=block, err=err_a,
                          out=outputs(T, E, R, k, dev), workspace=workspace)
        got = moe.layout_noalloc(ids_d, E, R, 8, align=align, block=block, err=err_b,
                                 out=outputs(T, E, R, k, dev))
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], want[key]), f"call {call}: {key} differs"
        assert int(err_b.item()) == int(err_a.item()), f"call {call}: error word differs"
