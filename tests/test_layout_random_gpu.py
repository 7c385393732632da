"""Seeded random shapes through the layout alone, against the oracle, many more
than the whole-path random shapes can afford: T from 0 to 20,000 (tile edges
and both sides of the one-launch / two-launch crossover), R from 1 to 64, E up
to 1024, k up to 16, -1 / duplicate / out-of-range ids, padded and masked
expert layouts, a hot expert in slot 0 of most tokens in a quarter of the
cases, and the layout form and the match of equal experts forced at random.
Bar: every count, offset, slot and pair row bit-exact, identical error words."""
import sys

import numpy as np
import pytest
import torch

import combine_topk_ids_02_amd as moe
import oracle
import pins

pytestmark = pytest.mark.gpu

N_CASES = 400
LAYOUT_KEYS = ("rank_counts", "rank_offsets", "expert_counts", "expert_offsets",
               "token_rank_slot", "pair_row")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests must run on an MI355X")
    moe.lib()


def draw(seed: int) -> dict:
    rng = np.random.default_rng(50000 + seed)
    R = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32, 64]))
    E = R * int(rng.integers(1, 1024 // R + 1))
    k = int(rng.integers(1, min(16, E) + 1))
    T = int(rng.choice([0, 1, 63, 64, 65, 255, 256, 257, 1023, 4096, 4097, 16383, 16384, 16385,
                        int(rng.integers(2, 512)), int(rng.integers(512, 20000))]))
    kind = str(rng.choice(["plain", "plain", "align", "block"]))
    align = int(rng.choice([2, 16, 128])) if kind == "align" else 1
    block = int(rng.integers(1, 3 * max(1, T * k // E) + 2)) if kind == "block" else 0
    p_neg = float(rng.choice([0.0, 0.05, 0.3]))
    p_dup = float(rng.choice([0.0, 0.0, 0.1])) if k > 1 else 0.0
    p_bad = float(rng.choice([0.0, 0.0, 0.0, 0.02]))
    hot = bool(rng.random() < 0.25)
    form = int(rng.choice([-1, 0, 1]))
    match = int(rng.choice([0, 1]))
    ids = pins.rand_ids(rng, T, E, k, p_neg=p_neg, p_dup=p_dup, p_bad=p_bad)
    if hot and T > 0:  # one expert in slot 0 of about 90% of the tokens
        h = int(rng.integers(0, E))
        ids[rng.random(T) < 0.9, 0] = h
    return dict(seed=seed, T=T, E=E, R=R, k=k, align=align, block=block, form=form,
                match=match, hot=hot, ids=ids)


@pytest.mark.parametrize("chunk", range(8), ids=[f"cases{c * N_CASES // 8}" for c in range(8)])
def test_layout_random_shapes(chunk):
    dev = torch.device("cuda:0")
    L = moe.lib()
    for seed in range(chunk * N_CASES // 8, (chunk + 1) * N_CASES // 8):
        c = draw(seed)
        T, E, R, k, ids = c["T"], c["E"], c["R"], c["k"], c["ids"]
        tag = {key: c[key] for key in ("seed", "T", "E", "R", "k", "align", "block", "form",
                                       "match", "hot")}
        shape = moe.Shape(T, 8, E, R, k, c["align"], c["block"])
        ws = moe.layout_workspace_bytes(shape)
        workspace = torch.zeros(((ws + 15) // 16 * 4,), dtype=torch.int32, device=dev) \
            if ws else None
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev) if T else \
            torch.zeros((0, k), dtype=torch.int32, device=dev)
        old_form = L.moe_testing_set_layout_form(c["form"])
        old_match = L.moe_testing_set_layout_match(c["match"])
        try:
            got = moe.layout(ids_d, E, R, 8, align=c["align"], block=c["block"], err=err,
                             workspace=workspace)
            torch.cuda.synchronize()
        finally:
            L.moe_testing_set_layout_form(old_form)
            L.moe_testing_set_layout_match(old_match)
        ref = oracle.layout(ids, E, R, align=c["align"], block=c["block"])
        for key in LAYOUT_KEYS:
            assert np.array_equal(got[key].cpu().numpy().reshape(ref[key].shape), ref[key]), \
                f"{tag}: {key} differs"
        assert int(err.item()) == int(ref["err"]), \
            f"{tag}: error word {int(err.item())}, oracle {int(ref['err'])}"
    say(f"[layout random] cases {chunk * N_CASES // 8}..{(chunk + 1) * N_CASES // 8 - 1} ok")
