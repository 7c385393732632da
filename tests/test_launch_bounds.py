"""Every global load and store of every kernel launch stays inside the buffer
it addresses, checked on the CPU with the host-side launch model
(tests/launch_model.py), no GPU involved:

* with the oracle's layout for the whole-path random shapes (the seeds the
  GPU tests run, and further seeds that the GPU tests do not run), the
  workloads, the edge shapes, the MX dispatch and the two-stage combine;
* with index arrays of arbitrary contents (slots, pair rows, offsets, counts
  and source tokens, the values the later calls take from the caller), for
  which the C ABI still promises that nothing is written out of bounds;
* the layout's LDS regions fit their allocation for every shape the library
  accepts at the region sizes' extremes.

Two earlier forms of the permute are replayed to show the model finds what
they did: the load of rank_src_token[i] before i was checked, and padding
marks that trusted the counts and offsets to keep their rows in the buffer.
"""
import numpy as np
import pytest

import launch_model as lm
import pins
import synth
import test_random_shapes_gpu as rs

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def case_of(c: dict, plain: bool = False) -> lm.Case:
    return lm.Case(c["T"], c["H"], c["E"], c["R"], c["k"], 1 if plain else c["align"],
                   0 if plain else c["block"], c["form"], c["match"])


def assert_clean(rep: lm.Report, what: str):
    assert not rep.violations, f"{what}: {rep.violations[:4]}"


@pytest.mark.parametrize("lo,hi", [(0, 192), (1000, 1100), (1100, 1400)])
def test_whole_path_random_shapes(lo, hi):
    """The whole-path random-shape generator of the GPU tests: seeds 0-191 (run
    on the GPU) and 1000-1399 (not run there), one- and two-stage."""
    for s in range(lo, hi):
        c = rs.draw(s)
        ids, _, _ = rs.inputs(c)
        assert_clean(lm.one_stage(case_of(c), ids), f"seed {s} one-stage")
        if c["align"] == 1 and c["block"] == 0:
            assert_clean(lm.two_stage(case_of(c), ids), f"seed {s} two-stage")


QFORMATS = {"mxfp8": (8, False), "mxfp4": (4, False), "nvfp4": (4, True)}


@pytest.mark.parametrize("fmt", list(QFORMATS))
def test_mx_random_shapes(fmt):
    bits, e4m3 = QFORMATS[fmt]
    for s in list(range(200, 224)) + list(range(10000, 10060)):
        c = rs.draw(s, mx=True)
        ids, _, _ = rs.inputs(c)
        assert_clean(lm.mx(case_of(c), ids, bits, e4m3=e4m3), f"{fmt} seed {s}")


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew", "adv"])
def test_workloads(name):
    w = synth.WORKLOADS[name]
    ids, _ = synth.routing(w)
    for form in (-1, 0, 1):
        c = lm.Case(w.T, w.H, w.E, w.R, w.k, form=form)
        assert_clean(lm.one_stage(c, ids), f"{name} form {form}")
    assert_clean(lm.two_stage(lm.Case(w.T, w.H, w.E, w.R, w.k), ids), f"{name} two-stage")
    if w.H % 512 == 0:
        for fmt, (bits, e4m3) in QFORMATS.items():
            assert_clean(lm.mx(lm.Case(w.T, w.H, w.E, w.R, w.k), ids, bits, e4m3=e4m3),
                         f"{name} {fmt}")


def test_undersized_caps():
    """Caps below the worst case (rows dropped and flagged, never written past)."""
    rng = np.random.default_rng(5)
    for T, H, E, R, k in [(300, 64, 16, 4, 3), (1100, 520, 64, 8, 6), (257, 8, 8, 8, 8)]:
        ids = pins.rand_ids(rng, T, E, k, p_neg=0.1)
        for cr, ce in [(0, 0), (1, 1), (T // 3, T * k // 2), (T * min(k, R) - 1, T * k - 1)]:
            c = lm.Case(T, H, E, R, k, cap_rank=cr, cap_expert=ce)
            assert_clean(lm.one_stage(c, ids), f"T={T} caps {cr}/{ce}")
            assert_clean(lm.two_stage(c, ids), f"T={T} caps {cr}/{ce} two-stage")


def test_arbitrary_index_arrays():
    """Whatever the slots, pair rows, offsets, counts and source tokens hold,
    no kernel addresses outside its buffers."""
    rng = np.random.default_rng(11)
    for s in range(150):
        c = rs.draw(3000 + s)
        ids, _, _ = rs.inputs(c)
        case = case_of(c)
        lay, src = lm.arbitrary_layout(rng, case)
        assert_clean(lm.one_stage(case, ids, lay=lay, rank_src=src), f"seed {3000 + s}")
        plain = case_of(c, plain=True)
        lay, src = lm.arbitrary_layout(rng, plain)
        assert_clean(lm.two_stage(plain, ids, lay=lay, rank_src=src), f"seed {3000 + s} 2-st")
    for s in range(40):
        c = rs.draw(12000 + s, mx=True)
        ids, _, _ = rs.inputs(c)
        case = case_of(c)
        lay, src = lm.arbitrary_layout(rng, case)
        for fmt, (bits, e4m3) in QFORMATS.items():
            assert_clean(lm.mx(case, ids, bits, lay=lay, rank_src=src, e4m3=e4m3),
                         f"{fmt} seed {12000 + s}")


def small_batch(s: int):
    """A random decode-sized case for moe_dispatch's one-launch form."""
    rng = np.random.default_rng(20000 + s)
    R = int(rng.choice([1, 2, 4, 8, 16, 33, 64]))
    E = R * int(rng.integers(1, 1024 // R + 1))
    k = int(rng.integers(1, min(16, E) + 1))
    T = int(rng.choice([0, 1, 2, 63, 64, int(rng.integers(3, 63)), 65, 256,
                        int(rng.integers(65, 257))]))
    H = 8 * int(rng.integers(1, 1025))
    block = int(rng.choice([0, 0, 1, int(rng.integers(1, 8))]))
    align = int(rng.choice([1, 1, 2, 16, 128])) if block == 0 else 1
    ids = pins.rand_ids(rng, T, E, k, p_neg=0.1, p_dup=0.1 if k > 1 else 0.0, p_bad=0.02)
    return lm.Case(T, H, E, R, k, align, block), ids, rng


def test_dispatch_one_launch():
    """moe_dispatch's one-launch form (T <= 256; plain, padded or blocked
    runs), full and undersized caps."""
    for s in range(300):
        c, ids, rng = small_batch(s)
        assert_clean(lm.dispatch_one_launch(c, ids), f"small batch {s}")
        cr = int(rng.integers(0, c.cap_rank + 1))
        ce = int(rng.integers(0, c.cap_expert + 1))
        c2 = lm.Case(c.T, c.H, c.E, c.R, c.k, c.align, c.block, cap_rank=cr, cap_expert=ce)
        assert_clean(lm.dispatch_one_launch(c2, ids), f"small batch {s} caps {cr}/{ce}")


def test_dispatch_quantised_one_launch():
    """moe_dispatch_quantised's one-launch form: codes and scale words of the
    MX formats (4 vec4 per scale block) and the 16-value rows (2), full and
    undersized caps, H a multiple of 512."""
    for s in range(150):
        c, ids, rng = small_batch(s)
        H = 512 * int(rng.integers(1, 21))
        for lpb in (4, 2):
            c1 = lm.Case(c.T, H, c.E, c.R, c.k, c.align, c.block)
            assert_clean(lm.dispatch_one_launch(c1, ids, lpb), f"q small batch {s} lpb {lpb}")
            cr = int(rng.integers(0, c1.cap_rank + 1))
            ce = int(rng.integers(0, c1.cap_expert + 1))
            c2 = lm.Case(c.T, H, c.E, c.R, c.k, c.align, c.block, cap_rank=cr, cap_expert=ce)
            assert_clean(lm.dispatch_one_launch(c2, ids, lpb),
                         f"q small batch {s} lpb {lpb} caps {cr}/{ce}")


@pytest.mark.parametrize("vec", [1, 2, 16])
def test_dispatch_pack_expand(vec, monkeypatch):
    """moe_dispatch past the one-launch form (layout, then pack and permute in
    one kernel): the whole-path random shapes (seeds run on the GPU and
    beyond), the workloads, undersized caps and arbitrary index arrays, for
    the kernel's vec4 per lane and two other widths."""
    monkeypatch.setattr(lm, "EXPAND_VEC", vec)
    rng = np.random.default_rng(13)
    for s in list(range(0, 96)) + list(range(1000, 1100)):
        c = rs.draw(s)
        ids, _, _ = rs.inputs(c)
        case = case_of(c)
        assert_clean(lm.dispatch_rows(case, ids), f"seed {s}")
        lay, _ = lm.arbitrary_layout(rng, case)
        assert_clean(lm.dispatch_rows(case, ids, lay=lay), f"seed {s} arbitrary")
        cr = int(rng.integers(0, case.cap_rank + 1))
        ce = int(rng.integers(0, case.cap_expert + 1))
        c2 = lm.Case(case.T, case.H, case.E, case.R, case.k, case.align, case.block,
                     cap_rank=cr, cap_expert=ce)
        assert_clean(lm.dispatch_rows(c2, ids), f"seed {s} caps {cr}/{ce}")
    for name in ("prefill", "skew", "adv"):
        w = synth.WORKLOADS[name]
        ids, _ = synth.routing(w)
        assert_clean(lm.dispatch_rows(lm.Case(w.T, w.H, w.E, w.R, w.k), ids), name)


def test_dispatch_quantised_pack_expand():
    """moe_dispatch_quantised past the one-launch form: codes and scale words
    of pack_expand_q for the MX formats (4 vec4 per block) and the 16-value
    rows (2), on the MX random shapes, arbitrary index arrays and undersized
    caps."""
    rng = np.random.default_rng(17)
    for s in list(range(200, 224)) + list(range(10000, 10060)):
        c = rs.draw(s, mx=True)
        ids, _, _ = rs.inputs(c)
        case = case_of(c)
        for lpb in (4, 2):
            assert_clean(lm.dispatch_rows(case, ids, lpb=lpb), f"seed {s} lpb {lpb}")
            lay, _ = lm.arbitrary_layout(rng, case)
            assert_clean(lm.dispatch_rows(case, ids, lay=lay, lpb=lpb), f"seed {s} arbitrary")
            c2 = lm.Case(case.T, case.H, case.E, case.R, case.k, case.align, case.block,
                         cap_rank=int(rng.integers(0, case.cap_rank + 1)),
                         cap_expert=int(rng.integers(0, case.cap_expert + 1)))
            assert_clean(lm.dispatch_rows(c2, ids, lpb=lpb), f"seed {s} caps")


def test_model_finds_the_earlier_permute_reads():
    """The unclamped source-token load of an earlier permute reads past
    cap_rank for a grid rounded up past the last row; the model says so."""
    hits = 0
    for s in range(1000, 1040):
        c = rs.draw(s)
        ids, _, _ = rs.inputs(c)
        rep = lm.one_stage(case_of(c), ids, unclamped_src=True)
        hits += any("rank_src_token" in v for v in rep.violations)
    assert hits >= 5


def test_model_finds_unclipped_padding_marks():
    """Padding marks that take their first row from the caller's offsets and
    counts unclipped store below the buffer when those disagree; clipped, they
    do not (masked and padded layouts, arbitrary counts and offsets)."""
    rng = np.random.default_rng(3)
    found = 0
    for s in range(400):
        c = rs.draw(5000 + s)
        if c["align"] == 1 and c["block"] == 0 or c["T"] == 0:
            continue
        ids, _, _ = rs.inputs(c)
        case = case_of(c)
        lay, src = lm.arbitrary_layout(rng, case)
        old = lm.one_stage(case, ids, lay=lay, rank_src=src, old_padding=True)
        found += any("expert_src_pair" in v for v in old.violations)
        assert_clean(lm.one_stage(case, ids, lay=lay, rank_src=src), f"seed {5000 + s}")
    assert found >= 10


def test_layout_lds_regions():
    """The layout's LDS regions fit (largest index in each, and each region in
    the allocation) at the extremes of every dimension the library accepts."""
    for E in (1, 2, 255, 256, 257, 511, 512, 960, 1023, 1024):
        for R in (1, 2, 3, 8, 32, 64):
            if E % R:
                continue
            for k in (1, 2, 6, 8, 15, 16):
                if k > E or pins_lds_too_big(k, E + R):
                    continue
                for match in (0, 1):
                    c = lm.Case(4096, 8, E, R, k, match=match)
                    assert not lm.layout_lds_regions(c), (E, R, k, match)


def pins_lds_too_big(k, ncols):
    """Shapes the library refuses (its LDS would not fit)."""
    return lm.layout_lds_bytes(k, ncols) > lm.LDS_LIMIT
