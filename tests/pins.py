"""Pins that tie the oracle to something other than itself.

Each pin is a plain function that raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix:
  * library routines the definition reduces to (stable sort, bincount, cumsum),
  * brute force on tiny inputs,
  * the closed-form copy count of the "A2A backends" page, section 1.3, exact
    over every k-subset and statistically over the seeded workloads,
  * prose examples of that page (sections 1.1, 3.3 and 4.1, constructed
    instances under tests/golden/),
  * combine special cases (identity experts, one-hot weights, k = 1, exact
    doubling, round-to-nearest-even ties) and the exact rational result within
    the standard error bound of a fused multiply-add chain.

The pins are collected by test_oracle_pins.py and replayed against
deliberately broken copies of the oracle by test_oracle_mutants.py.
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24  # unit roundoff of float32


# ----------------------------------------------------------------------------
# helpers (test side; none of them is the oracle's arithmetic)

def bf16_bits_to_float(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def closed_form_copies(E: int, R: int, k: int) -> Fraction:
    """Expected distinct ranks per token, uniform router ("A2A backends" page,
    section 1.3): R * (1 - C(E - E/R, k) / C(E, k)), as an exact fraction."""
    return R * (1 - Fraction(math.comb(E - E // R, k), math.comb(E, k)))


def rand_ids(rng, T, E, k, p_neg=0.0, p_dup=0.0, p_bad=0.0):
    """Random top-k ids: distinct experts per token, then some slots set to -1,
    some duplicated from slot 0, some set to out-of-range ids."""
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    if T and k > 1 and p_dup:
        dup = rng.random((T, k)) < p_dup
        dup[:, 0] = False
        ids = np.where(dup, ids[:, :1], ids)
    if T and p_neg:
        ids = np.where(rng.random((T, k)) < p_neg, -1, ids)
    if T and p_bad:
        bad = rng.random((T, k)) < p_bad
        ids = np.where(bad, rng.choice([-7, -2, E, E + 5], size=(T, k)), ids)
    return np.ascontiguousarray(ids, dtype=np.int32)


def valid_mask(ids, E):
    return (ids >= 0) & (ids < E)


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def expected_layout_by_sorting(ids: np.ndarray, E: int, R: int) -> dict:
    """The layout the definition reduces to, built from library routines only:
    stable argsort by key (expert; rank), bincount and cumsum."""
    T, k = ids.shape
    m = E // R
    flat = ids.reshape(-1)
    ok = valid_mask(flat, E)
    idx = np.nonzero(ok)[0]
    order = idx[np.argsort(flat[idx], kind="stable")]
    pair_row = np.full(T * k, -1, np.int64)
    pair_row[order] = np.arange(order.size)
    expert_counts = np.bincount(flat[idx], minlength=E)

    present = np.zeros((T, R), bool)
    tt = np.repeat(np.arange(T), k)[ok]
    present[tt, flat[ok] // m] = True
    t_of, r_of = np.nonzero(present)  # row-major: ascending t, then r
    order_r = np.argsort(r_of, kind="stable")
    slot = np.full((T, R), -1, np.int64)
    slot[t_of[order_r], r_of[order_r]] = np.arange(order_r.size)
    rank_counts = present.sum(0)
    return dict(
        rank_counts=rank_counts,
        rank_offsets=np.concatenate([[0], np.cumsum(rank_counts)]),
        expert_counts=expert_counts,
        expert_offsets=np.concatenate([[0], np.cumsum(expert_counts)]),
        token_rank_slot=slot,
        pair_row=pair_row.reshape(T, k),
    )


LAYOUT_KEYS = ("rank_counts", "rank_offsets", "expert_counts", "expert_offsets",
               "token_rank_slot", "pair_row")


def assert_layout_equal(got: dict, want: dict, what: str):
    for key in LAYOUT_KEYS:
        a = np.asarray(got[key]).astype(np.int64)
        b = np.asarray(want[key]).astype(np.int64)
        assert a.shape == b.shape and np.array_equal(a, b), f"{what}: {key} differs"


# ----------------------------------------------------------------------------
# layout pins

LAYOUT_CASES = [
    # (T, E, R, k, p_neg, p_dup, seed)
    (1, 4, 2, 2, 0.0, 0.0, 1),
    (7, 8, 4, 3, 0.2, 0.0, 2),
    (64, 16, 4, 2, 0.0, 0.0, 3),
    (100, 16, 16, 4, 0.1, 0.2, 4),
    (333, 384, 8, 6, 0.05, 0.05, 5),
    (257, 256, 8, 8, 0.0, 0.1, 6),
    (50, 12, 1, 5, 0.1, 0.0, 7),
    (129, 64, 64, 1, 0.3, 0.0, 8),
]


def pin_layout_stable_sort():
    """Rows of a rank segment / expert run ascend with the token index, which
    is exactly a stable sort of the (token, rank) copies by rank and of the
    (token, slot) pairs by expert; offsets are exclusive prefix sums of the
    counts ("A2A backends" page, sections 3.2 and 5.1)."""
    for T, E, R, k, pn, pd, seed in LAYOUT_CASES:
        ids = rand_ids(np.random.default_rng(seed), T, E, k, pn, pd)
        got = oracle.layout(ids, E, R)
        assert got["err"] == 0, "no bad ids in these cases"
        assert_layout_equal(got, expected_layout_by_sorting(ids, E, R),
                            f"stable-sort T={T} E={E} R={R} k={k}")


def pin_layout_brute_force():
    """Every position counted directly from its definition, O(T^2), tiny inputs."""
    rng = np.random.default_rng(11)
    for T, E, R, k in [(1, 2, 1, 1), (3, 4, 2, 2), (5, 6, 3, 2), (8, 8, 4, 4), (8, 8, 8, 3),
                       (6, 8, 2, 4)]:
        for rep in range(3):
            ids = rand_ids(rng, T, E, k, p_neg=0.15, p_dup=0.15)
            got = oracle.layout(ids, E, R)
            m = E // R
            pairs = [(t, j, int(ids[t, j])) for t in range(T) for j in range(k)
                     if 0 <= ids[t, j] < E]
            ranks_of = [sorted({int(e) // m for e in ids[t] if 0 <= e < E}) for t in range(T)]
            for t in range(T):
                for j in range(k):
                    e = int(ids[t, j])
                    if not 0 <= e < E:
                        assert got["pair_row"][t, j] == -1
                        continue
                    before = sum(1 for (_, _, e2) in pairs if e2 < e)
                    earlier = sum(1 for (t2, j2, e2) in pairs if e2 == e and (t2, j2) < (t, j))
                    assert got["pair_row"][t, j] == before + earlier, ("pair_row", T, E, R, k, t, j)
                for r in range(R):
                    if r not in ranks_of[t]:
                        assert got["token_rank_slot"][t, r] == -1
                        continue
                    before = sum(1 for t2 in range(T) for r2 in ranks_of[t2] if r2 < r)
                    earlier = sum(1 for t2 in range(t) if r in ranks_of[t2])
                    assert got["token_rank_slot"][t, r] == before + earlier, ("slot", t, r)
            for r in range(R):
                assert got["rank_counts"][r] == sum(r in rs for rs in ranks_of)
            for e in range(E):
                assert got["expert_counts"][e] == sum(1 for p in pairs if p[2] == e)


def pin_layout_invariants():
    """Counts and positions agree with each other on the seeded workloads."""
    for name in ("tiny", "decode", "prefill", "skew"):
        w = synth.WORKLOADS[name]
        ids, _ = synth.routing(w)
        lay = oracle.layout(ids, w.E, w.R)
        assert lay["err"] == 0
        D = np.array([len({int(e) // w.m for e in row}) for row in ids])
        C = int(D.sum())
        slots = lay["token_rank_slot"]
        assert int(lay["rank_counts"].sum()) == C == int(lay["rank_offsets"][-1])
        assert np.array_equal((slots >= 0).sum(1), D), "copies per token != distinct ranks"
        assert int(lay["expert_counts"].sum()) == w.T * w.k == int(lay["expert_offsets"][-1])
        s = np.sort(slots[slots >= 0])
        assert np.array_equal(s, np.arange(C)), "slots are not a bijection onto [0, C)"
        p = np.sort(lay["pair_row"].reshape(-1))
        assert np.array_equal(p, np.arange(w.T * w.k)), "pair rows not a bijection onto [0, P)"
        for r in range(w.R):
            col = slots[:, r]
            col = col[col >= 0]
            assert np.all(np.diff(col) == 1), "rank segment rows not ascending in t"
            assert col.size == 0 or col[0] == lay["rank_offsets"][r]


def pin_closed_form_exhaustive():
    """Over every k-subset of experts (one token each), the mean number of
    copies equals the closed form of the "A2A backends" page, section 1.3,
    exactly."""
    for E, R, k in [(8, 4, 3), (12, 4, 3), (12, 3, 5), (16, 8, 2), (10, 5, 4)]:
        ids = np.array(list(itertools.combinations(range(E), k)), dtype=np.int32)
        lay = oracle.layout(ids, E, R)
        got = Fraction(int(lay["rank_counts"].sum()), ids.shape[0])
        assert got == closed_form_copies(E, R, k), (E, R, k, got)
        assert int(lay["expert_counts"].sum()) == ids.size


def pin_closed_form_workloads():
    """Seeded uniform-router workloads: mean copies within 4 sigma of the closed
    form (the page's 4.43 for 384 experts, 8 GPUs, top-6)."""
    for name in ("tiny", "decode", "prefill"):
        w = synth.WORKLOADS[name]
        ids, _ = synth.routing(w)
        lay = oracle.layout(ids, w.E, w.R)
        D = (lay["token_rank_slot"] >= 0).sum(1)
        mu = float(closed_form_copies(w.E, w.R, w.k))
        sigma = float(D.std()) / math.sqrt(w.T)
        assert abs(D.mean() - mu) <= 4 * max(sigma, 1e-9), (name, D.mean(), mu, sigma)


def pin_page_bytes():
    """Bytes per GPU per layer at the prefill workload: the oracle's copy count
    times the 10,240-byte row lands on the page's 177 MB (per distinct GPU),
    well below 240 MB (per expert) and 320 MB (every GPU)."""
    w = synth.WORKLOADS["prefill"]
    ids, _ = synth.routing(w)
    lay = oracle.layout(ids, w.E, w.R)
    row = w.H * 2
    mib_gpu = int(lay["rank_offsets"][-1]) * row / 2 ** 20
    mib_expert = int(lay["expert_offsets"][-1]) * row / 2 ** 20
    assert abs(mib_gpu - 177) < 2.5, mib_gpu
    assert mib_expert == 240.0


def pin_figure1():
    rows = {r[0]: r[1:] for r in read_golden("figure1_token.txt")}
    E, R = int(rows["E"][0]), int(rows["R"][0])
    ids = np.array([[int(x) for x in rows["ids"]]], np.int32)
    lay = oracle.layout(ids, E, R)
    assert int((lay["token_rank_slot"] >= 0).sum()) == int(rows["copies"][0])
    hid = np.arange(16, dtype=np.uint16).reshape(1, 16)
    rank_buf, _, err = oracle.pack(hid, lay["token_rank_slot"], cap_rank=3)
    assert err == 0 and int(lay["rank_offsets"][-1]) == 2


def pin_figure4():
    """Five rows arrive at rank 1 and become seven expert rows."""
    rows = read_golden("figure4_regroup.txt")
    kv = {r[0]: r[1:] for r in rows if r[0] != "token"}
    E, R, rank = int(kv["E"][0]), int(kv["R"][0]), int(kv["rank"][0])
    ids = np.array([[int(x) for x in r[2:]] for r in rows if r[0] == "token"], np.int32)
    T, k = ids.shape
    H = 8
    hid = (np.arange(T * H, dtype=np.uint16) + 1).reshape(T, H)
    lay = oracle.layout(ids, E, R)
    assert int(lay["rank_counts"][rank]) == int(kv["arrived_rows"][0])
    m = E // R
    local = range(rank * m, (rank + 1) * m)
    assert int(sum(lay["expert_counts"][e] for e in local)) == int(kv["expert_rows"][0])
    rank_buf, src, _ = oracle.pack(hid, lay["token_rank_slot"], cap_rank=T * min(k, R))
    ebuf, esrc, err = oracle.permute(rank_buf, src, lay, ids, E,
                                     cap_expert=T * k)
    assert err == 0
    lo, hi = lay["expert_offsets"][rank * m], lay["expert_offsets"][(rank + 1) * m]
    assert hi - lo == 7
    seg = slice(lay["rank_offsets"][rank], lay["rank_offsets"][rank + 1])
    assert list(src[seg]) == [0, 1, 2, 3, 4], "rows arrive in token order a..e"
    # token a needs E2 and E3: it shows up in both runs
    for e in (2, 3):
        run = esrc[lay["expert_offsets"][e]:lay["expert_offsets"][e + 1]] // k
        assert 0 in run
    for row in range(lo, hi):
        assert np.array_equal(ebuf[row], hid[esrc[row] // k])


def pin_bad_ids():
    """Out-of-range ids are reported and then treated like -1."""
    rng = np.random.default_rng(21)
    for T, E, R, k in [(40, 16, 4, 3), (90, 64, 8, 6)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1, p_bad=0.15)
        bad = (ids != -1) & ~valid_mask(ids, E)
        assert bad.any()
        got = oracle.layout(ids, E, R)
        assert got["err"] & oracle.ERR_BAD_ID
        clean = np.where(bad, -1, ids)
        ref = oracle.layout(clean, E, R)
        assert ref["err"] == 0
        assert_layout_equal(got, ref, "bad ids vs -1")


# ----------------------------------------------------------------------------
# pack / permute pins

def pin_pack_permute_rows():
    """Every packed row is its source token's row, placed where the stable sort
    puts it; every expert row is the token row of its pair; rows past the
    counts are left alone (canaries)."""
    for T, E, R, k, pn, pd, seed in LAYOUT_CASES:
        rng = np.random.default_rng(100 + seed)
        ids = rand_ids(rng, T, E, k, pn, pd)
        H = 24
        hid = rng.integers(0, 65536, size=(T, H), dtype=np.uint16)
        lay = oracle.layout(ids, E, R)
        want = expected_layout_by_sorting(ids, E, R)
        cap_rank, cap_expert = T * min(k, R) + 3, T * k + 3
        canary = np.uint16(0xBEEF)
        rb = np.full((cap_rank, H), canary, np.uint16)
        src = np.full(cap_rank, -5, np.int32)
        rb, src, e1 = oracle.pack(hid, lay["token_rank_slot"], cap_rank, rb, src)
        C = int(want["rank_offsets"][-1])
        assert e1 == 0
        t_of = np.full(C, -1)
        ts, rs = np.nonzero(want["token_rank_slot"] >= 0)
        t_of[want["token_rank_slot"][ts, rs]] = ts
        assert np.array_equal(src[:C], t_of)
        assert np.array_equal(rb[:C], hid[t_of])
        assert np.all(rb[C:] == canary) and np.all(src[C:] == -5)

        eb = np.full((cap_expert, H), canary, np.uint16)
        es = np.full(cap_expert, -5, np.int32)
        eb, es, e2 = oracle.permute(rb, src, lay, ids, E,
                                    cap_expert, eb, es)
        assert e2 == 0
        P = int(want["expert_offsets"][-1])
        pr = want["pair_row"].reshape(-1)
        pair_of = np.full(P, -1)
        ok = pr >= 0
        pair_of[pr[ok]] = np.nonzero(ok)[0]
        assert np.array_equal(es[:P], pair_of)
        assert np.array_equal(eb[:P], hid[pair_of // k])
        assert np.all(eb[P:] == canary) and np.all(es[P:] == -5)


def pin_permute_reads_own_segment():
    """The permute of a rank segment reads only the rows that arrived in that
    segment: with every rank-buffer row made distinguishable, expert row
    pair_row[t, j] holds the copy of token t from the segment of rank(e_tj)."""
    rng = np.random.default_rng(27)
    for T, E, R, k in [(60, 16, 4, 4), (128, 384, 8, 6)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1)
        lay = oracle.layout(ids, E, R)
        C = int(lay["rank_offsets"][-1])
        H = 4
        rb = np.repeat(np.arange(C, dtype=np.uint16)[:, None], H, 1)  # row i holds i
        src = np.full(C, -1, np.int32)
        ts, rs = np.nonzero(lay["token_rank_slot"] >= 0)
        src[lay["token_rank_slot"][ts, rs]] = ts
        eb, es, err = oracle.permute(rb, src, lay, ids, E,
                                     T * k)
        assert err == 0
        m = E // R
        for t in range(T):
            for j in range(k):
                e = int(ids[t, j])
                if e < 0:
                    continue
                want = lay["token_rank_slot"][t, e // m]
                assert np.all(eb[lay["pair_row"][t, j]] == want), (t, j)


def pin_caps():
    """Undersized buffers: rows past the cap are dropped, never written out of
    bounds, and reported."""
    rng = np.random.default_rng(31)
    T, E, R, k, H = 50, 16, 4, 3, 8
    ids = rand_ids(rng, T, E, k)
    hid = rng.integers(0, 65536, size=(T, H), dtype=np.uint16)
    lay = oracle.layout(ids, E, R)
    C = int(lay["rank_offsets"][-1])
    cap = C - 7
    rb = np.zeros((cap, H), np.uint16)
    src = np.full(cap, -1, np.int32)
    rb, src, err = oracle.pack(hid, lay["token_rank_slot"], cap, rb, src)
    assert err == oracle.ERR_RANK_CAP
    assert np.all(src >= 0)
    P = int(lay["expert_offsets"][-1])
    eb = np.zeros((P - 5, H), np.uint16)
    es = np.full(P - 5, -1, np.int32)
    eb, es, err2 = oracle.permute(rb, src, lay, ids, E, P - 5,
                                  eb, es)
    assert err2 & oracle.ERR_EXPERT_CAP
    out, _, err3 = oracle.combine(eb, lay["pair_row"], np.ones((T, k), np.float32))
    assert err3 & oracle.ERR_EXPERT_CAP


def _padded_expected(ids, E, R, align=1, block=0):
    """The padded or masked layout from the plain one (stable sort): every
    pair keeps its index inside its expert's run; only where runs start
    changes (numpy cumsum of the rounded-up counts, or e * block)."""
    want = expected_layout_by_sorting(ids, E, R)
    counts = want["expert_counts"]
    base = want["expert_offsets"][:-1]
    if block > 0:
        offsets = np.arange(E + 1) * block
    else:
        offsets = np.concatenate([[0], np.cumsum(-(-counts // align) * align)])
    pr = want["pair_row"]
    e = np.where(pr >= 0, ids, 0)
    idx = pr - base[e]
    new_pr = np.where(pr >= 0, offsets[e] + idx, -1)
    over = (pr >= 0) & (block > 0) & (idx >= block)
    new_pr = np.where(over, -1, new_pr)
    out = dict(want, expert_offsets=offsets, pair_row=new_pr)
    return out, bool(over.any())


def pin_layout_padded_and_masked():
    """Runs padded to a multiple of `align` rows and fixed per-expert blocks:
    against the stable-sort layout with the run starts moved (cumsum of the
    rounded-up counts, or e * block) and pairs past a full block dropped
    and reported. The worst-case padded size T*k + E*(align-1) is never
    exceeded."""
    for (T, E, R, k, pn, pd, seed) in LAYOUT_CASES:
        rng = np.random.default_rng(seed + 100)
        ids = rand_ids(rng, T, E, k, p_neg=pn, p_dup=pd)
        for align in (1, 2, 8, 128):
            got = oracle.layout(ids, E, R, align=align)
            want, _ = _padded_expected(ids, E, R, align=align)
            assert_layout_equal(got, want, f"align {align} T{T} E{E} R{R} k{k}")
            assert got["err"] == 0
            assert got["expert_offsets"][-1] <= T * k + E * (align - 1)
        for block in (1, 3, 64):
            got = oracle.layout(ids, E, R, block=block)
            want, over = _padded_expected(ids, E, R, block=block)
            assert_layout_equal(got, want, f"block {block} T{T} E{E} R{R} k{k}")
            assert got["err"] == (oracle.ERR_EXPERT_CAP if over else 0), (block, got["err"])


def pin_permute_padding_rows():
    """After the permute of a padded or masked layout, every row that a pair
    fills holds that token's hidden row with its (token, slot) id, every other
    row of a run or block is marked -1, and rows past the last run are not
    touched. The combine does not see the difference: it equals the combine
    of the plain layout bit for bit (when no block overflows)."""
    rng = np.random.default_rng(103)
    for T, E, R, k, H, align, block in [(60, 16, 4, 3, 8, 8, 0), (40, 32, 8, 4, 16, 128, 0),
                                        (50, 16, 4, 2, 8, 1, 40), (30, 8, 2, 4, 8, 1, 7)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1)
        hid = synth.normal_bf16(21, 0, T * H).reshape(T, H)
        lay = oracle.layout(ids, E, R, align=align, block=block)
        cap_rank = T * min(k, R)
        cap_expert = E * block if block else T * k + E * (align - 1)
        rb, src, _ = oracle.pack(hid, lay["token_rank_slot"], cap_rank)
        eb, es, _ = oracle.permute(rb, src, lay, ids, E, cap_expert)
        filled = np.zeros(cap_expert, bool)
        for t in range(T):
            for j in range(k):
                row = lay["pair_row"][t, j]
                if row >= 0:
                    filled[row] = True
                    assert es[row] == t * k + j and np.array_equal(eb[row], hid[t])
        offs, cnts = lay["expert_offsets"], lay["expert_counts"]
        in_run = np.zeros(cap_expert, bool)
        for e in range(E):
            end = (e + 1) * block if block else offs[e + 1]
            in_run[offs[e]:end] = True
        assert np.all(es[in_run & ~filled] == -1)
        assert np.all(es[~in_run] == -2)  # untouched
        assert not np.any(filled & ~in_run)
        if block == 0 or not (lay["err"] & oracle.ERR_EXPERT_CAP):
            y = synth.normal_bf16(23, 2, T * k * H).reshape(T, k, H)
            w = rng.random((T, k)).astype(np.float32)
            plain = oracle.layout(ids, E, R)
            a = oracle.combine(oracle.place_slots(y, plain["pair_row"], T * k), plain["pair_row"], w)
            b = oracle.combine(oracle.place_slots(y, lay["pair_row"], cap_expert), lay["pair_row"], w)
            assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])


# ----------------------------------------------------------------------------
# combine pins

def _renormalised_weights(rng, T, k):
    w = rng.random((T, k)) + 0.05
    return (w / w.sum(1, keepdims=True)).astype(np.float32)


def pin_roundtrip_identity():
    """Identity experts and renormalised weights give back the hidden state
    bit for bit (the weights sum to 1 within a few float32 ulps, far below
    half a bf16 ulp): dispatch followed by combine is the identity."""
    for name in ("tiny", "decode"):
        w = synth.WORKLOADS[name]
        hid = synth.hidden(w)
        ids, wts = synth.routing(w)
        res = oracle.dispatch_combine(hid, ids, wts, w.E, w.R)
        assert res["err"] == 0
        a, b = res["out"], hid
        zero = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
        assert np.all((a == b) | zero), f"{name}: identity round trip differs"
    rng = np.random.default_rng(41)
    T, E, R, k, H = 77, 32, 4, 5, 40
    ids = rand_ids(rng, T, E, k, p_neg=0.2)
    ids[:, 0] = rng.integers(0, E, T)  # keep one valid slot per token
    wts = np.where(ids >= 0, rng.random((T, k)) + 0.05, 0.0)
    wts = (wts / wts.sum(1, keepdims=True)).astype(np.float32)
    hid = synth.normal_bf16(5, 0, T * H).reshape(T, H)
    res = oracle.dispatch_combine(hid, ids, wts, E, R)
    a, b = res["out"], hid
    assert np.all((a == b) | (((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)))


def pin_combine_one_hot():
    """A one-hot weight row selects exactly one expert output: the combine of
    token t is then y[t, j0] bit for bit, so every (token, slot) -> row link
    and every weight index is exercised."""
    rng = np.random.default_rng(51)
    for T, E, R, k, H in [(64, 16, 4, 4, 16), (200, 384, 8, 6, 24), (33, 8, 8, 8, 8)]:
        ids = rand_ids(rng, T, E, k)
        y = synth.normal_bf16(7, 2, T * k * H).reshape(T, k, H)
        lay = oracle.layout(ids, E, R)
        eo = oracle.place_slots(y, lay["pair_row"], T * k)
        for j0 in range(k):
            w = np.zeros((T, k), np.float32)
            w[:, j0] = 1.0
            out, out32, err = oracle.combine(eo, lay["pair_row"], w)
            assert err == 0
            assert np.array_equal(out, y[:, j0, :]), (T, E, k, j0)
        j0 = rng.integers(0, k, T)
        w = np.zeros((T, k), np.float32)
        w[np.arange(T), j0] = 1.0
        out, _, _ = oracle.combine(eo, lay["pair_row"], w)
        assert np.array_equal(out, y[np.arange(T), j0, :])


def pin_combine_scaling_and_skip():
    """Doubling every weight doubles the float32 sum exactly; slots whose id is
    -1 contribute nothing whatever their weight."""
    rng = np.random.default_rng(61)
    T, E, R, k, H = 90, 32, 8, 4, 32
    ids = rand_ids(rng, T, E, k, p_neg=0.25)
    y = synth.normal_bf16(9, 2, T * k * H).reshape(T, k, H)
    lay = oracle.layout(ids, E, R)
    eo = oracle.place_slots(y, lay["pair_row"], T * k)
    w = rng.random((T, k)).astype(np.float32)
    _, a32, _ = oracle.combine(eo, lay["pair_row"], w)
    _, b32, _ = oracle.combine(eo, lay["pair_row"], w * np.float32(2))
    assert np.array_equal(b32, a32 * np.float32(2))
    w2 = np.where(ids < 0, np.float32(1e30), w).astype(np.float32)
    _, c32, _ = oracle.combine(eo, lay["pair_row"], w2)
    assert np.array_equal(c32, a32)


def pin_combine_k1():
    rng = np.random.default_rng(71)
    T, E, R, H = 50, 8, 2, 16
    ids = rng.integers(0, E, (T, 1)).astype(np.int32)
    y = synth.normal_bf16(3, 2, T * H).reshape(T, 1, H)
    lay = oracle.layout(ids, E, R)
    eo = oracle.place_slots(y, lay["pair_row"], T)
    out, _, _ = oracle.combine(eo, lay["pair_row"], np.ones((T, 1), np.float32))
    assert np.array_equal(out, y[:, 0, :])


def pin_combine_exact_bound():
    """Against the exact rational sum: the float32 result of a chain of k fused
    multiply-adds is within gamma_k * sum|w*y| (gamma_k = k*u / (1 - k*u),
    u = 2^-24), the bf16 output is a nearest bf16 of the float32 result, and
    the double-precision variant is within 2^-50 of exact."""
    rng = np.random.default_rng(81)
    for T, E, R, k, H in [(24, 16, 4, 6, 8), (16, 64, 8, 8, 12), (20, 8, 2, 2, 8)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1)
        y = synth.normal_bf16(11, 2, T * k * H).reshape(T, k, H)
        w = (rng.standard_normal((T, k)) * 3).astype(np.float32)
        lay = oracle.layout(ids, E, R)
        eo = oracle.place_slots(y, lay["pair_row"], T * k)
        out, out32, _ = oracle.combine(eo, lay["pair_row"], w)
        out64, _ = oracle.combine_f64(eo, lay["pair_row"], w)
        yf = bf16_bits_to_float(y)
        gamma = k * U32 / (1 - k * U32)
        for t in range(T):
            for h in range(H):
                terms = [Fraction(float(w[t, j])) * Fraction(float(yf[t, j, h]))
                         for j in range(k) if ids[t, j] >= 0]
                exact = sum(terms, Fraction(0))
                mag = sum((abs(x) for x in terms), Fraction(0))
                err32 = abs(Fraction(float(out32[t, h])) - exact)
                assert err32 <= gamma * mag, (t, h, float(err32), float(mag))
                assert abs(Fraction(float(out64[t, h])) - exact) <= Fraction(2) ** -50 * mag
                # nearest bf16: no other bf16 is strictly closer to the float32 value
                o = int(out[t, h])
                acc = Fraction(float(out32[t, h]))
                mine = abs(Fraction(float(bf16_bits_to_float(o))) - acc)
                for nb in (o - 1, o + 1):
                    if 0 <= nb < 65536 and (nb & 0x7F80) != 0x7F80:
                        assert abs(Fraction(float(bf16_bits_to_float(nb))) - acc) >= mine


def pin_combine_rounding_ties():
    """Round to nearest, ties to even, on float32 sums that fall exactly
    halfway between two bf16 values (1 + 2^-8 lies halfway between 1 and
    1 + 2^-7; 1 + 3*2^-8 halfway between 1 + 2^-7 and 1 + 2^-6)."""
    E, R, H = 4, 2, 8
    ids = np.array([[0], [1], [2], [3]], np.int32)
    one = np.full((4, 1, H), 0x3F80, np.uint16)  # bf16 1.0
    lay = oracle.layout(ids, E, R)
    eo = oracle.place_slots(one, lay["pair_row"], 4)
    w = np.array([[1 + 2 ** -8], [1 + 3 * 2 ** -8], [-(1 + 2 ** -8)], [1 + 2 ** -7]],
                 np.float32)
    out, out32, _ = oracle.combine(eo, lay["pair_row"], w)
    # 1+2^-8 -> 1.0 (even mantissa 0x00); 1+3*2^-8 -> 1+2^-6 (0x3F82, even);
    # negative tie -> -1.0; 1+2^-7 is exact (0x3F81).
    assert list(out[:, 0]) == [0x3F80, 0x3F82, 0xBF80, 0x3F81], [hex(v) for v in out[:, 0]]


def pin_combine_single_rounding():
    """Each slot is one fused multiply-add (one rounding of w*y + acc), not a
    rounded product added afterwards. Hand-derived: with y = 1 + 2^-7 (bf16
    0x3F81) in both slots and w = -(1 + 2^-20), then 1 + 2^-20, the first
    product -(1 + 2^-7 + 2^-20 + 2^-27) rounds to -(1 + 2^-7 + 2^-20); the
    second fused step then leaves exactly 2^-27 (bf16 0x3200), where a
    rounded product would cancel to 0."""
    E, R, H = 4, 2, 8
    ids = np.array([[0, 3]], np.int32)
    y = np.full((1, 2, H), 0x3F81, np.uint16)
    w = np.array([[-(1 + 2 ** -20), 1 + 2 ** -20]], np.float32)
    lay = oracle.layout(ids, E, R)
    eo = oracle.place_slots(y, lay["pair_row"], 2)
    out, out32, _ = oracle.combine(eo, lay["pair_row"], w)
    assert np.all(out32 == np.float32(2 ** -27)), out32
    assert np.all(out == 0x3200)


# ----------------------------------------------------------------------------
# two-stage combine pins

def _two_stage(ids, y, w, E, R, cap_rank=None, cap_expert=None):
    T, k = ids.shape
    lay = oracle.layout(ids, E, R)
    cap_rank = T * min(k, R) if cap_rank is None else cap_rank
    cap_expert = T * k if cap_expert is None else cap_expert
    rb, src, _ = oracle.pack(np.zeros((T, 8), np.uint16), lay["token_rank_slot"], cap_rank)
    eo = oracle.place_slots(y, lay["pair_row"], cap_expert)
    part, part32, e1 = oracle.combine_rank_partial(eo, src, lay["rank_offsets"], ids,
                                                   lay["pair_row"], w, E, cap_rank)
    out, out32, e2 = oracle.combine_ranks(part, lay["token_rank_slot"])
    return dict(lay=lay, src=src, eo=eo, part=part, part32=part32, out=out, out32=out32,
                err=e1 | e2)


def pin_two_stage_order():
    """Hand-derived cases where the order of the float32 additions shows. Slot
    order inside a rank: three experts of rank 0 in slots (e2, e0, e1) with
    y = 2^-24, 2^-24, 1 (bf16 0x3380, 0x3380, 0x3F80) and w = 1 give
    2^-24 -> 2^-23 -> 1 + 2^-23 in slot order (expert-id or reversed slot
    order would give 1). Ascending rank order at home: partials 2^-24, 2^-24,
    1 on ranks 0, 1, 2 reached in slot order (r2, r0, r1) give 1 + 2^-23
    (slot order or descending ranks would give 1)."""
    H = 8
    tiny, one = 0x3380, 0x3F80
    ids = np.array([[2, 0, 1]], np.int32)
    y = np.array([[[tiny] * H, [tiny] * H, [one] * H]], np.uint16)
    w = np.ones((1, 3), np.float32)
    r = _two_stage(ids, y, w, E=6, R=2)
    assert np.all(r["part32"][0] == np.float32(1 + 2 ** -23)), r["part32"][0]
    y2 = np.array([[[one] * H, [tiny] * H, [tiny] * H]], np.uint16)
    r2 = _two_stage(ids, y2, w, E=3, R=3)
    assert np.all(r2["out32"][0] == np.float32(1 + 2 ** -23)), r2["out32"][0]
    assert np.all(r2["out"][0] == one)  # 1 + 2^-23 rounds to bf16 1.0


def pin_two_stage_single_rounding():
    """The first stage is the same fused chain: the hand-derived case of
    pin_combine_single_rounding with both experts on one rank leaves 2^-27
    in the partial row, and the home sum of that single row is 2^-27."""
    H = 8
    ids = np.array([[0, 1]], np.int32)
    y = np.full((1, 2, H), 0x3F81, np.uint16)
    w = np.array([[-(1 + 2 ** -20), 1 + 2 ** -20]], np.float32)
    r = _two_stage(ids, y, w, E=4, R=2)
    assert np.all(r["part32"][0] == np.float32(2 ** -27))
    assert np.all(r["part"][0] == 0x3200)
    assert np.all(r["out"][0] == 0x3200)


def pin_two_stage_exact_integers():
    """Small integer outputs and weights in {-1, 1/2, 1, 2}: every partial and
    every total is exact in float32 and in bf16, so each partial row must equal
    the plain integer sum over its rank's slots and each output the sum over
    all slots (checks which rows, slots and ranks take part)."""
    rng = np.random.default_rng(91)
    for T, E, R, k, H in [(40, 16, 4, 4, 8), (64, 64, 8, 8, 8), (30, 12, 2, 3, 16),
                          (25, 8, 8, 5, 8)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.2)
        yv = rng.integers(-4, 5, (T, k, H)).astype(np.float32)
        y = (yv.view(np.uint32) >> 16).astype(np.uint16)  # small integers are exact bf16
        w = rng.choice(np.array([-1, 0.5, 1, 2], np.float32), (T, k))
        r = _two_stage(ids, y, w, E, R)
        assert r["err"] == 0
        m = E // R
        ok = ids >= 0
        want = np.einsum("tk,tkh->th", np.where(ok, w, 0).astype(np.float64), yv)
        assert np.array_equal(r["out32"].astype(np.float64), want)
        assert np.array_equal(bf16_bits_to_float(r["out"]).astype(np.float64), want)
        slots = r["lay"]["token_rank_slot"]
        for t in range(T):
            for rk in range(R):
                on = ok[t] & (ids[t] // m == rk)
                if slots[t, rk] < 0:
                    assert not on.any()
                    continue
                part = (w[t, on].astype(np.float64)[:, None] * yv[t, on]).sum(0)
                assert np.array_equal(bf16_bits_to_float(r["part"][slots[t, rk]]), part)


def pin_two_stage_one_expert_per_rank():
    """With one expert per rank (E = R) each partial row is a single product:
    bf16(fl32(w * y)), checked against numpy's float32 multiply and torch's
    bfloat16 conversion (round to nearest even)."""
    import torch

    rng = np.random.default_rng(93)
    for T, E, k, H in [(30, 8, 3, 16), (20, 4, 4, 8)]:
        ids = rand_ids(rng, T, E, k)
        y = synth.normal_bf16(13, 2, T * k * H).reshape(T, k, H)
        w = (rng.standard_normal((T, k)) * 3).astype(np.float32)
        r = _two_stage(ids, y, w, E, E)
        prod = w[:, :, None] * bf16_bits_to_float(y)  # float32 * float32, one rounding
        want = torch.from_numpy(np.ascontiguousarray(prod)).to(torch.bfloat16).view(
            torch.int16).numpy().view(np.uint16)
        slots = r["lay"]["token_rank_slot"]
        for t in range(T):
            for j in range(k):
                s = slots[t, ids[t, j]]
                assert np.array_equal(r["part32"][s], prod[t, j]), (t, j)
                assert np.array_equal(r["part"][s], want[t, j]), (t, j)


def pin_two_stage_one_rank():
    """With a single rank the first stage is the whole fused chain in slot
    order and the second stage adds one row to +0: the two-stage result equals
    the one-stage combine bit for bit."""
    rng = np.random.default_rng(95)
    for T, E, k, H in [(50, 16, 4, 16), (37, 64, 8, 8)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1)
        ids[:, 0] = rng.integers(0, E, T)
        y = synth.normal_bf16(15, 2, T * k * H).reshape(T, k, H)
        w = (rng.standard_normal((T, k))).astype(np.float32)
        r = _two_stage(ids, y, w, E, 1)
        out, out32, _ = oracle.combine(r["eo"], r["lay"]["pair_row"], w)
        assert np.array_equal(r["src"], np.arange(T))
        assert np.array_equal(r["part32"], out32)
        assert np.array_equal(r["out"], out)


def pin_two_stage_exact_bound():
    """Against the exact rational sum: two-stage float32 result within
    ((k + R) u + 2^-8) * 1.01 * sum|w*y| (u = 2^-24: a fused chain per rank, one
    bf16 rounding of each partial, a chain of float32 adds over the ranks);
    doubling every weight doubles every partial and output exactly."""
    rng = np.random.default_rng(97)
    for T, E, R, k, H in [(20, 16, 4, 6, 8), (16, 64, 8, 8, 8)]:
        ids = rand_ids(rng, T, E, k, p_neg=0.1)
        y = synth.normal_bf16(17, 2, T * k * H).reshape(T, k, H)
        w = (rng.standard_normal((T, k)) * 3).astype(np.float32)
        r = _two_stage(ids, y, w, E, R)
        yf = bf16_bits_to_float(y)
        bound = ((k + R) * Fraction(1, 2 ** 24) + Fraction(1, 256)) * Fraction(101, 100)
        for t in range(T):
            for h in range(H):
                terms = [Fraction(float(w[t, j])) * Fraction(float(yf[t, j, h]))
                         for j in range(k) if ids[t, j] >= 0]
                exact = sum(terms, Fraction(0))
                mag = sum((abs(x) for x in terms), Fraction(0))
                assert abs(Fraction(float(r["out32"][t, h])) - exact) <= bound * mag, (t, h)
        r2 = _two_stage(ids, y, w * np.float32(2), E, R)
        assert np.array_equal(r2["part32"], r["part32"] * np.float32(2))
        assert np.array_equal(r2["out32"], r["out32"] * np.float32(2))


def pin_two_stage_caps():
    """Undersized buffers: a pair row past cap_expert contributes nothing (as a
    zero weight would) and is reported; rank-buffer rows past cap_rank get no
    partial and are reported by the home sum."""
    rng = np.random.default_rng(99)
    T, E, R, k, H = 40, 16, 4, 3, 8
    ids = rand_ids(rng, T, E, k)
    y = synth.normal_bf16(19, 2, T * k * H).reshape(T, k, H)
    w = rng.random((T, k)).astype(np.float32)
    full = _two_stage(ids, y, w, E, R)
    P = T * k
    r = _two_stage(ids, y, w, E, R, cap_expert=P - 4)
    assert r["err"] == oracle.ERR_EXPERT_CAP
    w0 = np.where(full["lay"]["pair_row"] >= P - 4, np.float32(0), w)
    r0 = _two_stage(ids, y, w0, E, R)
    assert np.array_equal(r["part32"], r0["part32"]) and np.array_equal(r["out"], r0["out"])
    C = int(full["lay"]["rank_offsets"][-1])
    rc = _two_stage(ids, y, w, E, R, cap_rank=C - 6)
    assert rc["err"] == oracle.ERR_RANK_CAP
    assert np.array_equal(rc["part32"], full["part32"][:C - 6])


# ----------------------------------------------------------------------------
# quantised dispatch (MXFP8) pins

def _bf16(x) -> np.ndarray:
    """float values exactly representable in bf16 -> bit patterns."""
    a = np.asarray(x, np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _e4m3_table():
    """Magnitudes of the 127 finite non-negative OCP E4M3 codes, from the
    format's definition (bias 7, 3 mantissa bits, subnormals at exponent 0)."""
    vals = []
    for c in range(0x7F):
        ef, mf = c >> 3, c & 7
        vals.append(mf * 2.0 ** -9 if ef == 0 else (1 + mf / 8) * 2.0 ** (ef - 7))
    return np.array(vals)


def pin_mxfp8_every_code_round_trips():
    """A block whose largest magnitude is 448 (the largest e4m3 normal) has
    scale 2^0; every finite e4m3 value, of either sign (-0 included), placed
    in such blocks comes back as its own code."""
    mags = _e4m3_table()
    codes = np.concatenate([np.arange(0x7F), np.arange(0x7F) | 0x80])
    blocks, want = [], []
    for i in range(0, codes.size, 31):
        chunk = list(codes[i:i + 31])
        chunk += [0x7E] * (31 - len(chunk))
        want.append([0x7E] + chunk)
    want = np.array(want)
    vals = np.where(want & 0x80, -1.0, 1.0) * mags[want & 0x7F]
    x = _bf16(vals.astype(np.float32))
    q, sc = oracle.quantize_mxfp8(x)
    assert np.all(sc == 127), sc
    assert np.array_equal(q, want), np.argwhere(q != want)[:5]


def pin_mxfp8_hand_cases():
    """Hand-derived cases of the OCP MX rule (scale 2^e, e = floor(log2 amax) - 8,
    clamped to [-127, 127]; nearest e4m3, ties to even, saturating at 448)."""
    H = 32

    def one_block(values, pad=0.0):
        v = list(values) + [pad] * (H - len(values))
        return oracle.quantize_mxfp8(_bf16(np.array([v], np.float32)))

    # amax 1 -> e = -8: 1 -> 256 = 2^8 (0x78); 0.5 -> 2^7 (0x70); -1.5 -> -384 (0xFC)
    q, sc = one_block([1.0, 0.5, -1.5])
    assert int(sc[0, 0]) == 127 - 8 and list(q[0, :3]) == [0x78, 0x70, 0xFC], (sc, q[0, :3])
    # with 448 present e = 0: 1.0625 is halfway between 1 (0x38) and 1.125 (0x39) -> even 0x38;
    # 1.1875 halfway between 1.125 and 1.25 -> 0x3A; 2^-9 -> 0x01; 2^-10 halfway between 0 and
    # 2^-9 -> 0x00; 3*2^-10 halfway between 2^-9 and 2^-8 -> 0x02; -2^-11 -> -0 (0x80)
    q, sc = one_block([448.0, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -2.0 ** -11])
    assert int(sc[0, 0]) == 127
    assert list(q[0, :7]) == [0x7E, 0x38, 0x3A, 0x01, 0x00, 0x02, 0x80], [hex(c) for c in q[0, :7]]
    # amax 510 -> e = 0 and 510 saturates to 448; 480 too
    q, sc = one_block([510.0, -480.0, 464.0])
    assert int(sc[0, 0]) == 127 and list(q[0, :3]) == [0x7E, 0xFE, 0x7E]
    # smallest bf16 subnormal 2^-133: e = -141 clamps to -127, 2^-133 / 2^-127 = 2^-6 (0x08)
    q, sc = oracle.quantize_mxfp8(np.array([[0x0001] + [0] * 31], np.uint16))
    assert int(sc[0, 0]) == 0 and q[0, 0] == 0x08 and np.all(q[0, 1:] == 0)
    # 1.5 * 2^127: e = 119, value / 2^119 = 384 (0x7C)
    q, sc = oracle.quantize_mxfp8(np.array([[0x7F40] + [0] * 31], np.uint16))
    assert int(sc[0, 0]) == 127 + 119 and q[0, 0] == 0x7C
    # an all-zero block: scale 2^-127, codes 0 (and 0x80 for -0)
    q, sc = oracle.quantize_mxfp8(np.array([[0x0000, 0x8000] + [0] * 30], np.uint16))
    assert int(sc[0, 0]) == 0 and q[0, 0] == 0x00 and q[0, 1] == 0x80
    # a NaN or an infinity makes the block's scale NaN (0xFF) and its codes NaN with their sign
    for bad in (0x7FC0, 0x7F80, 0xFF80):
        q, sc = oracle.quantize_mxfp8(np.array([[0x3F80, bad, 0xBF80] + [0] * 29], np.uint16))
        assert int(sc[0, 0]) == 0xFF and q[0, 0] == 0x7F and q[0, 2] == 0xFF
        assert q[0, 1] == (0xFF if bad & 0x8000 else 0x7F)


def pin_mxfp8_error_bound():
    """Random rows of several magnitudes: the block maximum lands in [256, 512)
    after scaling (e is the largest exponent that does not push it to 512 or
    past), and every element is within half an e4m3 step of its value
    (2^-4 relative for normals, 2^-10 absolute below 2^-6), unless it
    saturated at 448."""
    rng = np.random.default_rng(107)
    mags = _e4m3_table()
    for spread in (1.0, 8.0, 30.0):
        vals = rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-spread, spread, (64, 256)))
        x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16
        q, sc = oracle.quantize_mxfp8(x)
        xf = bf16_bits_to_float(x).astype(np.float64).reshape(64, 8, 32)
        e = sc.astype(np.int64) - 127
        scaled = np.abs(xf) / np.exp2(e)[:, :, None]
        top = scaled.max(axis=2)
        ok = (e > -127) & (e < 127)
        assert np.all((top[ok] >= 256) & (top[ok] < 512))
        deq = mags[(q & 0x7F).reshape(64, 8, 32)]
        sat = scaled > 448
        err = np.abs(deq - scaled)
        lim = np.maximum(np.exp2(np.floor(np.log2(np.maximum(scaled, 2.0 ** -6))) - 4), 2.0 ** -10)
        assert np.all((err <= lim) | sat)
        assert np.all(deq[sat] == 448)
        sign = (q.reshape(64, 8, 32) & 0x80) != 0
        assert np.all(sign == (xf < 0) | ((xf == 0) & np.signbit(xf)))


def pin_mxfp8_pack_and_permute():
    """The quantised dispatch moves bytes only: every packed row holds the codes
    and scales of its source token's quantised row, every expert row those of
    its rank-buffer row."""
    rng = np.random.default_rng(109)
    T, E, R, k, H = 80, 32, 4, 4, 128
    ids = rand_ids(rng, T, E, k, p_neg=0.1)
    hid = synth.normal_bf16(25, 0, T * H).reshape(T, H)
    lay = oracle.layout(ids, E, R)
    q, sc = oracle.quantize_mxfp8(hid)
    rq, rs, src, err = oracle.pack_mxfp8(hid, lay["token_rank_slot"], T * min(k, R))
    C = int(lay["rank_offsets"][-1])
    assert err == 0 and np.array_equal(rq[:C], q[src[:C]]) and np.array_equal(rs[:C], sc[src[:C]])
    eq, es, esrc, err2 = oracle.permute_mxfp8(rq, rs, src, lay, ids, E, T * k)
    P = int(lay["expert_offsets"][-1])
    t_of = esrc[:P] // k
    assert err2 == 0 and np.array_equal(eq[:P], q[t_of]) and np.array_equal(es[:P], sc[t_of])


def _e2m1_table():
    """Magnitudes of the 8 non-negative OCP E2M1 codes from the format's
    definition (bias 1, one mantissa bit, a subnormal at exponent 0)."""
    return np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack_nibbles(q):
    q = np.asarray(q, np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def pin_mxfp4_every_code_round_trips():
    """A block whose largest magnitude is 6 (the largest e2m1 value) has scale
    2^0; all 16 codes (both signs, -0 included) come back as themselves, the
    even-indexed value in the low nibble."""
    mags = _e2m1_table()
    codes = np.array([7] + list(range(16)) + [7] * 15)
    vals = np.where(codes & 8, -1.0, 1.0) * mags[codes & 7]
    q, sc = oracle.quantize_mxfp4(_bf16(vals[None, :].astype(np.float32)))
    assert int(sc[0, 0]) == 127
    assert np.array_equal(_unpack_nibbles(q)[0], codes), _unpack_nibbles(q)[0]
    assert q[0, 0] == 0x07 | (0x00 << 4) and q[0, 1] == 0x01 | (0x02 << 4)


def pin_mxfp4_hand_cases():
    """Hand-derived cases of the MX rule for e2m1 (e = floor(log2 amax) - 2):
    ties go to the even code, magnitudes past 6 saturate, the scale clamps."""
    H = 32

    def block(values, pad=0.0):
        v = list(values) + [pad] * (H - len(values))
        q, sc = oracle.quantize_mxfp4(_bf16(np.array([v], np.float32)))
        return _unpack_nibbles(q)[0], int(sc[0, 0])

    # with 6 present e = 0: 0.25 -> 0 (tie 0 / 0.5), 0.75 -> 1.0 (tie 0.5 / 1), 1.25 -> 1.0,
    # 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5.0 -> 4.0, -0.25 -> -0 (code 8)
    c, s = block([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25])
    assert s == 127 and list(c[:9]) == [7, 0, 2, 2, 4, 4, 6, 6, 8], list(c[:9])
    # amax 7 -> e = 0, 7 saturates to 6; amax 1 -> e = -2: 1 -> 4 (code 6), 0.375 -> 1.5 (3)
    c, s = block([7.0, -6.5])
    assert s == 127 and list(c[:2]) == [7, 15]
    c, s = block([1.0, 0.375, -0.0625])
    assert s == 127 - 2 and list(c[:3]) == [6, 3, 8 | 0], list(c[:3])  # -0.25 ties to -0
    # smallest bf16 subnormal: e = -135 clamps to -127, 2^-133 / 2^-127 = 2^-6 -> 0 (code 0)
    q, sc = oracle.quantize_mxfp4(np.array([[0x0001] + [0] * 31], np.uint16))
    assert int(sc[0, 0]) == 0 and np.all(q == 0)
    # NaN / infinity: scale 0xFF, codes of the largest magnitude with their sign
    q, sc = oracle.quantize_mxfp4(np.array([[0x3F80, 0x7FC0, 0xBF80, 0xFF80] + [0] * 28],
                                           np.uint16))
    assert int(sc[0, 0]) == 0xFF and list(_unpack_nibbles(q)[0, :4]) == [7, 7, 15, 15]


def pin_mxfp4_error_bound():
    """Random rows: after scaling the block maximum lies in [4, 8) and every
    value is within half an e2m1 step of its code (a quarter below 2, a half
    from 2 to 4, one from 4 to 6), unless it saturated at 6."""
    rng = np.random.default_rng(111)
    mags = _e2m1_table()
    vals = rng.standard_normal((64, 256)) * np.exp2(rng.uniform(-20, 20, (64, 256)))
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, sc = oracle.quantize_mxfp4(x)
    xf = bf16_bits_to_float(x).astype(np.float64).reshape(64, 8, 32)
    e = sc.astype(np.int64) - 127
    scaled = np.abs(xf) / np.exp2(e)[:, :, None]
    ok = (e > -127) & (e < 127)
    top = scaled.max(axis=2)
    assert np.all((top[ok] >= 4) & (top[ok] < 8))
    codes = _unpack_nibbles(q).reshape(64, 8, 32)
    deq = mags[codes & 7]
    sat = scaled > 6
    step = np.where(scaled < 2, 0.5, np.where(scaled < 4, 1.0, 2.0))
    assert np.all((np.abs(deq - scaled) <= step / 2) | sat)
    assert np.all(deq[sat] == 6)
    assert np.all(((codes & 8) != 0) == np.signbit(xf))


def pin_mxfp4_pack_and_permute():
    """The 4-bit dispatch moves bytes only: packed and regrouped rows hold the
    codes and scales of their source token's quantised row."""
    rng = np.random.default_rng(113)
    T, E, R, k, H = 70, 32, 4, 3, 128
    ids = rand_ids(rng, T, E, k, p_neg=0.1)
    hid = synth.normal_bf16(27, 0, T * H).reshape(T, H)
    lay = oracle.layout(ids, E, R)
    q, sc = oracle.quantize_mxfp4(hid)
    rq, rs, src, err = oracle.pack_mxfp4(hid, lay["token_rank_slot"], T * min(k, R))
    C = int(lay["rank_offsets"][-1])
    assert err == 0 and np.array_equal(rq[:C], q[src[:C]]) and np.array_equal(rs[:C], sc[src[:C]])
    eq, es, esrc, err2 = oracle.permute_mxfp4(rq, rs, src, lay, ids, E, T * k)
    P = int(lay["expert_offsets"][-1])
    t_of = esrc[:P] // k
    assert err2 == 0 and np.array_equal(eq[:P], q[t_of]) and np.array_equal(es[:P], sc[t_of])


def pin_nvfp4_row_bytes():
    """The pages' 4-bit row: 2,880 bytes for a 5,120-wide row ("A2A backends"
    page, section 7.2), 2,560 code bytes and one scale byte per 16 values."""
    q, sc = oracle.quantize_nvfp4(np.zeros((1, 5120), np.uint16))
    assert q.shape[1] + sc.shape[1] == 2880 and sc.shape[1] == 5120 // 16


def pin_nvfp4_every_code_round_trips():
    """A block whose largest magnitude is 6 has scale 1 (E4M3 code 0x38) and all
    16 codes (both signs, -0 included) come back as themselves; the same block
    times 1.5 has scale 1.5 (0x3C) and the same codes."""
    mags = _e2m1_table()
    codes = np.arange(16)
    vals = np.where(codes & 8, -1.0, 1.0) * mags[codes & 7]
    for factor, want in ((1.0, 0x38), (1.5, 0x3C)):
        q, sc = oracle.quantize_nvfp4(_bf16((vals * factor)[None, :].astype(np.float32)))
        assert int(sc[0, 0]) == want, hex(int(sc[0, 0]))
        assert np.array_equal(_unpack_nibbles(q)[0], codes), _unpack_nibbles(q)[0]


def pin_nvfp4_hand_cases():
    """Hand-derived cases of the 16-value rule: s = E4M3 nearest to amax / 6 with
    ties to the even code, codes = e2m1 nearest to |v| / s with ties to even."""
    def block(values):
        v = list(values) + [0.0] * (16 - len(values))
        q, sc = oracle.quantize_nvfp4(_bf16(np.array([v], np.float32)))
        return list(_unpack_nibbles(q)[0]), int(sc[0, 0])

    # amax 6.375: amax/6 = 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): 0x38
    c, s = block([6.375, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25])
    assert s == 0x38 and c[:9] == [7, 0, 2, 2, 4, 4, 6, 6, 8], (hex(s), c[:9])
    # amax 6.75: amax/6 = 1.125 exactly (0x39); 6.75/1.125 = 6, 2.25/1.125 = 2
    c, s = block([6.75, -2.25])
    assert s == 0x39 and c[:2] == [7, 12], (hex(s), c[:2])
    # amax 3072: 512 saturates to 448 (0x7E); 3072/448 = 6.9 saturates to 6
    c, s = block([3072.0, -448.0])
    assert s == 0x7E and c[:2] == [7, 8 | 2], (hex(s), c[:2])
    # amax 6 * 2^-9: the smallest subnormal scale 2^-9 (0x01)
    c, s = block([6 * 2.0 ** -9, -2.0 ** -9])
    assert s == 0x01 and c[:2] == [7, 8 | 2], (hex(s), c[:2])
    # amax 6 * 2^-10: amax/6 = 2^-10 ties between 0 and 2^-9, even code 0: a zero
    # scale, and every code zero with its sign
    c, s = block([6 * 2.0 ** -10, -2.0 ** -12])
    assert s == 0x00 and c[:2] == [0, 8], (hex(s), c[:2])
    # values far past 6 * 448: the scale saturates at 448 and those codes at 6, however
    # large the quotient (|v| / s up to 7.6e35)
    q, sc = oracle.quantize_nvfp4(np.array([[0x7F7F, 0xFF00, 0x4780, 0x3F80] + [0] * 12],
                                           np.uint16))
    c = list(_unpack_nibbles(q)[0, :4])
    assert int(sc[0, 0]) == 0x7E and c == [7, 15, 7, 0], (hex(int(sc[0, 0])), c)
    # an all-zero block: scale 0, codes 0
    c, s = block([])
    assert s == 0 and c == [0] * 16
    # NaN / infinity: the E4M3 NaN scale 0x7F, codes of the largest magnitude with signs
    q, sc = oracle.quantize_nvfp4(np.array([[0x3F80, 0x7FC0, 0xBF80, 0xFF80] + [0] * 12],
                                           np.uint16))
    assert int(sc[0, 0]) == 0x7F and list(_unpack_nibbles(q)[0, :4]) == [7, 7, 15, 15]


def pin_nvfp4_error_bound():
    """Random rows over 24 binades: a block's scale is within half an E4M3 step
    of amax / 6 (unless it saturated or went subnormal), and every value is
    within half an e2m1 step (times the scale) of its code unless it saturated
    at 6; signs are kept."""
    rng = np.random.default_rng(117)
    e4m3 = _e4m3_table()
    mags = _e2m1_table()
    binade = np.exp2(rng.uniform(-10, 14, (64, 16, 1))).repeat(16, axis=2).reshape(64, 256)
    vals = rng.standard_normal((64, 256)) * binade
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, sc = oracle.quantize_nvfp4(x)
    xf = bf16_bits_to_float(x).astype(np.float64).reshape(64, 16, 16)
    s = e4m3[sc.astype(np.int64)]
    t = np.abs(xf).max(axis=2) / 6
    normal = (sc >= 8) & (sc < 0x7E)
    assert normal.sum() > 400 and (sc == 0x7E).any() and (sc < 8).any()
    half_step = np.exp2(np.floor(np.log2(s[normal]))) / 16
    assert np.all(np.abs(s[normal] - t[normal]) <= half_step)
    codes = _unpack_nibbles(q).reshape(64, 16, 16)
    ok = s > 0
    scaled = np.abs(xf[ok]) / s[ok][:, None]
    deq = mags[codes[ok] & 7]
    sat = scaled > 6
    step = np.where(scaled < 2, 0.5, np.where(scaled < 4, 1.0, 2.0))
    assert np.all((np.abs(deq - scaled) <= step / 2) | sat)
    assert np.all(deq[sat] == 6)
    assert np.all(((codes & 8) != 0) == np.signbit(xf))


def pin_nvfp4_pack_and_permute():
    """The 16-value-block 4-bit dispatch moves bytes only: packed and regrouped
    rows hold the codes and scales of their source token's quantised row."""
    rng = np.random.default_rng(119)
    T, E, R, k, H = 70, 32, 4, 3, 128
    ids = rand_ids(rng, T, E, k, p_neg=0.1)
    hid = synth.normal_bf16(29, 0, T * H).reshape(T, H)
    lay = oracle.layout(ids, E, R)
    q, sc = oracle.quantize_nvfp4(hid)
    rq, rs, src, err = oracle.pack_nvfp4(hid, lay["token_rank_slot"], T * min(k, R))
    C = int(lay["rank_offsets"][-1])
    assert err == 0 and np.array_equal(rq[:C], q[src[:C]]) and np.array_equal(rs[:C], sc[src[:C]])
    eq, es, esrc, err2 = oracle.permute_nvfp4(rq, rs, src, lay, ids, E, T * k)
    P = int(lay["expert_offsets"][-1])
    t_of = esrc[:P] // k
    assert err2 == 0 and np.array_equal(eq[:P], q[t_of]) and np.array_equal(es[:P], sc[t_of])


PINS = [
    pin_layout_stable_sort,
    pin_layout_brute_force,
    pin_layout_invariants,
    pin_closed_form_exhaustive,
    pin_closed_form_workloads,
    pin_page_bytes,
    pin_figure1,
    pin_figure4,
    pin_bad_ids,
    pin_pack_permute_rows,
    pin_permute_reads_own_segment,
    pin_caps,
    pin_layout_padded_and_masked,
    pin_permute_padding_rows,
    pin_roundtrip_identity,
    pin_combine_one_hot,
    pin_combine_scaling_and_skip,
    pin_combine_k1,
    pin_combine_exact_bound,
    pin_combine_rounding_ties,
    pin_combine_single_rounding,
    pin_two_stage_order,
    pin_two_stage_single_rounding,
    pin_two_stage_exact_integers,
    pin_two_stage_one_expert_per_rank,
    pin_two_stage_one_rank,
    pin_two_stage_exact_bound,
    pin_two_stage_caps,
    pin_mxfp8_every_code_round_trips,
    pin_mxfp8_hand_cases,
    pin_mxfp8_error_bound,
    pin_mxfp8_pack_and_permute,
    pin_mxfp4_every_code_round_trips,
    pin_mxfp4_hand_cases,
    pin_mxfp4_error_bound,
    pin_mxfp4_pack_and_permute,
    pin_nvfp4_row_bytes,
    pin_nvfp4_every_code_round_trips,
    pin_nvfp4_hand_cases,
    pin_nvfp4_error_bound,
    pin_nvfp4_pack_and_permute,
]
