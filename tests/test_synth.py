"""The seeded input generator: deterministic, counter-based, shaped as stated."""
import numpy as np

import synth


def test_counter_based_chunks_agree():
    whole = synth.normal_bf16(123, 0, 10_000)
    parts = np.concatenate([synth.normal_bf16(123, 0, 3_000, base=0),
                            synth.normal_bf16(123, 0, 7_000, base=3_000)])
    assert np.array_equal(whole, parts)
    assert not np.array_equal(whole, synth.normal_bf16(124, 0, 10_000))
    assert not np.array_equal(whole, synth.normal_bf16(123, 1, 10_000))


def test_normal_moments():
    x = synth.normal_f32(5, 0, 400_000).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_router_is_topk_of_softmax():
    w = synth.WORKLOADS["tiny"]
    ids, wts = synth.routing(w)
    assert ids.shape == (w.T, w.k) and wts.shape == (w.T, w.k)
    assert ids.dtype == np.int32 and wts.dtype == np.float32
    assert np.all((ids >= 0) & (ids < w.E))
    assert all(len(set(r)) == w.k for r in ids)
    assert np.allclose(wts.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(wts, axis=1) <= 0), "slots come in descending weight order"
    # the chosen ids are the k largest logits
    logits = synth.normal_f32(w.seed, synth.STREAM_LOGITS, w.T * w.E).reshape(w.T, w.E)
    for t in range(0, w.T, 17):
        top = np.argsort(-logits[t], kind="stable")[: w.k]
        assert list(top) == list(ids[t])


def test_skew_and_adversarial_shapes():
    s = synth.WORKLOADS["skew"]
    ids, _ = synth.routing(s)
    counts = np.bincount(ids.reshape(-1), minlength=s.E)
    assert counts.max() > 0.9 * s.T, "the hottest expert takes most tokens"
    a = synth.WORKLOADS["adv"]
    ids, _ = synth.routing(a)
    forced = synth.forced_tokens(a).astype(bool)
    assert forced.sum() == a.T // 10
    assert np.all(ids[forced] < a.m), "forced tokens pick only rank-0 experts"
    assert not np.all(ids[~forced] < a.m)


def test_expert_out_depends_on_token_expert_column():
    ids = np.array([[3, 5], [5, 3]], np.int32)
    y = synth.expert_out_slots(9, 8, 16, ids)
    y2 = synth.expert_out_slots(9, 8, 16, np.array([[3, -1], [5, 3]], np.int32))
    assert np.array_equal(y[0, 0], y2[0, 0]) and np.all(y2[0, 1] == 0)
    assert not np.array_equal(y[0, 0], y[1, 1])  # same expert, other token
