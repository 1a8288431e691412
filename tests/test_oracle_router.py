"""Pins for oracle/router.py: top-k by exhaustive subsets, exact ties, weight invariants."""
import itertools

import numpy as np

import synth
from oracle import router as R


def _beats(l, i, j):
    return l[i] > l[j] or (l[i] == l[j] and i < j)


def test_topk_equals_unique_dominating_subset_tiny():
    """Over all C(8,2) = 28 subsets, exactly one has every member beating every
    non-member (higher logit, or equal logit and lower index); it is the oracle's."""
    cfg = synth.CONFIGS["tiny_bf16"]
    L = synth.make_layer(cfg)
    rng = np.random.default_rng(3)
    for trial in range(200):
        x = synth.to_bf16_bits(rng.normal(size=(1, cfg.H)))
        ids, w, lg = R.route(x, L["router_w"], None, cfg.k)
        l = lg[0]
        good = [S for S in itertools.combinations(range(cfg.E), cfg.k)
                if all(_beats(l, i, j) for i in S for j in range(cfg.E) if j not in S)]
        assert len(good) == 1
        assert set(ids[0].tolist()) == set(good[0])
        assert all(l[ids[0, j]] >= l[ids[0, j + 1]] for j in range(cfg.k - 1))


def test_exact_ties_go_to_lower_index():
    E, H, k = 8, 64, 3
    rng = np.random.default_rng(5)
    Wr = rng.normal(size=(E, H)).astype(np.float32) * 0.01
    Wr[6] = Wr[2] = np.abs(Wr[2]) + 1.0           # identical rows -> bit-identical logits
    Wr[4] = Wr[2]
    x = synth.to_bf16_bits(np.abs(rng.normal(size=(4, H))) + 0.1)
    ids, w, lg = R.route(x, Wr, None, k)
    for t in range(4):
        assert lg[t, 2] == lg[t, 4] == lg[t, 6]
        assert list(ids[t]) == [2, 4, 6]
    ids2, _, _ = R.route(x, Wr, None, 2)          # the tie straddles the cut: 6 is dropped
    assert all(list(r) == [2, 4] for r in ids2)


def test_weights_sum_to_one_and_follow_sigmoid():
    cfg = synth.CONFIGS["flint_w4a16"]
    L = synth.make_layer(cfg, experts=[])
    x = synth.make_x(cfg, 8)
    ids, w, lg = R.route(x, L["router_w"], None, cfg.k)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(lg, ids.astype(np.int64), 1)))
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)        # sorted by logit -> sorted by weight


def test_sigmoid_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 800.0, -800.0])
    s = R.sigmoid(z)
    assert s[0] == 0.5
    assert np.isclose(s[1] + s[2], 1.0, rtol=0, atol=1e-16)
    assert np.isclose(s[1], 1 / (1 + np.e ** -1), rtol=1e-15)
    assert s[5] == 1.0 and 0.0 <= s[6] < 1e-300
    assert np.all(np.isfinite(s))


def test_bias_enters_selection_and_weights():
    E, H = 8, 32
    Wr = np.zeros((E, H), np.float32)
    bias = np.zeros(E, np.float32)
    bias[5] = 3.0
    bias[1] = -1.0
    x = synth.to_bf16_bits(np.ones((1, H)))
    ids, w, lg = R.route(x, Wr, bias, 2)
    assert list(ids[0]) == [5, 0]                 # 5 by bias, then the lowest index among zeros
    s5, s0 = 1 / (1 + np.exp(-3.0)), 0.5
    assert np.allclose(w[0], [s5 / (s5 + s0), s0 / (s5 + s0)], rtol=1e-15)


def test_ambiguity_flag():
    lg = np.array([[3.0, 1.0, 1.0 + 1e-7, -2.0], [3.0, 2.0, 1.0, 0.0]])
    amb = R.ambiguous_tokens(lg, 2)
    assert list(amb) == [True, False]
