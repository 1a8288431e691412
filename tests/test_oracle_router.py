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


# ---------------------------------------------------------------- softmax routing
def test_softmax_over_all_experts_is_the_library_softmax():
    """With k = E nothing is left out: the weights are the softmax over every expert
    (scipy's implementation), in selection order."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    E, H = 8, 64
    Wr = rng.normal(size=(E, H)).astype(np.float32) * 0.3
    x = synth.to_bf16_bits(rng.normal(size=(5, H)))
    ids, w, lg = R.route(x, Wr, None, E, score="softmax")
    full = softmax(lg, axis=1)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-13, atol=0)


def _exact_logits(vals, H=32):
    """A router and one token whose FP64 logits are exactly vals (x = ones, Wr[e] = v/H)."""
    vals = np.asarray(vals, dtype=np.float64)
    Wr = np.repeat((vals / H)[:, None], H, axis=1).astype(np.float32)
    assert np.all(Wr.astype(np.float64) * H == vals[:, None])
    return synth.to_bf16_bits(np.ones((1, H))), Wr


def test_softmax_worked_example():
    x, Wr = _exact_logits([2.0, 1.0, 0.0, -1.0])
    ids, w, _ = R.route(x, Wr, None, 2, score="softmax")
    e = np.e
    assert list(ids[0]) == [0, 1]
    assert np.allclose(w[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-15)


def test_softmax_is_shift_invariant_and_sigmoid_is_not():
    rng = np.random.default_rng(12)
    E, H, k = 16, 64, 4
    Wr = rng.normal(size=(E, H)).astype(np.float32) * 0.1
    x = synth.to_bf16_bits(rng.normal(size=(6, H)))
    shift = np.full(E, 3.0, np.float32)
    i0, w0, _ = R.route(x, Wr, None, k, score="softmax")
    i1, w1, _ = R.route(x, Wr, shift, k, score="softmax")
    assert np.array_equal(i0, i1) and np.allclose(w0, w1, rtol=1e-12, atol=0)
    _, s0, _ = R.route(x, Wr, None, k)
    _, s1, _ = R.route(x, Wr, shift, k)
    assert not np.allclose(s0, s1, rtol=1e-6, atol=0)


def test_bias_select_only_selects_but_does_not_weigh():
    """Bare logits [0, 1, 2, 3], bias [10, 0, 0, 0]: the keys select expert 0 then 3;
    the weights come from the bare logits 0 and 3."""
    x, Wr = _exact_logits([0.0, 1.0, 2.0, 3.0])
    bias = np.array([10.0, 0.0, 0.0, 0.0], np.float32)
    sg = lambda z: 1.0 / (1.0 + np.exp(-z))
    ids, w, keys = R.route(x, Wr, bias, 2, bias_select_only=True)
    assert list(ids[0]) == [0, 3] and keys[0, 0] == 10.0
    assert np.allclose(w[0], [sg(0) / (sg(0) + sg(3)), sg(3) / (sg(0) + sg(3))], rtol=1e-15)
    ids, w, _ = R.route(x, Wr, bias, 2, score="softmax", bias_select_only=True)
    assert list(ids[0]) == [0, 3]
    assert np.allclose(w[0], [1 / (1 + np.e ** 3), np.e ** 3 / (1 + np.e ** 3)], rtol=1e-15)
    # with the bias in both, the selected expert 0 carries its key 10
    ids, w, _ = R.route(x, Wr, bias, 2)
    assert np.allclose(w[0], [sg(10) / (sg(10) + sg(3)), sg(3) / (sg(10) + sg(3))], rtol=1e-15)


def test_bias_select_only_with_zero_router_weighs_evenly():
    E, H = 8, 32
    Wr = np.zeros((E, H), np.float32)
    bias = np.zeros(E, np.float32)
    bias[5] = 3.0
    bias[1] = -1.0
    x = synth.to_bf16_bits(np.ones((1, H)))
    for score in ("sigmoid", "softmax"):
        ids, w, _ = R.route(x, Wr, bias, 2, score=score, bias_select_only=True)
        assert list(ids[0]) == [5, 0]
        assert np.all(w[0] == 0.5)
