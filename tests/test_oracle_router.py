"""Pins of the router oracle (oracle.router) against what the pages fix: the
group-limited selection of "Beam 1.0: Local RoPE, Global NoPE and Scalable
Softmax" (section "The surrounding model and serving boundary"), techfi24.com
("Architecture et mécanismes d'inférence") and news.hamidun.com (the MoE
paragraph). Hand-built cases where each plausible mistake changes the answer,
the reduction to a plain top-k, closed forms and invariants. CPU only."""
import math

import numpy as np
import pytest

from oracle import router as R


def _scores(groups):
    """float32 scores [1][256]: groups = {group: {slot: value}}, all others 0.01."""
    s = np.full((1, 256), 0.01, dtype=np.float32)
    for g, slots in groups.items():
        for j, v in slots.items():
            s[0, 32 * g + j] = v
    return s


ZERO_BIAS = np.zeros(256, dtype=np.float32)


def test_group_score_is_sum_of_two_largest():
    # group 0 holds the single largest score but a weak second; groups 1-4 two
    # strong ones. Top-2 sums: 1.09 vs 1.2 -> group 0 is dropped (a max rule
    # would keep it and choose expert 0 first).
    s = _scores({0: {0: 0.99, 1: 0.10}, 1: {0: 0.6, 1: 0.6}, 2: {0: 0.6, 1: 0.6}, 3: {0: 0.6, 1: 0.6},
                 4: {0: 0.6, 1: 0.6}})
    idx, w, kept = R.select(s, ZERO_BIAS)
    assert sorted(kept[0]) == [1, 2, 3, 4]
    assert 0 not in idx[0]
    assert sorted(idx[0]) == [32, 33, 64, 65, 96, 97, 128, 129]


def test_experts_outside_kept_groups_are_never_chosen():
    # group 7 holds the largest score of all, but its second score is small,
    # so its group score loses to four others; its top expert must not appear.
    s = _scores({7: {5: 0.95, 6: 0.05}, 0: {0: 0.5, 1: 0.5, 2: 0.3}, 1: {0: 0.5, 1: 0.5, 2: 0.3},
                 2: {0: 0.5, 1: 0.5, 2: 0.3}, 3: {0: 0.5, 1: 0.5, 2: 0.3}})
    idx, _, kept = R.select(s, ZERO_BIAS)
    assert 7 not in kept[0] and 32 * 7 + 5 not in idx[0]
    assert set(idx[0]) == {0, 1, 32, 33, 64, 65, 96, 97}


def test_bias_chooses_but_does_not_weigh():
    # Seven experts at 0.9 and experts 0 and 1 tied at 0.5 compete for eight
    # slots. Without a bias the tie goes to expert 0; a bias on expert 1 hands
    # it the slot, while its weight still uses the uncorrected 0.5.
    s = _scores({0: {0: 0.5, 1: 0.5, 2: 0.9, 3: 0.9, 4: 0.9, 5: 0.9, 6: 0.9, 7: 0.9, 8: 0.9}})
    idx0, _, _ = R.select(s, ZERO_BIAS)
    assert 0 in idx0[0] and 1 not in idx0[0]
    b = ZERO_BIAS.copy()
    b[1] = np.float32(0.25)
    idx, w, _ = R.select(s, b)
    assert 1 in idx[0] and 0 not in idx[0]
    assert list(idx[0]) == [2, 3, 4, 5, 6, 7, 8, 1]
    hi, lo = float(np.float32(0.9)), float(np.float32(0.5))
    assert w[0, 7] == pytest.approx(2.5 * lo / (7 * hi + lo), rel=1e-14)
    corrected = float(np.float32(0.5) + np.float32(0.25))
    assert not math.isclose(w[0, 7], 2.5 * corrected / (7 * hi + corrected), rel_tol=1e-3)


def test_weights_closed_form_and_sum():
    # four experts at 0.8 and four at 0.4 chosen: weights 2.5*0.8/4.8, 2.5*0.4/4.8
    s = _scores({0: {0: 0.8, 1: 0.8, 2: 0.4, 3: 0.4}, 1: {0: 0.8, 1: 0.8, 2: 0.4, 3: 0.4}})
    idx, w, _ = R.select(s, ZERO_BIAS)
    hi, lo = float(np.float32(0.8)), float(np.float32(0.4))
    assert list(idx[0]) == [0, 1, 32, 33, 2, 3, 34, 35]
    np.testing.assert_allclose(w[0, :4], 2.5 * hi / (4 * hi + 4 * lo), rtol=1e-14)
    np.testing.assert_allclose(w[0, 4:], 2.5 * lo / (4 * hi + 4 * lo), rtol=1e-14)
    assert w[0].sum() == pytest.approx(2.5, rel=1e-14)


def test_sigmoid_closed_forms_not_softmax():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -200.0])
    s = R.sigmoid_f32(z)
    assert s.dtype == np.float32
    assert list(s[:3]) == [0.5, 0.75, 0.25]
    assert s[3] == np.float32(1.0) and s[4] == np.float32(0.0)
    # a softmax would sum to one over the experts; sigmoid scores do not
    zz = np.linspace(-2, 2, 256)
    assert abs(float(R.sigmoid_f32(zz).sum()) - 128.0) < 1e-3


def test_ties_go_to_the_lower_index():
    s = np.full((1, 256), 0.5, dtype=np.float32)
    idx, w, kept = R.select(s, ZERO_BIAS)
    assert list(kept[0]) == [0, 1, 2, 3]
    assert list(idx[0]) == list(range(8))
    np.testing.assert_allclose(w[0], 2.5 / 8, rtol=1e-15)
    # equal group scores at the boundary: groups 3 and 6 tie for the fourth
    # place -> group 3 is kept
    s = _scores({0: {0: 0.9, 1: 0.9}, 1: {0: 0.9, 1: 0.9}, 2: {0: 0.9, 1: 0.9}, 3: {0: 0.7, 1: 0.7},
                 6: {0: 0.7, 1: 0.7}})
    _, _, kept = R.select(s, ZERO_BIAS)
    assert list(kept[0]) == [0, 1, 2, 3]


def test_four_groups_kept_not_more():
    # eight strong experts spread over eight groups: only four groups survive,
    # so the selection takes the second-best experts of the kept groups.
    groups = {g: {0: 0.9 - 0.01 * g, 1: 0.5 - 0.01 * g} for g in range(8)}
    s = _scores(groups)
    idx, _, kept = R.select(s, ZERO_BIAS)
    assert list(kept[0]) == [0, 1, 2, 3]
    assert set(idx[0]) == {0, 1, 32, 33, 64, 65, 96, 97}
    # keeping all eight groups would pick the eight 0.9-ish experts instead
    idx8, _, _ = R.select(s, ZERO_BIAS, topk_groups=8)
    assert set(idx8[0]) == {32 * g for g in range(8)}


def test_reduces_to_plain_top_k_with_every_group_kept():
    g = np.random.default_rng(5)
    for _ in range(20):
        # distinct logits 0.02 apart, so their float32 sigmoids stay distinct
        z = g.permutation(np.arange(256) * 0.02 - 2.56)[None, :]
        idx, w, _ = R.select(R.sigmoid_f32(z), ZERO_BIAS, topk_groups=8)
        want = np.argsort(-z[0])[:8]
        assert list(idx[0]) == list(want)
        sz = 1 / (1 + np.exp(-z[0, want]))
        np.testing.assert_allclose(w[0], 2.5 * sz / sz.sum(), rtol=1e-6)


def test_invariants_on_random_tokens():
    g = np.random.default_rng(9)
    s = R.sigmoid_f32(g.standard_normal((200, 256)) * 1.5)
    b = (g.standard_normal(256) * 0.05).astype(np.float32)
    idx, w, kept = R.select(s, b)
    for t in range(200):
        assert len(set(idx[t])) == 8
        assert set(int(e) // 32 for e in idx[t]) <= set(int(k) for k in kept[t])
        corr = s[t] + b
        c = corr[idx[t]]
        assert np.all(c[:-1] >= c[1:])                           # selection order
        others = [e for e in range(256) if e // 32 in set(kept[t]) and e not in set(idx[t])]
        assert corr[others].max() <= c.min()                      # the best inside kept groups
        gs = [np.sort(corr[32 * q:32 * q + 32])[-2:].sum(dtype=np.float32) for q in range(8)]
        dropped = [q for q in range(8) if q not in set(kept[t])]
        assert max(gs[q] for q in dropped) <= min(gs[q] for q in kept[t])
        assert w[t].sum() == pytest.approx(2.5, rel=1e-12)


def test_logits_are_exact_dot_products():
    # small integers: every product and sum is exact in float64
    x = np.array([[1.0, -2.0, 3.0, 0.5]], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = np.array([[1, 1, 1, 1], [2, 0, -1, 4], [0, 0, 0, 0]], dtype=np.float32)
    z = R.router_logits(bits, w)
    assert list(z[0]) == [2.5, 1.0, 0.0]
