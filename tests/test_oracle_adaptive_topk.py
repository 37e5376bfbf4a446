"""Pins for the adaptive top-k budget (a proposal: the RTPurboV2 article only
states that heads, lengths and queries need very different numbers of
tokens; the rule is: of the top-k candidates, keep the shortest prefix by
score whose softmax share within the k reaches the mass threshold)."""
import math

import numpy as np
import pytest

import oracle.indexer as oi
from oracle.indexer import topk_adaptive, topk_order
from oracle.prefill import layer_prefill
from synth.configs import Workload, HEAD_RETRIEVAL
from tests._util import oracle_arrays


def test_hand_worked_three_candidates():
    # budget k = 3 of four candidates: scores 3 (id 4), 2 (id 2), 1 (id 9) are
    # kept, 0.5 (id 7) is outside the budget.  Scale 1: weights 1, e^-1, e^-2;
    # shares 1/T, (1 + e^-1)/T, 1 with T = 1 + e^-1 + e^-2.
    s = np.array([3.0, 1.0, 2.0, 0.5])
    ids = np.array([4, 9, 2, 7])
    T = 1 + math.exp(-1) + math.exp(-2)
    share1, share2 = 1 / T, (1 + math.exp(-1)) / T
    assert abs(share1 - 0.665241) < 1e-6 and abs(share2 - 0.909969) < 1e-6
    assert list(topk_adaptive(s, ids, 3, 0.5, 1.0)) == [4]
    assert list(topk_adaptive(s, ids, 3, 0.66, 1.0)) == [4]
    assert list(topk_adaptive(s, ids, 3, 0.67, 1.0)) == [2, 4]
    assert list(topk_adaptive(s, ids, 3, 0.9, 1.0)) == [2, 4]
    assert list(topk_adaptive(s, ids, 3, 0.91, 1.0)) == [2, 4, 9]
    # scale 0 makes the shares uniform: 1/3, 2/3, 1
    assert list(topk_adaptive(s, ids, 3, 0.6, 0.0)) == [2, 4]


def test_mass_one_or_off_is_fixed_topk():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(200)
    ids = rng.permutation(1000)[:200]
    for k in (0, 1, 7, 64, 300):
        ref = topk_order(s, ids, k)
        for mass in (0.0, 1.0, 1.5):
            np.testing.assert_array_equal(topk_adaptive(s, ids, k, mass, 0.25), ref)


def test_equal_scores_keep_ceil_mass_times_k():
    ids = np.arange(10, 20)
    s = np.full(10, 2.5)
    for mass, n in ((0.05, 1), (0.35, 4), (0.55, 6), (0.99, 10)):
        assert list(topk_adaptive(s, ids, 10, mass, 1.0)) == list(range(10, 10 + n))
    # exactly reaching the threshold counts (shares r/4 are exact in binary)
    assert list(topk_adaptive(s[:4], ids[:4], 4, 0.5, 1.0)) == [10, 11]


def test_subset_of_budget_and_monotone_in_mass():
    rng = np.random.default_rng(9)
    for _ in range(20):
        s = rng.standard_normal(80) * 3
        ids = np.arange(80)
        full = set(topk_order(s, ids, 32).tolist())
        prev = set()
        for mass in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):
            cur = set(topk_adaptive(s, ids, 32, mass, 0.8).tolist())
            assert prev <= cur <= full
            assert len(cur) >= 1
            prev = cur


def test_dominant_score_keeps_one():
    s = np.array([0.0, 50.0, 1.0, 2.0])
    assert list(topk_adaptive(s, np.arange(4), 4, 0.999, 1.0)) == [1]


def _bad_all_eligible(scores, ids, k, mass, scale):
    # planted: the shares normalised over every eligible candidate, not the k
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -np.asarray(scores)))
    s = np.asarray(scores)[order]
    wts = np.exp(scale * (s - s[0]))
    share = np.cumsum(wts) / np.sum(wts)
    n = min(k, int(np.nonzero(share >= mass)[0][0]) + 1)
    return np.sort(ids[order[:n]])


def _bad_strict(scores, ids, k, mass, scale):
    # planted: the prefix must exceed the mass instead of reaching it
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -np.asarray(scores)))[:k]
    s = np.asarray(scores)[order]
    wts = np.exp(scale * (s - s[0]))
    share = np.cumsum(wts) / np.sum(wts)
    hits = np.nonzero(share > mass)[0]
    n = int(hits[0]) + 1 if hits.size else order.size
    return np.sort(ids[order[:n]])


@pytest.mark.parametrize("bad", [_bad_all_eligible, _bad_strict])
def test_planted_mistakes_fail_the_pins(bad):
    s = np.array([3.0, 1.0, 2.0, 0.5])
    ids = np.array([4, 9, 2, 7])
    eq = np.full(4, 2.5)
    failed = (list(bad(s, ids, 3, 0.9, 1.0)) != [2, 4]
              or list(bad(eq, np.arange(10, 14), 4, 0.5, 1.0)) != [10, 11])
    assert failed


def _layer(**kw):
    return Workload(name="ad", n_tokens=600, n_q_heads=4, n_kv_heads=2, head_dim=32,
                    head_kind=(HEAD_RETRIEVAL,) * 4, window=64, topk=6, q_block=32, k_block=32, **kw)


@pytest.mark.parametrize("extra", [dict(), dict(group_select=1),
                                   dict(n_clusters=20, kmeans_iters=2, kmeans_stride=30)])
def test_layer_adaptive_selection_is_a_prefix_of_the_fixed_one(extra):
    w = _layer(**extra)
    q, K, V, P, _, _ = oracle_arrays(w)
    fixed = layer_prefill(w, q, K, V, P)
    one = layer_prefill(w.with_(topk_mass=1.0), q, K, V, P)
    np.testing.assert_array_equal(one.O, fixed.O)          # mass 1 = fixed top-k
    ad = layer_prefill(w.with_(topk_mass=0.5, mass_scale=2.0), q, K, V, P)
    sizes = []
    for h in w.ret_heads:
        for b, S in ad.sel[h].items():
            F = fixed.sel[h][b]
            assert set(S.tolist()) <= set(F.tolist())
            E, sc = ad.scored[h][b]
            np.testing.assert_array_equal(S, topk_adaptive(sc, E, w.topk, 0.5, 2.0))
            sizes.append(len(S))
    assert min(sizes) < max(sizes)       # the budget adapts across heads and blocks


def test_layer_default_mass_scale_is_inverse_sqrt_rank(monkeypatch):
    w = _layer(topk_mass=0.6)
    q, K, V, P, _, _ = oracle_arrays(w)
    seen = []
    real = oi.topk_adaptive

    def spy(scores, ids, k, mass, scale):
        seen.append(scale)
        return real(scores, ids, k, mass, scale)
    import oracle.prefill as op
    monkeypatch.setattr(op, "topk_adaptive", spy)
    layer_prefill(w, q, K, V, P, blocks=[5])
    assert seen and all(abs(x - 0.25) < 1e-15 for x in seen)
