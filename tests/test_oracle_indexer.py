"""Pins for the oracle's low-rank indexer and block / cluster selection."""
import json
import os

import numpy as np
import pytest

from oracle.indexer import (block_scores, eligible_blocks, eligible_clusters, project,
                            select_blocks, topk_order, cluster_scores)
from oracle.prefill import retrieval_key_set

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_projection_orientation_identity_columns():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((33, 128))
    P = np.zeros((128, 16))
    P[np.arange(16), np.arange(16)] = 1.0       # P = [e_0 .. e_15]
    np.testing.assert_array_equal(project(X, P), X[:, :16])
    # a permutation picks the permuted coordinates
    perm = rng.permutation(128)[:16]
    P2 = np.zeros((128, 16))
    P2[perm, np.arange(16)] = 1.0
    np.testing.assert_array_equal(project(X, P2), X[:, perm])


def test_block_selection_matches_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "blocksel_n8.json")))
    kl = np.array(g["klow"], float)[:, None]
    ql = np.array(g["qlow"], float)[:, None]
    N, Bq, Bk, w = g["N"], g["Bq"], g["Bk"], g["w"]
    for case in g["cases"]:
        sel, scored = select_blocks(ql, kl, N, w, Bq, Bk, case["k"], case["f0"])
        for b in range(N // Bq):
            E, s = scored[b]
            assert list(E) == case["eligible"][b]
            assert list(s) == case["scores"][b]
            assert list(sel[b]) == case["selected"][b]
            rows = np.arange(b * Bq, (b + 1) * Bq)
            keys, vis = retrieval_key_set(rows, w, Bk, case["f0"], blocks=sel[b])
            m = vis(rows, keys)
            for t, i in enumerate(rows):
                assert sorted(keys[m[t]].tolist()) == case["key_sets"][i], (case, i)


def test_block_scores_match_double_loop():
    rng = np.random.default_rng(5)
    N, Bk, r = 200, 16, 4
    ql = rng.standard_normal((N, r))
    kl = rng.standard_normal((N, r))
    rows = np.arange(96, 112)
    blocks = np.arange(0, 7)
    s = block_scores(ql[rows], rows, kl, blocks, Bk)
    for t, c in enumerate(blocks):
        best = -np.inf
        for i in rows:
            for j in range(c * Bk, (c + 1) * Bk):
                if j <= i:
                    best = max(best, sum(ql[i, d] * kl[j, d] for d in range(r)))
        assert abs(best - s[t]) < 1e-12


def test_topk_ties_keep_lower_index():
    # duplicated key blocks give exactly equal scores; the lower block wins
    rng = np.random.default_rng(2)
    Bk, r = 8, 4
    base = rng.standard_normal((Bk, r))
    kl = np.concatenate([rng.standard_normal((Bk, r)) * 0.1, base, rng.standard_normal((Bk, r)) * 0.1,
                         base, base, rng.standard_normal((3 * Bk, r)) * 0.1])
    ql = np.ones((kl.shape[0], r))
    rows = np.arange(kl.shape[0] - Bk, kl.shape[0])
    blocks = np.arange(0, 6)
    s = block_scores(ql[rows], rows, kl, blocks, Bk)
    assert s[1] == s[3] == s[4]
    assert list(topk_order(s, blocks, 1)) == [1]
    assert list(topk_order(s, blocks, 2)) == [1, 3]
    assert list(topk_order(s, blocks, 3)) == [1, 3, 4]
    # reversed presentation order does not change the answer
    assert list(topk_order(s[::-1], blocks[::-1], 2)) == [1, 3]


def test_topk_bounds():
    s = np.array([3.0, 1.0, 2.0])
    ids = np.array([4, 9, 2])
    assert list(topk_order(s, ids, 0)) == []
    assert list(topk_order(s, ids, 10)) == [2, 4, 9]
    assert list(topk_order(s, ids, 2)) == [2, 4]


def test_eligibility_covers_every_out_of_window_key():
    # every causal key outside the window of some row of block b lies in an
    # eligible block, so "top-k >= all eligible" reaches every key.
    N, Bq, Bk = 300, 16, 16
    for w in (1, 5, 16, 40, 299, 400):
        for f0 in (0, 1):
            for b in range((N + Bq - 1) // Bq):
                rows = np.arange(b * Bq, min(N, (b + 1) * Bq))
                E = set(eligible_blocks(int(rows[-1]), w, f0, Bk).tolist())
                need = {j // Bk for i in rows for j in range(0, i - w + 1)}
                if f0:
                    need -= {0}
                assert need <= E
                # and nothing needless: every eligible block has such a key
                for c in E:
                    assert c * Bk <= rows[-1] - w


def test_eligible_clusters_first_member_rule():
    a = np.array([3, 1, 1, 0, 2, 3, 2, 0])
    assert list(eligible_clusters(a, 4, qe=7, w=5)) == [1, 3]      # keys 0..2
    assert list(eligible_clusters(a, 4, qe=7, w=8)) == []
    assert list(eligible_clusters(a, 4, qe=7, w=1)) == [0, 1, 2, 3]


def test_cluster_scores_max_over_block_rows():
    ql = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, -1.0]])
    C = np.array([[2.0, 0.0], [0.0, 3.0], [-1.0, 0.5]])
    s = cluster_scores(ql, C, np.array([0, 1, 2]))
    np.testing.assert_array_equal(s, [2.0, 3.0, 0.5])
