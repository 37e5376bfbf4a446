"""Pins for the oracle's Lloyd k-means of low-rank keys."""
import json
import os

import numpy as np

from oracle.kmeans import assign_step, kmeans_objective, lloyd, update_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_1d_iterations():
    g = json.load(open(os.path.join(GOLDEN, "kmeans_1d.json")))
    X = np.array(g["X"])
    C, a, hist = lloyd(X, g["M"], g["stride"], len(g["iters"]), keep_history=True)
    for t, it in enumerate(g["iters"]):
        Ct, at = hist[t]
        assert list(at) == it["assign"]
        np.testing.assert_allclose(Ct, it["centroids"], rtol=1e-15)


def test_every_key_its_own_centroid():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((50, 16))
    C, a, _ = lloyd(X, 50, 1, 3)
    np.testing.assert_array_equal(a, np.arange(50))
    np.testing.assert_array_equal(C, X)


def test_separated_blobs_known_labels():
    rng = np.random.default_rng(1)
    centers = np.array([[0.0] * 16, [50.0] * 16, [-50.0] + [0.0] * 15, [0.0] * 15 + [80.0]])
    # seeds every 4th key: interleave so that keys 0,4,8,12 come from the 4 blobs
    n_per = 25
    X = np.zeros((4 * n_per, 16))
    lab = np.zeros(4 * n_per, dtype=int)
    for t in range(4 * n_per):
        X[t] = centers[t % 4] + 0.1 * rng.standard_normal(16)
        lab[t] = t % 4
    # stride 1 seeds keys 0..3, one per blob
    C, a, _ = lloyd(X, 4, 1, 4)
    np.testing.assert_array_equal(a, lab)
    for m in range(4):
        np.testing.assert_allclose(C[m], X[lab == m].mean(0), rtol=1e-13)


def test_centroid_is_mean_of_members_and_empty_keeps_previous():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((40, 3))
    a = rng.integers(0, 5, 40)
    a[a == 3] = 4                      # cluster 3 empty
    C_prev = rng.standard_normal((5, 3))
    C = update_step(X, a, C_prev)
    for m in range(5):
        mem = [X[j] for j in range(40) if a[j] == m]
        if mem:
            expect = [sum(v[d] for v in mem) / len(mem) for d in range(3)]
            np.testing.assert_allclose(C[m], expect, rtol=1e-13, atol=1e-15)
        else:
            np.testing.assert_array_equal(C[m], C_prev[m])


def test_ties_go_to_lowest_centroid():
    X = np.array([[0.0, 0.0], [1.0, 1.0]])
    C = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]])   # x0 equidistant to all three
    assert assign_step(X, C)[0] == 0
    C2 = np.array([[5.0, 5.0], [0.0, 1.0], [1.0, 0.0]])
    assert assign_step(X, C2)[0] == 1


def test_objective_non_increasing():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((600, 16)) + rng.integers(0, 6, (600, 1)) * 0.7
    _, _, hist = lloyd(X, 30, 20, 8, keep_history=True)
    objs = []
    C = X[np.arange(30) * 20]
    for Ct, at in hist:
        objs.append(kmeans_objective(X, C, at))   # assignment step objective
        objs.append(kmeans_objective(X, Ct, at))  # after the update step
        C = Ct
    assert all(objs[t + 1] <= objs[t] + 1e-9 for t in range(len(objs) - 1))


def test_planted_update_bug_is_caught():
    # a centroid update that forgets to divide by the count fails the golden
    g = json.load(open(os.path.join(GOLDEN, "kmeans_1d.json")))
    X = np.array(g["X"])
    a = np.array(g["iters"][0]["assign"])
    sums = np.zeros((2, 1))
    np.add.at(sums, a, X)
    assert not np.allclose(sums, g["iters"][0]["centroids"])
    np.testing.assert_allclose(update_step(X, a, X[:2]), g["iters"][0]["centroids"], rtol=1e-15)
