"""Pins for the oracle's masked softmax and static key sets (CPU only).

Each test checks the oracle against something other than itself: a pure-Python
brute force, a closed form, a hand-drawn mask picture from tests/golden, or an
invariant the pages' definitions imply.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.attention import softmax_attention, visible_dense, visible_swa, visible_triangle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _picture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c == "1" for c in line])
    return np.array(rows, dtype=bool)


def _brute(q, k, v, vis, scale):
    """Pure-Python softmax per row with math.exp / math.fsum."""
    n, m = vis.shape
    out = []
    for i in range(n):
        ss = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))
              for j in range(m) if vis[i, j]]
        js = [j for j in range(m) if vis[i, j]]
        mx = max(ss)
        e = [math.exp(s - mx) for s in ss]
        den = math.fsum(e)
        out.append([math.fsum(e[t] * float(v[js[t]][d]) for t in range(len(js))) / den
                    for d in range(v.shape[1])])
    return np.array(out)


@pytest.mark.parametrize("kind", ["dense", "swa", "triangle"])
def test_softmax_matches_pure_python_bruteforce(kind):
    rng = np.random.default_rng(7)
    N, D = 48, 8
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    i = np.arange(N)
    vis = {"dense": visible_dense(i, i), "swa": visible_swa(i, i, 5),
           "triangle": visible_triangle(i, i, N, 3, 4, 6)}[kind]
    o = softmax_attention(q, k, v, vis, 0.37)
    np.testing.assert_allclose(o, _brute(q, k, v, vis, 0.37), rtol=0, atol=1e-12)


def test_swa_picture_matches_golden():
    i = np.arange(8)
    np.testing.assert_array_equal(visible_swa(i, i, 3), _picture("swa_n8_w3.txt"))


def test_triangle_picture_matches_golden():
    i = np.arange(10)
    np.testing.assert_array_equal(visible_triangle(i, i, 10, 2, 3, 2),
                                  _picture("triangle_n10_s2_w3_l2.txt"))


def test_zero_query_gives_mean_over_key_set_and_one_hot_reads_weights():
    # Q = 0: every visible key has the same score, so o_i is the plain mean of
    # v_j over K(i).  With V = identity (N <= D) the output row is the weight row.
    N = 10
    i = np.arange(N)
    vis = _picture("triangle_n10_s2_w3_l2.txt")
    o = softmax_attention(np.zeros((N, 4)), np.ones((N, 4)), np.eye(N), vis, 1.0)
    expect = vis / vis.sum(1, keepdims=True)
    np.testing.assert_allclose(o, expect, atol=1e-15)
    assert set(np.nonzero(o[5] > 0)[0]) == {0, 1, 3, 4, 5}


def test_closed_form_weights_proportional_to_j_plus_one():
    # s_ij = ln(j+1) makes the weights proportional to (j+1); with v_j = j the
    # dense causal row i is sum (j+1) j / sum (j+1) = 2i/3 exactly.
    N = 30
    k = np.zeros((N, 2))
    k[:, 0] = np.log(np.arange(1, N + 1))
    q = np.zeros((N, 2))
    q[:, 0] = 1.0
    v = np.stack([np.arange(N, dtype=float), np.ones(N)], 1)
    i = np.arange(N)
    o = softmax_attention(q, k, v, visible_dense(i, i), 1.0)
    np.testing.assert_allclose(o[:, 0], 2.0 * i / 3.0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[:, 1], 1.0, rtol=1e-14)
    # window w=4 row 10: keys 7..10 -> sum (j+1)j / sum (j+1) as an exact fraction
    o4 = softmax_attention(q, k, v, visible_swa(i, i, 4), 1.0)
    fr = Fraction(sum((j + 1) * j for j in range(7, 11)), sum(j + 1 for j in range(7, 11)))
    assert abs(o4[10, 0] - float(fr)) < 1e-13


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    N = 64
    q, k = rng.standard_normal((N, 16)) * 3, rng.standard_normal((N, 16)) * 3
    i = np.arange(N)
    _, wgt = softmax_attention(q, k, np.zeros((N, 1)), visible_triangle(i, i, N, 4, 8, 5), 0.5,
                               return_weights=True)
    assert np.max(np.abs(wgt.sum(1) - 1.0)) <= 1e-12


def test_special_cases_reduce():
    N = 40
    i = np.arange(N)
    # w >= N: SWA is dense
    np.testing.assert_array_equal(visible_swa(i, i, N), visible_dense(i, i))
    np.testing.assert_array_equal(visible_swa(i, i, 10 * N), visible_dense(i, i))
    # triangle with L = N is dense; with sink = L = 0 it is SWA; with w >= N dense
    np.testing.assert_array_equal(visible_triangle(i, i, N, 3, 5, N), visible_dense(i, i))
    np.testing.assert_array_equal(visible_triangle(i, i, N, 0, 5, 0), visible_swa(i, i, 5))
    np.testing.assert_array_equal(visible_triangle(i, i, N, 4, N, 0), visible_dense(i, i))


def test_window_one_returns_own_value():
    rng = np.random.default_rng(1)
    N = 20
    q, k, v = (rng.standard_normal((N, 8)) for _ in range(3))
    i = np.arange(N)
    o = softmax_attention(q, k, v, visible_swa(i, i, 1), 0.3)
    np.testing.assert_allclose(o, v, atol=1e-15)


def test_planted_off_by_one_is_caught(monkeypatch):
    # A plausible mistake (window i-w <= j <= i, one key too many) must fail the
    # golden picture.
    def bad(rows, keys, w):
        d = rows[:, None] - keys[None, :]
        return (d >= 0) & (d <= w)
    i = np.arange(8)
    assert not np.array_equal(bad(i, i, 3), _picture("swa_n8_w3.txt"))
    # and a dropped causal test in the triangle mask
    def bad_tri(rows, keys, n, sink, w, last):
        d = rows[:, None] - keys[None, :]
        return (keys[None, :] < sink) | ((d >= 0) & (d < w)) | (rows[:, None] >= n - last)
    i = np.arange(10)
    assert not np.array_equal(bad_tri(i, i, 10, 2, 3, 2), _picture("triangle_n10_s2_w3_l2.txt"))


def test_planted_scale_error_is_caught():
    # the closed-form pin rejects a softmax that forgets the scale
    N = 12
    k = np.zeros((N, 2)); k[:, 0] = np.log(np.arange(1, N + 1))
    q = np.zeros((N, 2)); q[:, 0] = 2.0
    v = np.stack([np.arange(N, dtype=float), np.ones(N)], 1)
    i = np.arange(N)
    good = softmax_attention(q, k, v, visible_dense(i, i), 0.5)
    bad = softmax_attention(q, k, v, visible_dense(i, i), 1.0)
    np.testing.assert_allclose(good[:, 0], 2.0 * i / 3.0, atol=1e-12)
    assert np.max(np.abs(bad[:, 0] - 2.0 * i / 3.0)) > 0.1
