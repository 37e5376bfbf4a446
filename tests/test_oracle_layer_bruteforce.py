"""Layer-level pins: the oracle's whole-layer output against an N x N brute
force written from the masks' definitions, and closed forms for the Orthros
scale-offset query.  Every pin has a planted-mistake counterpart that must
fail it (the mistake is planted in the oracle, on the CPU).

Definitions used by the brute force (key j visible to query row i):
  DENSE                 j <= i
  SWA(w)                j <= i and i - j < w
  TRIANGLE(sink, w, L)  j <= i and (j < sink or i - j < w or i >= N - L)
                        (36kr interview, TriangleMix introduction: streaming
                        region = sink keys + local band; last Q-K region)
  RETRIEVAL, block mode j <= i and (i - j < w or j // Bk in S_b or (f0 and j < Bk))
  RETRIEVAL, clusters   j <= i and (i - j < w or a_j in S_b)
                        (RTPurbo post: exact attention over the selected
                        candidates; the local window as for streaming heads)
S_b (the selection of the row's query block) is taken from the oracle's own
result: the selection is pinned separately; what is checked here is how the
layer assembles each row's key set from it.

Orthros (qingkeai "一个 Attention,两种工作模式", scale-offset design and
"Prefilling"): the output position p attends over keys 0..p with the query
q' = q * s + o.
"""
import math

import numpy as np
import pytest

import oracle.prefill as op
from oracle.prefill import layer_prefill, orthros_cross
from synth.configs import Workload, HEAD_DENSE, HEAD_RETRIEVAL, HEAD_SWA, HEAD_TRIANGLE
from tests._util import oracle_arrays


def _brute_row(q, K, V, keys, scale):
    """Softmax of one query over the listed keys, in pure Python."""
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q, K[j])) for j in keys]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    den = math.fsum(e)
    return np.array([math.fsum(e[t] * float(V[keys[t]][d]) for t in range(len(keys))) / den
                     for d in range(V.shape[1])])


def _visible(kind, i, j, N, w, sink=0, last=0, Bk=64, f0=0, S=(), assign=None):
    if j > i:
        return False
    if kind == HEAD_DENSE:
        return True
    if kind == HEAD_SWA:
        return i - j < w
    if kind == HEAD_TRIANGLE:
        return j < sink or i - j < w or i >= N - last
    if assign is not None:
        return i - j < w or int(assign[j]) in S
    return i - j < w or (j // Bk) in S or (f0 and j < Bk)


def _brute_layer(w, res, q, K, V):
    """O for every row and head of a small layer by brute force; retrieval
    heads use the oracle's selections res.sel."""
    N, Hq, Hkv = w.n_tokens, w.n_q_heads, w.n_kv_heads
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(w.head_dim)
    Q = q(0, N)
    out = np.zeros((N, Hq, w.head_dim))
    for h in range(Hq):
        g = h // G
        kind = w.head_kind[h]
        for i in range(N):
            S = ()
            assign = None
            if kind == HEAD_RETRIEVAL:
                S = set(int(x) for x in res.sel[h][i // w.q_block])
                if w.n_clusters:
                    assign = res.assign[g]
            keys = [j for j in range(N) if _visible(kind, i, j, N, w.window, w.sink, w.last_q, w.k_block,
                                                     w.force_block0, S, assign)]
            out[i, h] = _brute_row(Q[i, h], K[:, g], V[:, g], keys, sc)
    return out


def _layer(kinds, N=150, Hkv=2, D=16, **kw):
    return Workload(name="bf", n_tokens=N, n_q_heads=len(kinds), n_kv_heads=Hkv, head_dim=D,
                    head_kind=tuple(kinds), **kw)


CASES = {
    # windows shorter than a query block, so rows of one block see different
    # window starts; N not a multiple of the block
    "swa": _layer([HEAD_SWA] * 4, window=5, q_block=32, k_block=32),
    "dense": _layer([HEAD_DENSE] * 2, Hkv=1, q_block=32, k_block=32),
    # 0 < sink, 0 < L < N, w < N: middle rows need the sink keys, the last L
    # rows every key
    "triangle": _layer([HEAD_TRIANGLE] * 4, window=7, sink=3, last_q=20, q_block=32, k_block=32),
    "retrieval_blocks": _layer([HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_TRIANGLE], window=9, topk=2,
                               sink=2, last_q=11, q_block=16, k_block=16),
    "retrieval_blocks_f0": _layer([HEAD_RETRIEVAL] * 4, window=6, topk=1, force_block0=1,
                                  q_block=16, k_block=16),
    "retrieval_group": _layer([HEAD_RETRIEVAL] * 4, window=6, topk=2, group_select=1, q_block=16, k_block=16),
    "retrieval_clusters": _layer([HEAD_RETRIEVAL] * 4, N=128, window=10, topk=3, n_clusters=8,
                                 kmeans_iters=2, kmeans_stride=16, q_block=16, k_block=16),
}


def _max_err(w, **kw):
    q, K, V, P, xs, xo = oracle_arrays(w)
    res = layer_prefill(w, q, K, V, P, **kw)
    ref = _brute_layer(w, res, q, K, V)
    return float(np.max(np.abs(res.O - ref)))


@pytest.mark.parametrize("case", sorted(CASES))
def test_layer_matches_nxn_bruteforce(case):
    assert _max_err(CASES[case]) <= 1e-12


def test_triangle_case_exercises_every_region():
    # the brute-force case is only a pin if sink, band and last rows all matter
    w = CASES["triangle"]
    N = w.n_tokens
    mid = [i for i in range(N) if i - w.window >= w.sink and i < N - w.last_q]
    assert mid and w.last_q < N and w.window < N and w.sink > 0


def _bad_static_late(kind, r0, r1, N, w, sink, last):
    # planted: the band starts one key late
    if kind == HEAD_SWA:
        return np.arange(max(0, r0 - w + 2), r1, dtype=np.int64)
    if kind == HEAD_TRIANGLE and r1 <= N - last:
        return np.unique(np.r_[np.arange(0, min(sink, r1)), np.arange(max(0, r0 - w + 2), r1)]).astype(np.int64)
    return _good_static(kind, r0, r1, N, w, sink, last)


def _bad_static_no_sink(kind, r0, r1, N, w, sink, last):
    # planted: triangle rows outside the last region lose the sink keys
    if kind == HEAD_TRIANGLE and r1 <= N - last:
        return np.arange(max(0, r0 - w + 1), r1, dtype=np.int64)
    return _good_static(kind, r0, r1, N, w, sink, last)


_good_static = op.static_key_candidates


@pytest.mark.parametrize("bad,case", [(_bad_static_late, "swa"), (_bad_static_late, "triangle"),
                                      (_bad_static_no_sink, "triangle")])
def test_planted_static_range_mistakes_fail(monkeypatch, bad, case):
    monkeypatch.setattr(op, "static_key_candidates", bad)
    assert _max_err(CASES[case]) > 1e-3


_good_retrieval = op.retrieval_key_set


def _bad_retrieval_late(rows, w, Bk, f0, **kw):
    # planted: the window part starts one key late (rows whose window start is
    # r0 - w + 1 lose that key unless it was selected)
    keys, vis = _good_retrieval(rows, w, Bk, f0, **kw)
    lo = int(rows[0]) - w + 1

    def vis2(ri, kj):
        m = vis(ri, kj)
        return m & ~((kj[None, :] == lo) & (ri[:, None] == rows[0]))
    return keys, vis2


def _bad_retrieval_no_causal(rows, w, Bk, f0, **kw):
    # planted: selected keys taken without the causal test
    keys, vis = _good_retrieval(rows, w, Bk, f0, **kw)
    r1 = int(rows[-1]) + 1
    blocks = kw.get("blocks")
    extra = np.zeros(0, dtype=np.int64) if blocks is None else \
        np.concatenate([np.arange(c * Bk, (c + 1) * Bk) for c in blocks] + [np.zeros(0, np.int64)])
    extra = extra[extra < r1]
    keys2 = np.unique(np.r_[keys, extra]).astype(np.int64)

    def vis2(ri, kj):
        m = vis(ri, kj)
        return m | np.isin(kj // Bk, np.asarray(blocks if blocks is not None else [], np.int64))[None, :]
    return keys2, vis2


@pytest.mark.parametrize("bad,case", [(_bad_retrieval_late, "retrieval_blocks"),
                                      (_bad_retrieval_late, "retrieval_clusters"),
                                      (_bad_retrieval_no_causal, "retrieval_blocks_f0")])
def test_planted_retrieval_key_set_mistakes_fail(monkeypatch, bad, case):
    monkeypatch.setattr(op, "retrieval_key_set", bad)
    assert _max_err(CASES[case]) > 1e-3


# ---------------------------------------------------------------------------
# Orthros scale-offset query

def _hand_case():
    # q' = q * s + o = [1*3 - 1, 2*0.5 + 0] = [2, 1]; keys e0, e1 give scores
    # [2, 1] (scale 1), weights [e/(e+1), 1/(e+1)]; V rows [10, 0], [0, 20]
    q = np.array([1.0, 2.0])
    s = np.array([3.0, 0.5])
    o = np.array([-1.0, 0.0])
    K = np.eye(2)
    V = np.array([[10.0, 0.0], [0.0, 20.0]])
    e = math.e
    expect = np.array([10.0 * e / (e + 1.0), 20.0 / (e + 1.0)])
    return q, s, o, K, V, expect


def test_orthros_hand_worked_scale_offset():
    q, s, o, K, V, expect = _hand_case()
    np.testing.assert_allclose(orthros_cross(q, s, o, K, V, 1, 1.0), expect, rtol=0, atol=1e-13)
    # output position 0 sees key 0 only
    np.testing.assert_allclose(orthros_cross(q, s, o, K, V, 0, 1.0), V[0], atol=0)


def _bad_drop_offset(q, s, o, K, V, p, scale):
    return _good_cross(q, s, np.zeros_like(np.asarray(o, float)), K, V, p, scale)


def _bad_offset_before_scale(q, s, o, K, V, p, scale):
    # (q + o) * s instead of q * s + o
    qp = (np.asarray(q, float) + np.asarray(o, float)) * np.asarray(s, float)
    return _good_cross(qp, np.ones_like(qp), np.zeros_like(qp), K, V, p, scale)


_good_cross = op.orthros_cross


@pytest.mark.parametrize("bad", [_bad_drop_offset, _bad_offset_before_scale])
def test_planted_affine_mistakes_fail_hand_case(bad):
    q, s, o, K, V, expect = _hand_case()
    assert np.max(np.abs(bad(q, s, o, K, V, 1, 1.0) - expect)) > 0.1


def _orthros_layer():
    return Workload(name="xa", n_tokens=90, n_q_heads=4, n_kv_heads=2, head_dim=16, head_kind=(HEAD_SWA,) * 4,
                    window=8, n_out=5)


def _zero_query_pin_err():
    # Q = 0 makes q' = o: every output row is the softmax of scale * o_h . k_j
    # over keys 0..p, written out here in pure Python
    w = _orthros_layer()
    _, K, V, _, xs, xo = oracle_arrays(w)
    Qz = np.zeros((w.n_tokens, w.n_q_heads, w.head_dim))
    res = layer_prefill(w, lambda a, b: Qz[a:b], K, V, None, xs, xo)
    sc = 1.0 / math.sqrt(w.head_dim)
    err = 0.0
    for t in range(w.n_out):
        p = w.n_tokens - w.n_out + t
        for h in range(w.n_q_heads):
            g = h // 2
            ref = _brute_row(xo[h], K[:, g], V[:, g], list(range(p + 1)), sc)
            err = max(err, float(np.max(np.abs(res.O_out[t, h] - ref))))
    return err


def _double_scale_pin_err():
    # s = 2, o = 0: q' = 2q, i.e. the dense causal rows with twice the scale
    w = _orthros_layer()
    q, K, V, _, xs, xo = oracle_arrays(w)
    res = layer_prefill(w, q, K, V, None, 2.0 * np.ones_like(xs), np.zeros_like(xo))
    dense = layer_prefill(w.with_(head_kind=(HEAD_DENSE,) * 4, n_out=0), q, K, V,
                          scale=2.0 / math.sqrt(w.head_dim))
    return float(np.max(np.abs(res.O_out - dense.O[-w.n_out:])))


def test_orthros_zero_query_gives_offset_query():
    assert _zero_query_pin_err() <= 1e-12


def test_orthros_scale_two_is_dense_with_double_scale():
    assert _double_scale_pin_err() <= 1e-12


@pytest.mark.parametrize("bad", [_bad_drop_offset, _bad_offset_before_scale])
def test_planted_affine_mistakes_fail_layer_pins(monkeypatch, bad):
    monkeypatch.setattr(op, "orthros_cross", bad)
    assert max(_zero_query_pin_err(), _double_scale_pin_err()) > 1e-3
