"""Layer-level pins for the oracle: special cases that reduce to dense or SWA
attention, Orthros' identity scale-offset, and discrimination checks."""
import numpy as np
import pytest

import synth
from synth.configs import Workload, HEAD_DENSE, HEAD_RETRIEVAL, HEAD_SWA, HEAD_TRIANGLE
from oracle.prefill import layer_prefill
from tests._util import oracle_arrays


def _w(kind, N=320, Hq=4, Hkv=2, D=32, **kw):
    return Workload(name="t", n_tokens=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                    head_kind=(kind,) * Hq, **kw)


def _run(w, **kw):
    q, K, V, P, xs, xo = oracle_arrays(w)
    return layer_prefill(w, q, K, V, P, xs, xo, **kw)


def test_retrieval_topk_all_is_dense():
    w = _w(HEAD_RETRIEVAL, window=40, topk=1000, q_block=32, k_block=32)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4))
    r = _run(w)
    np.testing.assert_allclose(r.O, d.O, atol=1e-12)


def test_retrieval_topk_all_with_block0_is_dense():
    w = _w(HEAD_RETRIEVAL, window=70, topk=1000, force_block0=1, q_block=32, k_block=32)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4))
    np.testing.assert_allclose(_run(w).O, d.O, atol=1e-12)


def test_retrieval_topk_zero_is_swa():
    w = _w(HEAD_RETRIEVAL, window=40, topk=0, q_block=32, k_block=32)
    s = _run(w.with_(head_kind=(HEAD_SWA,) * 4))
    np.testing.assert_allclose(_run(w).O, s.O, atol=1e-12)


def test_retrieval_topk_zero_block0_is_swa_plus_block0():
    w = _w(HEAD_RETRIEVAL, window=40, topk=0, force_block0=1, q_block=32, k_block=32)
    q, K, V, P, _, _ = oracle_arrays(w)
    r = layer_prefill(w, q, K, V, P)
    # reference: explicit key sets {i-w < j <= i} U {j < 32, j <= i}, per row
    from oracle.attention import softmax_attention
    Q = q(0, w.n_tokens)
    for h in range(4):
        g = h // 2
        for i in (0, 31, 32, 100, 319):
            ks = sorted(set(range(max(0, i - 39), i + 1)) | set(range(0, min(32, i + 1))))
            o = softmax_attention(Q[i:i + 1, h], K[ks, g], V[ks, g], np.ones((1, len(ks)), bool),
                                  1 / np.sqrt(32))
            np.testing.assert_allclose(r.O[i, h], o[0], atol=1e-12)


def test_retrieval_window_covering_all_is_dense():
    w = _w(HEAD_RETRIEVAL, window=400, topk=3, q_block=32, k_block=32)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4))
    np.testing.assert_allclose(_run(w).O, d.O, atol=1e-12)


def test_cluster_mode_every_key_a_cluster_topk_all_is_dense():
    w = _w(HEAD_RETRIEVAL, N=192, window=30, topk=10000, n_clusters=192, kmeans_iters=2,
           kmeans_stride=1, q_block=32, k_block=32)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4, n_clusters=0))
    r = _run(w)
    np.testing.assert_array_equal(r.assign[0], np.arange(192))
    np.testing.assert_allclose(r.O, d.O, atol=1e-12)


def test_cluster_mode_topk_zero_is_swa():
    w = _w(HEAD_RETRIEVAL, N=256, window=30, topk=0, n_clusters=16, kmeans_iters=2,
           kmeans_stride=16, q_block=32, k_block=32)
    s = _run(w.with_(head_kind=(HEAD_SWA,) * 4, n_clusters=0))
    np.testing.assert_allclose(_run(w).O, s.O, atol=1e-12)


def test_triangle_reductions_at_layer_level():
    w = _w(HEAD_TRIANGLE, window=50, sink=16, last_q=320)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4))
    np.testing.assert_allclose(_run(w).O, d.O, atol=1e-12)
    w2 = _w(HEAD_TRIANGLE, window=50, sink=0, last_q=0)
    s = _run(w2.with_(head_kind=(HEAD_SWA,) * 4))
    np.testing.assert_allclose(_run(w2).O, s.O, atol=1e-12)


def test_swa_window_at_least_n_is_dense():
    w = _w(HEAD_SWA, window=320)
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4))
    np.testing.assert_allclose(_run(w).O, d.O, atol=1e-12)


def test_orthros_identity_affine_is_dense_last_row():
    w = _w(HEAD_SWA, window=16, n_out=1)
    q, K, V, P, xs, xo = oracle_arrays(w)
    r = layer_prefill(w, q, K, V, None, np.ones_like(xs), np.zeros_like(xo))
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4, n_out=0))
    np.testing.assert_allclose(r.O_out[0], d.O[-1], atol=1e-12)
    # and with the drawn affine the output differs (the affine matters)
    r2 = layer_prefill(w, q, K, V, None, xs, xo)
    assert np.max(np.abs(r2.O_out[0] - d.O[-1])) > 1e-3


def test_orthros_every_position_identity_affine_is_dense():
    # pre-training: every position is an output position; with s = 1, o = 0
    # each cross-attention row is the dense causal row
    w = _w(HEAD_SWA, N=200, window=16, n_out=200)
    q, K, V, P, xs, xo = oracle_arrays(w)
    r = layer_prefill(w, q, K, V, None, np.ones_like(xs), np.zeros_like(xo))
    d = _run(w.with_(head_kind=(HEAD_DENSE,) * 4, n_out=0))
    np.testing.assert_allclose(r.O_out, d.O, atol=1e-12)
    # output position t is row N - n_out + t: a suffix of the rows
    w2 = w.with_(n_out=37)
    r2 = layer_prefill(w2, q, K, V, None, np.ones_like(xs), np.zeros_like(xo))
    np.testing.assert_allclose(r2.O_out, d.O[-37:], atol=1e-12)


def test_orthros_out_rows_subset_equals_full():
    w = _w(HEAD_SWA, N=150, window=16, n_out=40)
    full = _run(w)
    part = _run(w, out_rows=[0, 17, 39])
    assert list(part.out_rows) == [0, 17, 39]
    np.testing.assert_allclose(part.O_out, full.O_out[[0, 17, 39]], atol=0)


def test_blocks_subset_equals_full_rows():
    w = _w(HEAD_RETRIEVAL, window=40, topk=2, q_block=32, k_block=32)
    full = _run(w)
    part = _run(w, blocks=[3, 7])
    rows = np.r_[96:128, 224:256]
    np.testing.assert_allclose(part.O, full.O[rows], atol=0)


def test_needle_rows_differ_from_swa_only():
    # discrimination: on a needle row the retrieval output is far from the
    # SWA-only output, so the output tolerances reject a path that drops selection
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, 8192, n_clusters=128, window=512, n_needles=4)
    w = w.with_(kmeans_stride=64)
    q, K, V, P, _, _ = oracle_arrays(w)
    nd = synth.inputs.needles(w)
    blocks = sorted({int(r) // 64 for r in nd.q_row})
    r = layer_prefill(w, q, K, V, P, blocks=blocks)
    s = layer_prefill(w.with_(head_kind=(HEAD_SWA,) * 16, n_clusters=0), q, K, V, None, blocks=blocks)
    diffs = []
    for n in range(nd.q_row.size):
        i, h = int(nd.q_row[n]), int(nd.q_head[n])
        t = int(np.nonzero(r.rows == i)[0][0])
        diffs.append(np.max(np.abs(r.O[t, h] - s.O[t, h])))
    assert max(diffs) > 0.5
