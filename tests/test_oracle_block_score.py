"""Pins for the cheaper block scores of the oracle (block representatives):
a hand-worked layer where the three scores pick three different blocks, the
order max-pair >= mean and bound >= max-pair on fully causal blocks,
reductions when a block's keys are all equal, and brute force on tiny input."""
import numpy as np

from synth.configs import Workload, HEAD_RETRIEVAL, HEAD_SWA
from oracle.indexer import block_extremes, block_means, block_scores, block_scores_mean, block_scores_minmax
from oracle.prefill import layer_prefill
from tests._util import oracle_arrays

D = 32
N = 256


def _fixture():
    """One retrieval head, P keeps the first 16 dims.  Every query row is
    (1, -1, 0, ...).  Key blocks (dims 0 and 1 only):
        block 0: keys alternate (6, 0) and (0, 0)     -> max-pair 6,   mean 3,   bound 6
        block 1: every key (5.5, 0)                   -> 5.5,          5.5,      5.5
        block 2: keys alternate (5, 0) and (0, -5)    -> 5,            5,        10
    Query block 3 (rows 192..255, window 64) has eligible blocks 0, 1, 2, all
    keys causal for every row; top-1 picks block 0 / 1 / 2 by max-pair /
    mean / bound."""
    K = np.zeros((N, 1, D))
    K[0:64:2, 0, 0] = 6.0
    K[64:128, 0, 0] = 5.5
    K[128:192:2, 0, 0] = 5.0
    K[129:192:2, 0, 1] = -5.0
    K[192:, 0, 2] = 1.0
    V = np.zeros((N, 1, D))
    for c in range(4):
        V[c * 64:(c + 1) * 64, 0, 8 + c] = 1.0
    Q = np.zeros((N, 1, D))
    Q[:, 0, 0] = 1.0
    Q[:, 0, 1] = -1.0
    P = np.zeros((1, D, 16))
    for r in range(16):
        P[0, r, r] = 1.0
    return (lambda a, b: Q[a:b]), K, V, P


def _w(**kw):
    return Workload(name="bs", n_tokens=N, n_q_heads=1, n_kv_heads=1, head_dim=D,
                    head_kind=(HEAD_RETRIEVAL,), window=64, topk=1, **kw)


def test_hand_worked_three_scores_three_blocks():
    q, K, V, P = _fixture()
    want = {0: ([6.0, 5.5, 5.0], [0]), 1: ([3.0, 5.5, 5.0], [1]), 2: ([6.0, 5.5, 10.0], [2])}
    for mode, (scores, sel) in want.items():
        r = layer_prefill(_w(block_score=mode), q, K, V, P)
        E, s = r.scored[0][3]
        assert list(E) == [0, 1, 2]
        np.testing.assert_allclose(s, scores, atol=1e-12)
        assert list(r.sel[0][3]) == sel
        # the output of the last row reads the chosen block's V coordinate
        row = list(r.rows).index(255)
        assert r.O[row, 0, 8 + sel[0]] > 0.0
        assert all(r.O[row, 0, 8 + c] == 0.0 for c in range(3) if c != sel[0])


def test_score_order_on_causal_blocks():
    # window >= 2 blocks: every eligible block lies before every row of the
    # query block, so mean <= max-pair <= bound for every candidate
    w = Workload(name="o", n_tokens=1000, n_q_heads=4, n_kv_heads=2, head_dim=D,
                 head_kind=(HEAD_RETRIEVAL,) * 4, window=130, topk=3)
    q, K, V, P, _, _ = oracle_arrays(w)
    res = [layer_prefill(w.with_(block_score=m), q, K, V, P) for m in (0, 1, 2)]
    for h in range(4):
        for b in res[0].scored[h]:
            E, s0 = res[0].scored[h][b]
            _, s1 = res[1].scored[h][b]
            _, s2 = res[2].scored[h][b]
            assert np.all(s1 <= s0 + 1e-12) and np.all(s0 <= s2 + 1e-12)


def test_equal_keys_in_a_block_make_all_scores_equal():
    rng = np.random.default_rng(5)
    klow = np.repeat(rng.standard_normal((6, 16)), 64, axis=0)       # 6 blocks of equal keys
    ql = rng.standard_normal((64, 16))
    rows = np.arange(448, 512)
    E = np.arange(0, 6)
    s0 = block_scores(ql, rows, klow, E, 64)
    s1 = block_scores_mean(ql, block_means(klow, 64), E)
    kmax, kmin = block_extremes(klow, 64)
    s2 = block_scores_minmax(ql, kmax, kmin, E)
    np.testing.assert_allclose(s1, s0, atol=1e-12)
    np.testing.assert_allclose(s2, s0, atol=1e-12)


def test_brute_force_representatives_ragged_tail():
    rng = np.random.default_rng(6)
    N2, Bk = 150, 64                         # last block holds 22 keys
    klow = rng.standard_normal((N2, 16))
    ql = rng.standard_normal((5, 16))
    means = block_means(klow, Bk)
    kmax, kmin = block_extremes(klow, Bk)
    for c in range(3):
        keys = [j for j in range(N2) if j // Bk == c]
        m = [sum(klow[j][d] for j in keys) / len(keys) for d in range(16)]
        mx = [max(klow[j][d] for j in keys) for d in range(16)]
        mn = [min(klow[j][d] for j in keys) for d in range(16)]
        np.testing.assert_allclose(means[c], m, atol=1e-12)
        np.testing.assert_allclose(kmax[c], mx, atol=0)
        np.testing.assert_allclose(kmin[c], mn, atol=0)
        best_mean = max(sum(ql[i][d] * m[d] for d in range(16)) for i in range(5))
        best_bound = max(sum(max(ql[i][d] * mx[d], ql[i][d] * mn[d]) for d in range(16)) for i in range(5))
        np.testing.assert_allclose(block_scores_mean(ql, means, np.array([c]))[0], best_mean, atol=1e-12)
        np.testing.assert_allclose(block_scores_minmax(ql, kmax, kmin, np.array([c]))[0], best_bound, atol=1e-12)


def test_topk_all_is_dense_for_every_score():
    w = Workload(name="d", n_tokens=400, n_q_heads=2, n_kv_heads=1, head_dim=D,
                 head_kind=(HEAD_RETRIEVAL, HEAD_RETRIEVAL), window=50, topk=1000)
    q, K, V, P, _, _ = oracle_arrays(w)
    dense = layer_prefill(w.with_(head_kind=(3, 3)), q, K, V, P)
    for m in (1, 2):
        np.testing.assert_allclose(layer_prefill(w.with_(block_score=m), q, K, V, P).O, dense.O, atol=1e-12)


# ---------------------------------------------------------------------------
# 8-bit indexer keys

from oracle.indexer import dequantize_keys, quantize_keys_int8  # noqa: E402


def test_quantize_hand_worked_codes():
    # max |k| = 127 -> scale exactly 1: the codes are the keys rounded to
    # nearest with ties to even (0.5 -> 0, 1.5 -> 2, -2.5 -> -2)
    k = np.zeros((2, 16), dtype=np.float32)
    k[0, :6] = [127.0, -3.4, 2.6, 0.5, 1.5, -2.5]
    codes, s = quantize_keys_int8(k)
    assert s[0] == np.float32(1.0)
    assert list(codes[0, :6]) == [127, -3, 3, 0, 2, -2]
    assert s[1] == 0.0 and not codes[1].any()        # an all-zero key


def test_quantize_bounds_and_round_trip():
    rng = np.random.default_rng(7)
    k = (rng.standard_normal((500, 16)) * rng.uniform(0.01, 30, (500, 1))).astype(np.float32)
    codes, s = quantize_keys_int8(k)
    assert codes.dtype == np.int8 and np.abs(codes.astype(int)).max() <= 127
    assert np.all(np.abs(codes.astype(int)).max(axis=1) == 127)   # the largest component maps to +-127
    err = np.abs(dequantize_keys(codes, s) - k.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * 0.5000001 + 1e-12)


def test_int8_scores_use_the_dequantized_keys():
    # the layer's block scores with 8-bit keys are the max-pair scores of the
    # dequantized keys; exactly representable keys (scale 1) change nothing
    w = Workload(name="q8", n_tokens=512, n_q_heads=2, n_kv_heads=1, head_dim=D,
                 head_kind=(HEAD_RETRIEVAL, HEAD_SWA), window=64, topk=2)
    q, K, V, P, _, _ = oracle_arrays(w)
    r = layer_prefill(w.with_(index_bits=8), q, K, V, P)
    codes, s = r.kcodes[0]
    kq = dequantize_keys(codes, s)
    for b, (E, sc) in r.scored[0].items():
        rows = np.arange(b * 64, min(512, b * 64 + 64))
        np.testing.assert_allclose(sc, block_scores(r.qlow[0][b], rows, kq, E, 64), atol=1e-12)
    qf, Kf, Vf, Pf = _fixture()
    a = layer_prefill(_w(), qf, Kf, Vf, Pf)
    b8 = layer_prefill(_w(index_bits=8), qf, Kf, Vf, Pf)
    np.testing.assert_array_equal(a.O, b8.O)
