"""Pins for GQA-group-shared selection in the oracle: a hand-worked two-head
layer whose per-head and group selections differ, in block and in cluster
mode, and the cases where the group choice must equal the per-head one."""
import numpy as np

import synth
from synth.configs import Workload, HEAD_RETRIEVAL, HEAD_SWA
from oracle.prefill import layer_prefill
from tests._util import oracle_arrays

D = 32
N = 256          # four query / key blocks of 64


def _fixture_arrays():
    """Two retrieval heads in one KV group.  P keeps the first 16 dims, every
    key of key block c is the unit vector e_c, and every query row of head A is
    (3, 1, 2, 0, ...), of head B (0, 5, 2.5, 0, ...).  For query block 3 (rows
    192..255, window 64) the eligible key blocks are 0, 1, 2 and the block
    scores are the query's coordinates:
        head A: (3, 1, 2)   -> its own top-2 = {0, 2}
        head B: (0, 5, 2.5) -> its own top-2 = {1, 2}
        group max (3, 5, 2.5) -> shared top-2 = {0, 1}
    (a sum (3, 6, 4.5) or mean over the heads would pick {1, 2})."""
    K = np.zeros((N, 1, D))
    for c in range(4):
        K[c * 64:(c + 1) * 64, 0, c] = 1.0
    V = np.zeros((N, 1, D))
    for c in range(4):
        V[c * 64:(c + 1) * 64, 0, 8 + c] = 1.0     # V reads back the key block
    Q = np.zeros((N, 2, D))
    Q[:, 0, :3] = (3.0, 1.0, 2.0)
    Q[:, 1, :3] = (0.0, 5.0, 2.5)
    P = np.zeros((1, D, 16))
    for r in range(16):
        P[0, r, r] = 1.0
    return (lambda a, b: Q[a:b]), K, V, P


def _w(**kw):
    return Workload(name="gsel", n_tokens=N, n_q_heads=2, n_kv_heads=1, head_dim=D,
                    head_kind=(HEAD_RETRIEVAL, HEAD_RETRIEVAL), window=64, topk=2, **kw)


def test_block_mode_hand_worked_selection():
    q, K, V, P = _fixture_arrays()
    per = layer_prefill(_w(), q, K, V, P)
    grp = layer_prefill(_w(group_select=1), q, K, V, P)
    assert list(per.sel[0][3]) == [0, 2]
    assert list(per.sel[1][3]) == [1, 2]
    assert list(grp.sel[0][3]) == [0, 1]
    assert list(grp.sel[1][3]) == [0, 1]
    # blocks 0..2 have at most two eligible key blocks: both modes keep all
    for b in range(3):
        assert list(per.sel[0][b]) == list(grp.sel[0][b])
    # the outputs follow the selections: row 255 of head A reads blocks
    # {0, 2} + window (block 3) per head, {0, 1} + window in group mode, so
    # the V coordinate of block 1 is zero in one and positive in the other
    r = list(per.rows).index(255)
    assert per.O[r, 0, 8 + 1] == 0.0 and grp.O[r, 0, 8 + 1] > 0.0
    assert per.O[r, 0, 8 + 2] > 0.0 and grp.O[r, 0, 8 + 2] == 0.0
    # and agree wherever the selections agree (query blocks 0..2)
    rows = [i for i, x in enumerate(per.rows) if x < 192]
    np.testing.assert_array_equal(per.O[rows], grp.O[rows])


def test_cluster_mode_hand_worked_selection():
    # clusters = the key blocks (cluster m = key block m, centroid e_m); the
    # eligibility test uses the first member (64 m <= qe - w) as block mode does
    q, K, V, P = _fixture_arrays()
    C = np.zeros((4, 16))
    for m in range(4):
        C[m, m] = 1.0
    assign = np.repeat(np.arange(4), 64)
    km = {0: (C, assign)}
    w = _w(n_clusters=4, kmeans_iters=1, kmeans_stride=64)
    per = layer_prefill(w, q, K, V, P, kmeans_override=km)
    grp = layer_prefill(w.with_(group_select=1), q, K, V, P, kmeans_override=km)
    assert list(per.sel[0][3]) == [0, 2]
    assert list(per.sel[1][3]) == [1, 2]
    assert list(grp.sel[0][3]) == [0, 1]
    assert list(grp.sel[1][3]) == [0, 1]


def test_one_retrieval_head_per_group_equals_per_head():
    # retrieval heads 0 and 4 sit in different KV groups (G = 4)
    kinds = tuple(HEAD_RETRIEVAL if h in (0, 4) else HEAD_SWA for h in range(8))
    w = Workload(name="g1", n_tokens=640, n_q_heads=8, n_kv_heads=2, head_dim=D, head_kind=kinds,
                 window=100, topk=3)
    q, K, V, P, _, _ = oracle_arrays(w)
    a = layer_prefill(w, q, K, V, P)
    b = layer_prefill(w.with_(group_select=1), q, K, V, P)
    np.testing.assert_array_equal(a.O, b.O)
    for h in (0, 4):
        for blk in a.sel[h]:
            np.testing.assert_array_equal(a.sel[h][blk], b.sel[h][blk])


def test_identical_queries_in_a_group_equal_per_head():
    # heads 0 and 1 (same KV group) get the same queries: the group max is the
    # head score, so both modes select alike
    w = Workload(name="g2", n_tokens=640, n_q_heads=4, n_kv_heads=2, head_dim=D,
                 head_kind=(HEAD_RETRIEVAL,) * 4, window=100, topk=3)
    q, K, V, P, _, _ = oracle_arrays(w)
    Q = q(0, w.n_tokens).copy()
    Q[:, 1] = Q[:, 0]
    Q[:, 3] = Q[:, 2]
    qq = lambda a, b: Q[a:b]
    a = layer_prefill(w, qq, K, V, P)
    b = layer_prefill(w.with_(group_select=1), qq, K, V, P)
    np.testing.assert_array_equal(a.O, b.O)


def test_group_selection_is_shared_and_scores_are_group_max():
    # every retrieval head of a group reports the same selection, and its
    # recorded scores are not below any single head's scores
    w = Workload(name="g3", n_tokens=640, n_q_heads=4, n_kv_heads=2, head_dim=D,
                 head_kind=(HEAD_RETRIEVAL,) * 4, window=100, topk=3, group_select=1)
    q, K, V, P, _, _ = oracle_arrays(w)
    g = layer_prefill(w, q, K, V, P)
    p = layer_prefill(w.with_(group_select=0), q, K, V, P)
    for blk in g.sel[0]:
        np.testing.assert_array_equal(g.sel[0][blk], g.sel[1][blk])
        np.testing.assert_array_equal(g.sel[2][blk], g.sel[3][blk])
        for h in range(4):
            E, s = g.scored[h][blk]
            Ep, sp = p.scored[h][blk]
            np.testing.assert_array_equal(E, Ep)
            assert np.all(s >= sp)
