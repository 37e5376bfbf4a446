"""The benchmark's exact work accounting (pairs per layer, keys gathered
outside the window) against key sets enumerated one row at a time from the
oracle's selections, on small layers (CPU only)."""
import numpy as np
import pytest

import bench
from oracle.prefill import layer_prefill
from synth.configs import Workload, HEAD_DENSE, HEAD_RETRIEVAL, HEAD_SWA, HEAD_TRIANGLE
from tests._util import oracle_arrays


def _enumerate(w, res):
    """(pairs, gathered keys) by brute force: every row's key set, and per
    (retrieval head, query block) the keys outside the window that some row
    of the block sees."""
    N, G = w.n_tokens, w.n_q_heads // w.n_kv_heads
    pairs = gathered = 0
    per_block = np.zeros(w.n_qb, dtype=np.int64)
    for h, k in enumerate(w.head_kind):
        for b in range(w.n_qb):
            rows = range(b * 64, min(N, (b + 1) * 64))
            far = set()
            for i in rows:
                for j in range(i + 1):
                    if k == HEAD_DENSE:
                        vis = True
                    elif k == HEAD_SWA:
                        vis = i - j < w.window
                    elif k == HEAD_TRIANGLE:
                        vis = j < w.sink or i - j < w.window or i >= N - w.last_q
                    else:
                        S = set(int(x) for x in res.sel[h][b])
                        chosen = (int(res.assign[h // G][j]) in S) if w.n_clusters else \
                            ((j // 64) in S or (w.force_block0 and j < 64))
                        vis = i - j < w.window or chosen
                        if chosen and i - j >= w.window:
                            far.add(j)
                    pairs += vis
                    per_block[b] += vis
            gathered += len(far)
    return pairs, gathered, per_block


@pytest.mark.parametrize("kw", [
    dict(head_kind=(HEAD_RETRIEVAL, HEAD_SWA, HEAD_TRIANGLE, HEAD_DENSE), window=70, topk=2, sink=5, last_q=30),
    dict(head_kind=(HEAD_RETRIEVAL,) * 4, window=40, topk=3, force_block0=1),
    dict(head_kind=(HEAD_RETRIEVAL,) * 4, window=50, topk=4, n_clusters=12, kmeans_iters=2, kmeans_stride=20),
])
def test_layer_work_matches_enumerated_key_sets(kw):
    w = Workload(name="acct", n_tokens=300, n_q_heads=4, n_kv_heads=2, head_dim=16, **kw)
    q, K, V, P, _, _ = oracle_arrays(w)
    res = layer_prefill(w, q, K, V, P)
    G = w.n_q_heads // w.n_kv_heads
    sel = np.full((len(w.ret_heads), w.n_qb, max(1, w.topk)), -1, dtype=np.int32)
    for t, h in enumerate(w.ret_heads):
        for b in range(w.n_qb):
            s = res.sel[h][b]
            sel[t, b, :len(s)] = s
    csr = None
    if w.n_clusters:
        off = np.stack([np.r_[0, np.cumsum(np.bincount(res.assign[g], minlength=w.n_clusters))]
                        for g in range(w.n_kv_heads)])
        mem = np.stack([np.lexsort((np.arange(w.n_tokens), res.assign[g])) for g in range(w.n_kv_heads)])
        csr = (off, mem)
    act, dense, ret_pairs, gathered = bench.layer_work(w, sel, csr)
    pairs, far, per_block = _enumerate(w, res)
    assert act == pairs
    assert gathered == far
    assert dense == w.n_q_heads * w.n_tokens * (w.n_tokens + 1) // 2
    # the CPU baseline's count for one sampled block matches the enumeration
    assign = res.assign if w.n_clusters else None
    for b in (0, 2, w.n_qb - 1):
        assert bench._oracle_block_pairs(w, b, res, assign) == per_block[b]


def test_eligible_block_pairs_matches_oracle_eligibility():
    from oracle.indexer import eligible_blocks
    for win, f0 in ((1, 0), (64, 1), (100, 0), (5000, 0)):
        w = Workload(name="e", n_tokens=1000, n_q_heads=1, n_kv_heads=1, head_kind=(HEAD_RETRIEVAL,),
                     window=win, force_block0=f0)
        ref = sum(eligible_blocks(min(1000, (b + 1) * 64) - 1, win, f0, 64).size for b in range(w.n_qb))
        assert bench.eligible_block_pairs(w) == ref
