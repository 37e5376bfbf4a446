"""Cluster scoring's approximate pass and exact re-scoring of candidates.

The selection is defined by the split-operand scores (bf16 hi/lo parts,
products hi*hi + hi*lo + lo*hi, fp32 accumulation).  The kernel scores every
cluster with one product (hi*hi), keeps the clusters within twice the error
bound of the prefilter threshold, and re-scores only those with the three
products; when a wave's candidates overflow it scores every cluster exactly.
Either way the top-k must be the exact one, so these tests compare the GPU's
selection with the top-k of the three-product scores emulated on the host (the
same bf16 splits, products summed in fp64), within a tie band of 1e-5 of
max|q| max|C| -- far below the one-product error (about 2^-7 of it), so a
candidate lost by the prefilter shows up.
"""
import numpy as np
import pytest
import torch

import hybrid_attention_prefill_amd as ha

pytestmark = pytest.mark.gpu
BAND = 1e-5


def bf16_rn(x):
    """fp32 -> nearest bf16 (ties to even), returned as fp32."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split(x):
    x = np.asarray(x, dtype=np.float32)
    hi = bf16_rn(x)
    lo = bf16_rn(x - hi)
    return hi.astype(np.float64), lo.astype(np.float64)


def scores3(q, C):
    qh, ql = split(q)
    ch, cl = split(C)
    return qh @ ch.T + qh @ cl.T + ql @ ch.T


def _run(N, M, topk, window, qlow, cent, assign, n_q_heads, n_kv_heads, group_select, blocks):
    """GPU selection vs the emulated exact top-k on the listed query blocks."""
    print(f"\n[case] select prefilter N={N} M={M} k={topk} w={window} gs={group_select}", flush=True)
    d = ha.make_desc(N, n_q_heads, n_kv_heads, 128, window=window, topk=topk, n_clusters=M, kmeans_iters=1,
                     kmeans_stride=N // M, group_select=group_select)
    kinds = [1] * n_q_heads
    off = np.zeros((n_kv_heads, M + 1), dtype=np.int32)
    mem = np.zeros((n_kv_heads, N), dtype=np.int32)
    first = np.full((n_kv_heads, M), np.iinfo(np.int64).max, dtype=np.int64)
    for g in range(n_kv_heads):
        off[g] = np.r_[0, np.cumsum(np.bincount(assign[g], minlength=M))]
        mem[g] = np.lexsort((np.arange(N), assign[g]))
        np.minimum.at(first[g], assign[g], np.arange(N))
    n_qb = (N + 63) // 64
    sel = torch.full((n_q_heads, n_qb, topk), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(ha.ha_workspace_bytes(d, kinds), dtype=torch.uint8, device="cuda")
    ha.ha_select_clusters(d, kinds, torch.from_numpy(qlow).cuda(), torch.from_numpy(cent).cuda(),
                          torch.from_numpy(off).cuda(), torch.from_numpy(mem).cuda(), sel, ws)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    G = n_q_heads // n_kv_heads
    units = [[h] for h in range(n_q_heads)] if not group_select else \
        [list(range(g * G, (g + 1) * G)) for g in range(n_kv_heads)]
    n_diff = 0
    for u in units:
        g = u[0] // G
        cn = np.sqrt((cent[g].astype(np.float64) ** 2).sum(1)).max()
        for b in blocks:
            r0, r1 = b * 64, min(N, b * 64 + 64)
            lim = r1 - 1 - window
            elig = np.nonzero(first[g] <= lim)[0]
            s = np.max([scores3(qlow[h, r0:r1], cent[g]).max(0) for h in u], axis=0)
            qn = max(np.sqrt((qlow[h, r0:r1].astype(np.float64) ** 2).sum(1)).max() for h in u)
            kk = min(topk, elig.size)
            for h in u:
                got = [int(x) for x in sel[h, b] if x >= 0]
                assert got == sorted(got) and len(set(got)) == len(got), f"unit {u} block {b}"
                assert len(got) == kk and all(x == -1 for x in sel[h, b][kk:]), f"unit {u} block {b}: {len(got)}"
                assert list(sel[h, b]) == list(sel[u[0], b]), f"unit {u} block {b}: slots differ"
            if kk == 0:
                continue
            es = s[elig]
            order = np.lexsort((elig, -es))
            tau = es[order[kk - 1]]
            ref = set(int(x) for x in elig[order[:kk]])
            sc = dict(zip((int(x) for x in elig), es))
            for c in ref.symmetric_difference(got):
                assert c in sc, f"unit {u} block {b}: cluster {c} not eligible"
                assert abs(sc[c] - tau) <= BAND * qn * cn, \
                    f"unit {u} block {b}: cluster {c} score {sc[c]:.9g} vs k-th {tau:.9g} (band {BAND * qn * cn:.3g})"
                n_diff += 1
    print(f"near-tie differences: {n_diff}")


def _blocks(N):
    n_qb = (N + 63) // 64
    rng = np.random.default_rng(1)
    return sorted(set([0, 1, n_qb // 2, n_qb - 2, n_qb - 1] + list(rng.choice(n_qb, 24, replace=False))))


@pytest.mark.parametrize("scale", [1.0, 1e15, 1e-15])
def test_prefilter_random_centroids(scale):
    # the 1M layer's cluster count and budget on a shorter sequence
    N, M, topk, window = 32768 - 17, 16384, 64, 512
    rng = np.random.default_rng(3)
    qlow = (rng.standard_normal((2, N, 16)) * 2 * scale).astype(np.float32)
    cent = (rng.standard_normal((1, M, 16)) * scale).astype(np.float32)
    assign = rng.integers(0, M, size=(1, N))
    _run(N, M, topk, window, qlow, cent, assign, 2, 1, 0, _blocks(N))


def test_prefilter_overflow_near_equal_centroids():
    # every centroid within 1e-4 of one vector: all eligible clusters are
    # candidates, the waves overflow and the block is scored exactly
    N, M, topk, window = 16384, 4096, 64, 256
    rng = np.random.default_rng(4)
    qlow = rng.standard_normal((2, N, 16)).astype(np.float32)
    c0 = rng.standard_normal(16)
    cent = (c0[None, None, :] + 1e-4 * rng.standard_normal((1, M, 16))).astype(np.float32)
    assign = rng.integers(0, M, size=(1, N))
    _run(N, M, topk, window, qlow, cent, assign, 2, 1, 0, _blocks(N))


def test_prefilter_group_units_and_few_eligible():
    # units of four slots (max over slots), short sequence, clusters of
    # uneven size (many late, so early blocks have few eligible clusters)
    N, M, topk, window = 8192 + 5, 1024, 48, 128
    rng = np.random.default_rng(5)
    qlow = rng.standard_normal((8, N, 16)).astype(np.float32)
    cent = rng.standard_normal((2, M, 16)).astype(np.float32)
    assign = np.minimum(M - 1, (rng.random((2, N)) ** 0.5 * M).astype(np.int64))
    _run(N, M, topk, window, qlow, cent, assign, 8, 2, 1, _blocks(N))


def test_prefilter_large_budget_takes_the_exact_path():
    # a budget above 128 skips the approximate pass
    N, M, topk, window = 8192, 2048, 200, 64
    rng = np.random.default_rng(6)
    qlow = rng.standard_normal((1, N, 16)).astype(np.float32)
    cent = rng.standard_normal((1, M, 16)).astype(np.float32)
    assign = rng.integers(0, M, size=(1, N))
    _run(N, M, topk, window, qlow, cent, assign, 1, 1, 0, _blocks(N))


@pytest.mark.parametrize("M,topk", [(50, 4), (64, 4), (700, 16), (1000, 64), (1056, 128), (33, 32)])
def test_prefilter_cluster_counts_off_the_tile_grid(M, topk):
    # cluster counts that leave a partial last tile and waves whose last
    # group of tiles runs past the end
    N, window = 4096 + 9, 200
    rng = np.random.default_rng(M)
    qlow = rng.standard_normal((2, N, 16)).astype(np.float32)
    cent = rng.standard_normal((1, M, 16)).astype(np.float32)
    assign = rng.integers(0, M, size=(1, N))
    _run(N, M, topk, window, qlow, cent, assign, 2, 1, 0, _blocks(N))
