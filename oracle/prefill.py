"""One attention layer's prefill, head by head, in fp64.

Head roles follow [RTPurboV2] (retrieval vs streaming heads, ~15% / ~85%) and
the all-sparse case where every head is a retrieval head; the static masks
follow [TriangleMix] and [Orthros].

Retrieval head h, query block b (rows R_b):
  K(i) = SWA(w)(i)  U  {j <= i : block(j) in S_b}  U  (f0 ? {j <= i : j < Bk} : {})
  (cluster mode: {j <= i : a_j in S_b} in place of the block term)
With group-shared selection ([TriangleMix] interview, GQA answer: the queries
of one GQA group share the same keys, and sharing work across the group is
the usual practice), S_b is chosen once per (KV head, query block) from the
group score max over the group's retrieval heads of the head scores, and
every retrieval head of the group uses it.  Block mode scores candidates by
the max over causal (query, key) pairs, or, with `block_score` 1 / 2, by the
block's mean key / the bound from its per-dimension key extremes
(oracle.indexer).
[RTPurbo]: exact softmax over the selected candidates in full dimension, with
the local window of the head's own neighbourhood.

Orthros, output positions p in [N - n_out, N):
  q'_{h,p} = q_{h,p} * s_h + o_h   (elementwise, per head; [Orthros] "Scale-Offset"
  separates the cross-attention query from the SWA query that shares weights)
  O_out[p, h] = attention of q' over keys {0..p}   ("Prefilling" section: only
  the last prompt token runs full cross-attention over the whole KV).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Sequence

import numpy as np

from .attention import attend_rows, softmax_attention, visible_dense, visible_swa, visible_triangle
from .indexer import (block_extremes, block_means, block_scores, block_scores_mean, block_scores_minmax,
                      cluster_scores, dequantize_keys, eligible_blocks, eligible_clusters, project,
                      quantize_keys_int8, topk_adaptive, topk_order)
from .kmeans import lloyd

SWA, RETRIEVAL, TRIANGLE, DENSE = 0, 1, 2, 3


def head_group(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads KV head h // (Hq / Hkv) (consecutive GQA groups)."""
    return h // (Hq // Hkv)


def static_key_candidates(kind: int, r0: int, r1: int, N: int, w: int, sink: int, last: int) -> np.ndarray:
    """Key ids that can be visible to some query row in [r0, r1) under a static
    mask (a superset of each row's key set; the exact mask is applied on top):
      DENSE     0 .. r1-1
      SWA(w)    r0-w+1 .. r1-1 (clipped at 0)
      TRIANGLE  rows reaching the last L rows: 0 .. r1-1; otherwise the sink
                keys 0 .. sink-1 and the band r0-w+1 .. r1-1.
    Pinned by a layer-level N x N brute force against the masks' definitions
    (tests/test_oracle_prefill.py)."""
    if kind == DENSE or (kind == TRIANGLE and r1 > N - last):
        return np.arange(0, r1, dtype=np.int64)
    band = np.arange(max(0, r0 - w + 1), r1, dtype=np.int64)
    if kind == SWA:
        return band
    if kind == TRIANGLE:
        return np.unique(np.r_[np.arange(0, min(sink, r1), dtype=np.int64), band])
    raise ValueError(f"no static key set for head kind {kind}")


def retrieval_key_set(rows: np.ndarray, w: int, Bk: int, f0: int, *,
                      blocks: Optional[np.ndarray] = None,
                      clusters: Optional[np.ndarray] = None,
                      assign: Optional[np.ndarray] = None,
                      n_clusters: int = 0):
    """Candidate key ids and the exact visibility predicate for a retrieval
    head's query block (window  U  selected blocks or clusters  U  block 0)."""
    r0, r1 = int(rows[0]), int(rows[-1]) + 1
    parts = [np.arange(max(0, r0 - w + 1), r1, dtype=np.int64)]
    if blocks is not None:
        for c in blocks:
            parts.append(np.arange(c * Bk, min(r1, (c + 1) * Bk), dtype=np.int64))
    if f0:
        parts.append(np.arange(0, min(r1, Bk), dtype=np.int64))
    sel_mask = None
    if clusters is not None:
        sel_mask = np.zeros(max(n_clusters, int(assign.max()) + 1 if assign.size else 1), dtype=bool)
        if clusters.size:
            sel_mask[clusters] = True
        members = np.nonzero(sel_mask[assign[:r1]])[0].astype(np.int64)
        parts.append(members)
    keys = np.unique(np.concatenate(parts))
    blockset = np.zeros(0, dtype=np.int64) if blocks is None else np.asarray(blocks, dtype=np.int64)

    def visible(ri, kj):
        win = visible_swa(ri, kj, w)
        causal = kj[None, :] <= ri[:, None]
        chosen = np.isin(kj // Bk, blockset)
        if f0:
            chosen = chosen | (kj < Bk)
        if clusters is not None:
            chosen = chosen | sel_mask[assign[kj]]
        return win | (causal & chosen[None, :])

    return keys, visible


@dataclasses.dataclass
class OracleResult:
    rows: np.ndarray                       # query rows computed, ascending
    O: np.ndarray                          # [len(rows), Hq, D] fp64
    O_out: Optional[np.ndarray]            # [len(out_rows), Hq, D] fp64
    sel: Dict[int, Dict[int, np.ndarray]]  # head -> query block -> selected ids
    scored: Dict[int, Dict[int, tuple]]    # head -> block -> (eligible ids, scores)
    klow: Dict[int, np.ndarray]            # KV head -> [N, r]
    qlow: Dict[int, Dict[int, np.ndarray]]  # head -> block -> [rows, r]
    centroids: Dict[int, np.ndarray]
    assign: Dict[int, np.ndarray]
    out_rows: Optional[np.ndarray] = None  # output positions t (row N - n_out + t) held in O_out
    kcodes: Optional[Dict[int, tuple]] = None  # 8-bit indexer: KV head -> (codes, scales)


def orthros_cross(q: np.ndarray, s: np.ndarray, o: np.ndarray, K: np.ndarray,
                  V: np.ndarray, p: int, scale: float) -> np.ndarray:
    """Cross-attention of the scale-offset query at output position p over
    keys {0..p}.  Pinned: s = 1, o = 0 gives the dense causal row p; a
    hand-worked two-key case; Q = 0 gives the softmax of o over the keys; s = 2,
    o = 0 gives the dense row at twice the scale (planted "q * s" and
    "(q + o) * s" fail these)."""
    qp = np.asarray(q, np.float64) * np.asarray(s, np.float64) + np.asarray(o, np.float64)
    keys = np.arange(p + 1)
    vis = np.ones((1, p + 1), dtype=bool)
    return softmax_attention(qp[None, :], K[keys], V[keys], vis, scale)[0]


def layer_prefill(w, q_rows: Callable[[int, int], np.ndarray], K: np.ndarray, V: np.ndarray,
                  P: Optional[np.ndarray] = None, xa_scale=None, xa_offset=None, *,
                  blocks: Optional[Sequence[int]] = None,
                  heads: Optional[Sequence[int]] = None,
                  sel_override: Optional[Dict[int, Dict[int, np.ndarray]]] = None,
                  kmeans_override: Optional[Dict[int, tuple]] = None,
                  klow32_override: Optional[Dict[int, np.ndarray]] = None,
                  scale: Optional[float] = None,
                  with_out: bool = True,
                  out_rows: Optional[Sequence[int]] = None) -> OracleResult:
    """Oracle output of one layer.

    w          a ``synth.Workload`` (sizes, head roles, parameters)
    q_rows     (r0, r1) -> Q rows [r1-r0, Hq, D] as fp64
    K, V       [N, Hkv, D] fp64
    P          [Hkv, D, r] indexer projection (retrieval heads only)
    blocks     query blocks to compute (default: all)
    sel_override  head -> block -> selection to use instead of the oracle's own
                  (to grade attention given a validated GPU selection)
    kmeans_override  KV head -> (centroids, assign) to use instead of Lloyd
    klow32_override  8-bit indexer: KV head -> fp32 low-rank keys to quantize
                  (the GPU's, so the float-to-integer step is taken on the same
                  fp32 values); default: the oracle's keys rounded to fp32
    out_rows   Orthros output positions t in [0, n_out) to compute (default: all)
    """
    N, Hq, Hkv, D = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
    Bq, Bk = w.q_block, w.k_block
    n_qb = (N + Bq - 1) // Bq
    sc = (1.0 / np.sqrt(D)) if scale is None else scale
    blocks = list(range(n_qb)) if blocks is None else sorted(set(int(b) for b in blocks))
    heads = list(range(Hq)) if heads is None else list(heads)
    rows_all = np.concatenate([np.arange(b * Bq, min(N, (b + 1) * Bq)) for b in blocks]) \
        if blocks else np.zeros(0, dtype=np.int64)
    O = np.zeros((rows_all.size, Hq, D), dtype=np.float64)
    res = OracleResult(rows_all, O, None, {}, {}, {}, {}, {}, {})

    ret = [h for h in heads if w.head_kind[h] == RETRIEVAL]
    rep_klow = {}        # 8-bit indexer: dequantized keys used for block scores
    for g in sorted({head_group(h, Hq, Hkv) for h in ret}):
        res.klow[g] = project(K[:, g], P[g])
        if w.n_clusters > 0:
            if kmeans_override is not None and g in kmeans_override:
                C, a = kmeans_override[g]
                C = np.asarray(C, np.float64)
                a = np.asarray(a, np.int64)
            else:
                C, a, _ = lloyd(res.klow[g], w.n_clusters, w.kmeans_stride, w.kmeans_iters)
            res.centroids[g], res.assign[g] = C, a
        elif w.index_bits == 8:
            k32 = (klow32_override[g] if klow32_override is not None and g in klow32_override
                   else res.klow[g].astype(np.float32))
            codes, s = quantize_keys_int8(k32)
            if res.kcodes is None:
                res.kcodes = {}
            res.kcodes[g] = (codes, s)
            rep_klow[g] = dequantize_keys(codes, s)

    def choose(scores, E):
        """The selection S_b from the eligible candidates' scores: fixed top-k,
        or the adaptive budget (topk_mass > 0) with the indexer softmax scale
        mass_scale (<= 0: 1/sqrt(r), the scaled dot product of the rank-r
        space)."""
        if w.topk_mass > 0:
            ms = w.mass_scale if w.mass_scale > 0 else 1.0 / np.sqrt(w.rank)
            return topk_adaptive(scores, E, w.topk, w.topk_mass, ms)
        return topk_order(scores, E, w.topk)

    eligible_memo = {}   # (KV head, block) -> eligible clusters (shared by the group's heads)
    group_memo = {}      # (KV head, block) -> (eligible, group scores, selection)
    rep_memo = {}        # block representatives per KV head
    ret_of_group = {}
    for hh in range(Hq):   # all of a group's retrieval heads, even outside `heads`
        if w.head_kind[hh] == RETRIEVAL:
            ret_of_group.setdefault(head_group(hh, Hq, Hkv), []).append(hh)

    def scores_for(hh, g, b, Qb, rows, qe):
        """(eligible ids, scores) of retrieval head hh for query block b."""
        ql = project(Qb[:, hh], P[g])
        if w.n_clusters > 0:
            C, a = res.centroids[g], res.assign[g]
            if (g, b) not in eligible_memo:
                eligible_memo[(g, b)] = eligible_clusters(a, C.shape[0], qe, w.window)
            E = eligible_memo[(g, b)]
            return ql, E, cluster_scores(ql, C, E)
        E = eligible_blocks(qe, w.window, w.force_block0, Bk)
        if not E.size:
            return ql, E, np.zeros(0)
        if w.block_score == 1:
            if ("mean", g) not in rep_memo:
                rep_memo[("mean", g)] = block_means(res.klow[g], Bk)
            return ql, E, block_scores_mean(ql, rep_memo[("mean", g)], E)
        if w.block_score == 2:
            if ("ext", g) not in rep_memo:
                rep_memo[("ext", g)] = block_extremes(res.klow[g], Bk)
            kmax, kmin = rep_memo[("ext", g)]
            return ql, E, block_scores_minmax(ql, kmax, kmin, E)
        return ql, E, block_scores(ql, rows, rep_klow.get(g, res.klow[g]), E, Bk)

    off = 0
    for b in blocks:
        r0, r1 = b * Bq, min(N, (b + 1) * Bq)
        rows = np.arange(r0, r1, dtype=np.int64)
        Qb = q_rows(r0, r1)
        qe = r1 - 1
        for h in heads:
            g = head_group(h, Hq, Hkv)
            kind = w.head_kind[h]
            q = Qb[:, h]
            if kind == DENSE:
                keys = static_key_candidates(DENSE, r0, r1, N, w.window, w.sink, w.last_q)
                o = attend_rows(q, rows, K[:, g], V[:, g], keys, visible_dense, sc)
            elif kind == SWA:
                keys = static_key_candidates(SWA, r0, r1, N, w.window, w.sink, w.last_q)
                o = attend_rows(q, rows, K[:, g], V[:, g], keys,
                                lambda ri, kj: visible_swa(ri, kj, w.window), sc)
            elif kind == TRIANGLE:
                keys = static_key_candidates(TRIANGLE, r0, r1, N, w.window, w.sink, w.last_q)
                o = attend_rows(q, rows, K[:, g], V[:, g], keys,
                                lambda ri, kj: visible_triangle(ri, kj, N, w.sink, w.window, w.last_q), sc)
            elif kind == RETRIEVAL:
                ql, E, s = scores_for(h, g, b, Qb, rows, qe)
                res.qlow.setdefault(h, {})[b] = ql
                if w.group_select:
                    if (g, b) not in group_memo:
                        sg = np.max(np.stack([scores_for(hh, g, b, Qb, rows, qe)[2]
                                              for hh in ret_of_group[g]]), axis=0) if E.size else s
                        group_memo[(g, b)] = (sg, choose(sg, E))
                    s, S = group_memo[(g, b)]
                else:
                    S = choose(s, E)
                if sel_override is not None:
                    S = np.asarray(sel_override[h][b], dtype=np.int64)
                if w.n_clusters > 0:
                    keys, vis = retrieval_key_set(rows, w.window, Bk, 0, clusters=S, assign=res.assign[g],
                                                  n_clusters=res.centroids[g].shape[0])
                else:
                    keys, vis = retrieval_key_set(rows, w.window, Bk, w.force_block0, blocks=S)
                res.sel.setdefault(h, {})[b] = S
                res.scored.setdefault(h, {})[b] = (E, s)
                o = attend_rows(q, rows, K[:, g], V[:, g], keys, vis, sc)
            else:
                raise ValueError(f"unknown head kind {kind}")
            O[off:off + rows.size, h] = o
        off += rows.size

    if with_out and w.n_out > 0:
        ts = np.arange(w.n_out) if out_rows is None else np.asarray(sorted(set(int(t) for t in out_rows)))
        Oo = np.zeros((ts.size, Hq, D), dtype=np.float64)
        for x, t in enumerate(ts):
            p = N - w.n_out + t
            qp = q_rows(p, p + 1)[0]
            for h in heads:
                g = head_group(h, Hq, Hkv)
                Oo[x, h] = orthros_cross(qp[h], xa_scale[h], xa_offset[h], K[:, g], V[:, g], p, sc)
        res.O_out = Oo
        res.out_rows = ts
    return res
