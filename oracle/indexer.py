"""Low-rank indexer: projection, candidate scoring and top-k selection (fp64).

[RTPurboV2] key finding 2: a learned projector maps each head's D-dim query
and key to r = 16 dims that keep the low-frequency (semantic) RoPE components.
[RTPurbo]: the 16-dim indexer acts as a scout that picks candidate keys from
the past context; exact attention then runs on that small set in full
dimension.  [TriangleMix] interview, top-k matching: keys are grouped into
blocks and a query is scored against block representatives; the selection is
the top-k of those scores.

Block mode (one selection per query head and query block b of Bq rows):
  rows R_b = [b*Bq, min(N, (b+1)*Bq)), qe = max R_b
  eligible E_b = {c >= f0 : c*Bk <= qe - w}     (blocks holding a causal key
                 that some row of b can only reach through selection)
  s_{b,c} = max{ qlow_i . klow_j : i in R_b, j in block c, j <= i }
  S_b = the k best of E_b by (score desc, index asc); all of E_b if |E_b| <= k
Cluster mode replaces key blocks by k-means clusters of the low-rank keys:
  E_b = {m : cluster m has a member j <= qe - w}
  s_{b,m} = max_{i in R_b} qlow_i . C_m

Cheaper block scores ([TriangleMix] interview, top-k matching: a block is
represented by one point; the representatives named are the mean of its keys
and a point built from each dimension's largest and smallest key value).
With the block's keys K_c = {j in block c, j < N}:
  mean:    s_{b,c} = max_{i in R_b} qlow_i . mean_{j in K_c} klow_j
  min/max: s_{b,c} = max_{i in R_b} sum_d max(q_d kmax_{c,d}, q_d kmin_{c,d}),
           kmax / kmin = per-dimension max / min over K_c: the largest dot
           product any point of the box spanned by the block's keys can
           reach, so it bounds every key's score from above.
Causality inside a block is not applied by either representative.

8-bit indexer (Baidu developer article "深度解析：超长上下文注意力架构的分层优化策略",
mixed-precision index section: the indexer is stored in 8 bits): each low-rank key is kept as int8 codes with
one fp32 scale, scale_j = max_d |k_jd| / 127 and code_jd = k_jd / scale_j
rounded to nearest (ties to even); block scores use the dequantized keys
scale_j * code_j.  The float-to-integer step is taken in fp32, as the
kernel takes it.
"""
from __future__ import annotations

import numpy as np


def project(X: np.ndarray, P: np.ndarray) -> np.ndarray:
    """xlow = x P, X [n, D], P [D, r] -> [n, r] in fp64.
    Pinned: P = [e_0 .. e_{r-1}] returns the first r coordinates of x."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(P, dtype=np.float64)


def eligible_blocks(qe: int, w: int, f0: int, Bk: int) -> np.ndarray:
    """Key blocks c >= f0 with c*Bk <= qe - w (empty when qe < w)."""
    if qe - w < 0:
        return np.zeros(0, dtype=np.int64)
    c_hi = (qe - w) // Bk
    return np.arange(f0, c_hi + 1, dtype=np.int64)


def block_scores(qlow_rows: np.ndarray, row_ids: np.ndarray, klow: np.ndarray,
                 blocks: np.ndarray, Bk: int) -> np.ndarray:
    """Max over causal (query, key) pairs of the low-rank dot product, per
    candidate key block.  Pinned by a double-loop brute force (N <= 256)."""
    N = klow.shape[0]
    out = np.empty(blocks.size, dtype=np.float64)
    row_ids = np.asarray(row_ids, dtype=np.int64)
    for t, c in enumerate(blocks):
        keys = np.arange(c * Bk, min(N, (c + 1) * Bk), dtype=np.int64)
        dots = qlow_rows @ klow[keys].T                      # [rows, keys]
        causal = keys[None, :] <= row_ids[:, None]
        out[t] = np.max(np.where(causal, dots, -np.inf))
    return out


def block_means(klow: np.ndarray, Bk: int) -> np.ndarray:
    """Mean low-rank key of every key block (keys c*Bk .. min(N, (c+1)*Bk)-1)."""
    N = klow.shape[0]
    n_kb = (N + Bk - 1) // Bk
    return np.stack([np.mean(klow[c * Bk: min(N, (c + 1) * Bk)], axis=0) for c in range(n_kb)])


def block_extremes(klow: np.ndarray, Bk: int):
    """Per-dimension (max, min) of the low-rank keys of every key block."""
    N = klow.shape[0]
    n_kb = (N + Bk - 1) // Bk
    kmax = np.stack([np.max(klow[c * Bk: min(N, (c + 1) * Bk)], axis=0) for c in range(n_kb)])
    kmin = np.stack([np.min(klow[c * Bk: min(N, (c + 1) * Bk)], axis=0) for c in range(n_kb)])
    return kmax, kmin


def block_scores_mean(qlow_rows: np.ndarray, means: np.ndarray, blocks: np.ndarray) -> np.ndarray:
    """max_{i in block} qlow_i . mean_c for each candidate block c."""
    if blocks.size == 0:
        return np.zeros(0)
    return np.max(qlow_rows @ means[blocks].T, axis=0)


def block_scores_minmax(qlow_rows: np.ndarray, kmax: np.ndarray, kmin: np.ndarray,
                        blocks: np.ndarray) -> np.ndarray:
    """max_{i in block} sum_d max(q_id kmax_cd, q_id kmin_cd) per candidate block c."""
    if blocks.size == 0:
        return np.zeros(0)
    q = qlow_rows[:, None, :]                                   # [rows, 1, r]
    bound = np.maximum(q * kmax[blocks][None], q * kmin[blocks][None]).sum(axis=2)
    return np.max(bound, axis=0)


def quantize_keys_int8(klow32: np.ndarray):
    """Per-key symmetric 8-bit codes [n, r] int8 and scales [n] fp32, computed
    in fp32 (IEEE division, round half to even); an all-zero key gets scale 0
    and zero codes."""
    k = np.asarray(klow32, dtype=np.float32)
    amax = np.max(np.abs(k), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.rint(k / safe[:, None])
    codes = np.where(scale[:, None] > 0, codes, 0.0)
    return codes.astype(np.int8), scale


def dequantize_keys(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """scale_j * code_j in fp64."""
    return codes.astype(np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


def topk_adaptive(scores: np.ndarray, ids: np.ndarray, k: int, mass: float, scale: float) -> np.ndarray:
    """Adaptive budget ([RTPurboV2], fixed-top-k passage: different heads,
    sequence lengths and queries need very different numbers of context
    tokens; the method that follows that passage is missing from the page, so
    this rule is a proposal, not the page's).  The k best ids by (score desc,
    id asc) are the budget; of them, keep the shortest prefix in that order
    whose share of sum_j exp(scale * s_j) over the k reaches `mass`.  mass <= 0
    or >= 1 keeps all k (fixed top-k).  Returned in ascending id order.
    Pinned: mass >= 1 equals topk_order; a hand-worked three-candidate case;
    equal scores keep ceil(mass * k)."""
    ids = np.asarray(ids, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float64)
    if k <= 0 or ids.size == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((ids, -scores))[:k]
    if mass <= 0.0 or mass >= 1.0:
        return np.sort(ids[order])
    s = scores[order]
    wts = np.exp(scale * (s - s[0]))          # s[0] is the largest score
    share = np.cumsum(wts) / np.sum(wts)
    n = int(np.nonzero(share >= mass)[0][0]) + 1 if np.any(share >= mass) else order.size
    return np.sort(ids[order[:n]])


def topk_order(scores: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The k best ids by (score desc, id asc), returned in ascending id order.
    Pinned: exact ties planted by duplicated key blocks keep the lower ids."""
    ids = np.asarray(ids, dtype=np.int64)
    if k <= 0 or ids.size == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((ids, -np.asarray(scores, dtype=np.float64)))
    return np.sort(ids[order[:k]])


def select_blocks(qlow_h: np.ndarray, klow_g: np.ndarray, N: int, w: int,
                  Bq: int, Bk: int, k: int, f0: int):
    """Per query block: the selected key blocks (ascending) and the scores of
    all eligible blocks (for tie-band checks)."""
    n_qb = (N + Bq - 1) // Bq
    sel, scored = [], []
    for b in range(n_qb):
        rows = np.arange(b * Bq, min(N, (b + 1) * Bq), dtype=np.int64)
        qe = int(rows[-1])
        E = eligible_blocks(qe, w, f0, Bk)
        s = block_scores(qlow_h[rows], rows, klow_g, E, Bk) if E.size else np.zeros(0)
        sel.append(topk_order(s, E, k))
        scored.append((E, s))
    return sel, scored


def eligible_clusters(assign: np.ndarray, M: int, qe: int, w: int) -> np.ndarray:
    """Clusters with at least one member key j <= qe - w."""
    lim = qe - w
    if lim < 0:
        return np.zeros(0, dtype=np.int64)
    members = assign[: lim + 1]
    return np.unique(members).astype(np.int64)


def cluster_scores(qlow_rows: np.ndarray, C: np.ndarray, clusters: np.ndarray) -> np.ndarray:
    """max_{i in block} qlow_i . C_m for each candidate cluster m."""
    if clusters.size == 0:
        return np.zeros(0)
    return np.max(qlow_rows @ C[clusters].T, axis=0)
