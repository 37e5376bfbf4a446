"""Masked softmax attention in fp64 and the static key-set predicates.

o_i = sum_{j in K(i)} exp(s_ij - m_i) v_j / sum_{j in K(i)} exp(s_ij - m_i),
s_ij = scale * q_i . k_j,  m_i = max_{j in K(i)} s_ij.

The key sets K(i) (all causal, j <= i):
  dense      {0..i}
  SWA(w)     {j : i-w < j <= i}        [RTPurboV2] streaming heads use a
             sliding window; [Orthros] "Prefilling" section: every token runs SWA.
  triangle   {j <= i : j < sink  or  i-j < w  or  i >= N-L}
             [TriangleMix] introduction: keep the streaming region (initial
             sink keys plus the local band) and the last Q-K region (the last
             L query rows attend to every earlier key); the middle is dropped.
"""
from __future__ import annotations

import numpy as np


def visible_dense(rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Causal: key j visible to query i iff j <= i.  Pinned by brute force."""
    return keys[None, :] <= rows[:, None]


def visible_swa(rows: np.ndarray, keys: np.ndarray, w: int) -> np.ndarray:
    """Sliding window of w keys ending at the query itself: i-w < j <= i.
    Pinned: w >= N reduces to dense; w = 1 gives o_i = v_i."""
    d = rows[:, None] - keys[None, :]
    return (d >= 0) & (d < w)


def visible_triangle(rows: np.ndarray, keys: np.ndarray, n_tokens: int,
                     sink: int, w: int, last: int) -> np.ndarray:
    """TriangleMix mask: causal and (sink or band or last rows).
    Pinned: L = N -> dense; sink = L = 0 -> SWA(w); w >= N -> dense; a hand
    drawn 8x8 picture in tests/golden."""
    d = rows[:, None] - keys[None, :]
    causal = d >= 0
    sink_k = keys[None, :] < sink
    band = d < w
    last_r = rows[:, None] >= n_tokens - last
    return causal & (sink_k | band | last_r)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      visible: np.ndarray, scale: float,
                      return_weights: bool = False):
    """Plain masked softmax in fp64.

    q [n, D], k [m, D], v [m, Dv], visible [n, m] bool.  Rows with no visible
    key give zeros (never produced by the masks above: the query itself is
    always visible).  Pinned by a pure-Python brute force (N <= 256), the
    Q = 0 closed form (uniform mean over the key set) and one-hot V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    has = np.isfinite(m)
    m = np.where(has, m, 0.0)
    p = np.where(visible, np.exp(s - m), 0.0)
    den = p.sum(axis=1, keepdims=True)
    den = np.where(has, den, 1.0)
    wgt = p / den
    o = wgt @ v
    if return_weights:
        return o, wgt
    return o


def attend_rows(q_rows: np.ndarray, row_ids: np.ndarray, K: np.ndarray, V: np.ndarray,
                key_ids: np.ndarray, visible_fn, scale: float) -> np.ndarray:
    """Attention for the given query rows over the candidate keys ``key_ids``
    (a superset of every row's key set), with the exact mask from
    ``visible_fn(row_ids, key_ids)``."""
    key_ids = np.asarray(key_ids, dtype=np.int64)
    vis = visible_fn(np.asarray(row_ids, dtype=np.int64), key_ids)
    return softmax_attention(q_rows, K[key_ids], V[key_ids], vis, scale)
