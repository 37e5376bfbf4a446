"""Lloyd k-means of the low-rank keys, fp64.

[RTPurboV2] key finding 3: once the projector filters the high-frequency
positional noise, semantically similar keys gather in the low-rank space, so
the key sequence can be compressed by clustering and whole clusters of
unrelated keys skipped.  The pages name clustering but not the algorithm; the
reading here is plain Lloyd iteration with squared Euclidean distance:

  C^0_m = klow_{m * stride}                          (m = 0 .. M-1)
  for t = 1 .. iters:
      a_j   = argmin_m ||klow_j - C^{t-1}_m||^2       (lowest m on exact ties)
      C^t_m = mean{klow_j : a_j = m}, or C^{t-1}_m if no key is assigned to m
  result: centroids C^iters and assignment a from the last iteration.
"""
from __future__ import annotations

import numpy as np


def assign_step(X: np.ndarray, C: np.ndarray, chunk: int = 64) -> np.ndarray:
    """argmin of the squared distance, computed from its definition
    sum_d (x_d - c_d)^2 in fp64; np.argmin keeps the first (lowest) index on
    exact ties.  Pinned: M = N with stride 1 gives the identity; separated
    blobs give their known labels."""
    X = np.asarray(X, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    out = np.empty(X.shape[0], dtype=np.int64)
    for a in range(0, X.shape[0], chunk):
        diff = X[a:a + chunk, None, :] - C[None, :, :]
        d = np.einsum("nmr,nmr->nm", diff, diff)
        out[a:a + chunk] = np.argmin(d, axis=1)
    return out


def sq_dist(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """||x - c||^2 from the definition, fp64 (x [n, r], c [n, r])."""
    d = np.asarray(x, dtype=np.float64) - np.asarray(c, dtype=np.float64)
    return np.einsum("nr,nr->n", d, d)


def update_step(X: np.ndarray, assign: np.ndarray, C_prev: np.ndarray) -> np.ndarray:
    """Each centroid becomes the mean of its members; an empty cluster keeps
    its previous centroid.  Pinned: result equals the per-cluster mean taken
    one cluster at a time."""
    X = np.asarray(X, dtype=np.float64)
    M, r = C_prev.shape
    cnt = np.bincount(assign, minlength=M).astype(np.float64)
    sums = np.zeros((M, r), dtype=np.float64)
    np.add.at(sums, assign, X)
    C = np.array(C_prev, dtype=np.float64, copy=True)
    nz = cnt > 0
    C[nz] = sums[nz] / cnt[nz, None]
    return C


def kmeans_objective(X: np.ndarray, C: np.ndarray, assign: np.ndarray) -> float:
    return float(sq_dist(X, np.asarray(C, dtype=np.float64)[assign]).sum())


def lloyd(X: np.ndarray, M: int, stride: int, iters: int, keep_history: bool = False):
    """Returns (C, assign, history); history[t] = (C^{t+1}, a^{t+1}) if kept."""
    X = np.asarray(X, dtype=np.float64)
    if M * stride > X.shape[0] or M <= 0 or stride <= 0 or iters < 1:
        raise ValueError("k-means needs M * stride <= N and at least one iteration")
    C = X[np.arange(M) * stride].copy()
    a = None
    hist = []
    for _ in range(iters):
        a = assign_step(X, C)
        C = update_step(X, a, C)
        if keep_history:
            hist.append((C.copy(), a.copy()))
    return C, a, hist
