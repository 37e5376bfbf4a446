"""Seeded synthetic layer inputs.

Every tensor is drawn in chunks of 65536 token rows; chunk ``c`` of tensor
``tag`` comes from ``numpy.random.default_rng([seed, tag, c])``, so any row
range can be regenerated on its own (the oracle regenerates only the rows it
samples) and chunks can be drawn in parallel threads.

Q, K and V are returned as raw bfloat16 bit patterns (``uint16``), rounded
from float32 draws with round-to-nearest-even.  ``bf16_to_f64`` widens them
exactly.  Per-head parameters (indexer projection P, Orthros scale/offset) are
float32.

Recipes (input structure only; no attention arithmetic lives here):
  plain            Q, K, V ~ N(0, 1)
  planted_lowfreq  keys additionally carry, on the low-frequency rotate-half
                   dims {48..63} U {112..127}, twice a topic vector chosen per
                   1024-token segment from 16 topics per KV head
  needles          per KV head, ``n_needles`` keys are replaced by 32*u (u a
                   random unit vector) and one later query row of one head of
                   that group (beyond window + 64) is set to the same 32*u
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from .configs import Workload

CHUNK = 65536
TAG_Q, TAG_K, TAG_V, TAG_P, TAG_XS, TAG_XO, TAG_TOPIC, TAG_NEEDLE = range(1, 9)
LOWFREQ_DIMS = np.r_[48:64, 112:128]
TOPIC_SEGMENT = 1024
N_TOPICS = 16


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_to_f32(b).astype(np.float64)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(seed: int, tag: int, row_shape, r0: int, r1: int, out: np.ndarray, finish,
             std: float = 1.0, mean: float = 0.0):
    """Draw rows [r0, r1) chunk by chunk (threads), pass each float32 chunk
    through ``finish(rows_lo, rows_hi, x) -> array`` and store it in ``out``."""
    if r1 <= r0:
        return out
    c0, c1 = r0 // CHUNK, (r1 - 1) // CHUNK

    def one(c):
        rng = np.random.default_rng([seed, tag, c])
        lo, hi = c * CHUNK, (c + 1) * CHUNK
        a, b = max(lo, r0), min(hi, r1)
        blk = rng.standard_normal((CHUNK,) + tuple(row_shape), dtype=np.float32)
        if a != lo or b != hi:
            blk = blk[a - lo:b - lo]
        if std != 1.0:
            blk *= np.float32(std)
        if mean != 0.0:
            blk += np.float32(mean)
        out[a - r0:b - r0] = finish(a, b, blk)

    cs = list(range(c0, c1 + 1))
    if len(cs) == 1:
        one(cs[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, cs))
    return out


def gen_rows(seed: int, tag: int, row_shape, r0: int, r1: int,
             std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 normal draws for token rows [r0, r1) of a chunked tensor."""
    out = np.empty((max(0, r1 - r0),) + tuple(row_shape), dtype=np.float32)
    return _chunked(seed, tag, row_shape, r0, r1, out, lambda a, b, x: x, std, mean)


def gen_rows_bf16(seed: int, tag: int, row_shape, r0: int, r1: int, plant=None) -> np.ndarray:
    """Like gen_rows, rounded to bf16 bit patterns per chunk; ``plant(a, b, x)``
    may modify the float32 rows [a, b) in place before rounding."""
    out = np.empty((max(0, r1 - r0),) + tuple(row_shape), dtype=np.uint16)

    def finish(a, b, x):
        if plant is not None:
            plant(a, b, x)
        return bf16_round(x)
    return _chunked(seed, tag, row_shape, r0, r1, out, finish)


def gen_param(seed: int, tag: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    rng = np.random.default_rng([seed, tag])
    x = rng.standard_normal(tuple(shape), dtype=np.float64) * std + mean
    return x.astype(np.float32)


# ----------------------------------------------------------------------------
# recipes


def _topics(w: Workload):
    rng = np.random.default_rng([w.seed, TAG_TOPIC])
    z = rng.standard_normal((w.n_kv_heads, N_TOPICS, LOWFREQ_DIMS.size)).astype(np.float32)
    nseg = (w.n_tokens + TOPIC_SEGMENT - 1) // TOPIC_SEGMENT
    seg_topic = rng.integers(0, N_TOPICS, size=(w.n_kv_heads, nseg))
    return z, seg_topic


@dataclasses.dataclass
class Needles:
    kv_head: np.ndarray    # [n]
    key_pos: np.ndarray    # [n]
    q_head: np.ndarray     # [n]
    q_row: np.ndarray      # [n]
    vec: np.ndarray        # [n, D] float32 (before bf16 rounding)


def needles(w: Workload) -> Optional[Needles]:
    if w.recipe != "needles" or w.n_needles <= 0:
        return None
    rng = np.random.default_rng([w.seed, TAG_NEEDLE])
    G = w.n_q_heads // w.n_kv_heads
    hi_key = w.n_tokens - w.window - 128
    if hi_key <= 0:
        return None
    kv, kp, qh, qr, vec = [], [], [], [], []
    for g in range(w.n_kv_heads):
        for n in range(w.n_needles):
            p = int(rng.integers(0, hi_key))
            u = rng.standard_normal(w.head_dim)
            u = u / np.linalg.norm(u)
            i = int(rng.integers(p + w.window + 64, w.n_tokens))
            kv.append(g); kp.append(p); qh.append(G * g + (n % G)); qr.append(i)
            vec.append((32.0 * u).astype(np.float32))
    return Needles(np.array(kv), np.array(kp), np.array(qh), np.array(qr), np.stack(vec))


def gen_q(w: Workload, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    r1 = w.n_tokens if r1 is None else r1
    nd = needles(w)

    def plant(a, b, x):
        if nd is not None:
            for n in range(nd.q_row.size):
                i = int(nd.q_row[n])
                if a <= i < b:
                    x[i - a, nd.q_head[n]] = nd.vec[n]
    return gen_rows_bf16(w.seed, TAG_Q, (w.n_q_heads, w.head_dim), r0, r1, plant)


def gen_k(w: Workload, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    r1 = w.n_tokens if r1 is None else r1
    nd = needles(w)
    topics = _topics(w) if w.recipe == "planted_lowfreq" else None

    def plant(a, b, x):
        if topics is not None:
            z, seg_topic = topics
            seg = np.arange(a, b) // TOPIC_SEGMENT
            for g in range(w.n_kv_heads):
                add = 2.0 * z[g, seg_topic[g, seg]]            # [rows, 32]
                x[:, g, LOWFREQ_DIMS] += add.astype(np.float32)
        if nd is not None:
            for n in range(nd.key_pos.size):
                p = int(nd.key_pos[n])
                if a <= p < b:
                    x[p - a, nd.kv_head[n]] = nd.vec[n]
    return gen_rows_bf16(w.seed, TAG_K, (w.n_kv_heads, w.head_dim), r0, r1, plant)


def gen_v(w: Workload, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    r1 = w.n_tokens if r1 is None else r1
    return gen_rows_bf16(w.seed, TAG_V, (w.n_kv_heads, w.head_dim), r0, r1)


def gen_proj(w: Workload) -> np.ndarray:
    """Indexer projection P [Hkv, D, r] ~ N(0, 1/D) (variance 1/D)."""
    return gen_param(w.seed, TAG_P, (w.n_kv_heads, w.head_dim, w.rank), std=1.0 / np.sqrt(w.head_dim))


def gen_scale_offset(w: Workload):
    """Orthros cross-attention query affine: s = 1 + N(0, 0.05), o = N(0, 0.05)
    (0.05 read as the variance), [Hq, D] float32."""
    sd = float(np.sqrt(0.05))
    s = gen_param(w.seed, TAG_XS, (w.n_q_heads, w.head_dim), std=sd, mean=1.0)
    o = gen_param(w.seed, TAG_XO, (w.n_q_heads, w.head_dim), std=sd)
    return s, o


@dataclasses.dataclass
class LayerInputs:
    w: Workload
    Q: np.ndarray                      # uint16 bf16 bits [N, Hq, D]
    K: np.ndarray                      # uint16 bf16 bits [N, Hkv, D]
    V: np.ndarray                      # uint16 bf16 bits [N, Hkv, D]
    P: Optional[np.ndarray]            # float32 [Hkv, D, r]
    xa_scale: Optional[np.ndarray]     # float32 [Hq, D]
    xa_offset: Optional[np.ndarray]    # float32 [Hq, D]
    needles: Optional[Needles] = None


def make_layer_inputs(w: Workload, *, with_q: bool = True) -> LayerInputs:
    Q = gen_q(w) if with_q else None
    K = gen_k(w)
    V = gen_v(w)
    P = gen_proj(w) if w.ret_heads else None
    xs = xo = None
    if w.n_out > 0:
        xs, xo = gen_scale_offset(w)
    return LayerInputs(w, Q, K, V, P, xs, xo, needles(w))
