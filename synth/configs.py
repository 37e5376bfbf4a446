"""Workload shapes for the hybrid attention prefill layer.

Each workload is one attention layer's prefill: its sizes, the role of every
query head and the selection / mask parameters.  The five named workloads
stand in for the models and context lengths the pages measure on (the real
weights and benchmark suites are not available; inputs are synthetic).

Head roles (one per query head):
  HEAD_SWA        streaming head, causal sliding window
  HEAD_RETRIEVAL  retrieval head, low-rank indexer + selected keys + window
  HEAD_TRIANGLE   TriangleMix mask: sink + band + dense last rows
  HEAD_DENSE      plain causal attention
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

HEAD_SWA = 0
HEAD_RETRIEVAL = 1
HEAD_TRIANGLE = 2
HEAD_DENSE = 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    n_q_heads: int
    n_kv_heads: int
    head_kind: Tuple[int, ...]
    head_dim: int = 128
    window: int = 0
    rank: int = 16
    q_block: int = 64
    k_block: int = 64
    topk: int = 0
    force_block0: int = 0
    n_clusters: int = 0
    kmeans_iters: int = 0
    kmeans_stride: int = 0
    sink: int = 0
    last_q: int = 0
    n_out: int = 0
    # 1: one selection per (KV head, query block), scored by the max over the
    # group's retrieval heads and shared by them (GQA-group-shared selection)
    group_select: int = 0
    # block-mode candidate score: 0 max over causal (query, key) pairs,
    # 1 the block's mean key (representative), 2 the bound from the block's
    # per-dimension key maxima and minima
    block_score: int = 0
    # low-rank key storage of the block scores: 0 fp32, 8 int8 codes with one
    # fp32 scale per key (max-pair block scores only)
    index_bits: int = 0
    # adaptive budget: 0 keeps the fixed top-k; in (0, 1) each query block
    # keeps the shortest prefix of its top-k (score desc) whose softmax share,
    # at scale mass_scale (0: 1/sqrt(rank)), reaches topk_mass
    topk_mass: float = 0.0
    mass_scale: float = 0.0
    # input recipe: "plain", "planted_lowfreq" (keys carry per-segment topic
    # vectors on the low-frequency dims), "needles" (planted key/query pairs)
    recipe: str = "plain"
    n_needles: int = 0
    seed: int = 0

    @property
    def n_qb(self) -> int:
        return (self.n_tokens + self.q_block - 1) // self.q_block

    @property
    def ret_heads(self) -> Tuple[int, ...]:
        return tuple(h for h, k in enumerate(self.head_kind) if k == HEAD_RETRIEVAL)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def desc_dict(self) -> dict:
        """The numeric fields of the C layer descriptor, by name."""
        return dict(
            n_tokens=self.n_tokens, n_q_heads=self.n_q_heads,
            n_kv_heads=self.n_kv_heads, head_dim=self.head_dim,
            softmax_scale=0.0, window=self.window, rank=self.rank,
            q_block=self.q_block, k_block=self.k_block, topk=self.topk,
            force_block0=self.force_block0, n_clusters=self.n_clusters,
            kmeans_iters=self.kmeans_iters, kmeans_stride=self.kmeans_stride,
            sink=self.sink, last_q=self.last_q, n_out=self.n_out,
            group_select=self.group_select, block_score=self.block_score, index_bits=self.index_bits,
            topk_mass=self.topk_mass, mass_scale=self.mass_scale,
        )


def _kinds(n: int, ret: Tuple[int, ...] = (), default: int = HEAD_SWA) -> Tuple[int, ...]:
    return tuple(HEAD_RETRIEVAL if h in ret else default for h in range(n))


# Tiny hybrid layer: 2 retrieval + 6 streaming heads, window 256, top-8 key
# blocks of 64 plus key block 0.
TINY_HYBRID_2K = Workload(
    name="tiny_hybrid_2k", n_tokens=2048, n_q_heads=8, n_kv_heads=2,
    head_kind=_kinds(8, (0, 1)), window=256, topk=8, force_block0=1)

# Qwen3-30B-A3B-shaped attention layer at 32K: 5 retrieval heads (~15%),
# 27 streaming heads with window 8192, top-32 key blocks.
QWEN3_30B_32K = Workload(
    name="qwen3_30b_a3b_32k", n_tokens=32768, n_q_heads=32, n_kv_heads=4,
    head_kind=_kinds(32, (0, 7, 14, 21, 28)), window=8192, topk=32,
    recipe="planted_lowfreq")

# Llama-3.1-8B-shaped TriangleMix layer at 128K (the deep layers).
TRIANGLE_8B_128K = Workload(
    name="trianglemix_llama8b_128k", n_tokens=131072, n_q_heads=32, n_kv_heads=8,
    head_kind=(HEAD_TRIANGLE,) * 32, window=2048, sink=64, last_q=128)

# The same shape as a dense causal layer (the shallow layers).
DENSE_8B_128K = TRIANGLE_8B_128K.with_(
    name="dense_llama8b_128k", head_kind=(HEAD_DENSE,) * 32, window=0, sink=0, last_q=0)

# Orthros prefill, 8B shape at 128K: SWA 4096 for all rows, full cross
# attention for the last prompt token.
ORTHROS_8B_128K = Workload(
    name="orthros_8b_128k", n_tokens=131072, n_q_heads=32, n_kv_heads=8,
    head_kind=(HEAD_SWA,) * 32, window=4096, n_out=1)

# Orthros with many output positions (SFT: the response tokens predict): the
# same layer with its last 8192 rows as output positions.  The response
# length is this suite's choice; the pages give none.
ORTHROS_8B_128K_SFT = ORTHROS_8B_128K.with_(name="orthros_8b_128k_sft8k", n_out=8192)

# The 32K hybrid layer with the cheaper block scores: each key block scored by
# its mean low-rank key, or by the bound from its per-dimension extremes.
QWEN3_30B_32K_MEAN = QWEN3_30B_32K.with_(name="qwen3_30b_a3b_32k_mean", block_score=1)
QWEN3_30B_32K_MINMAX = QWEN3_30B_32K.with_(name="qwen3_30b_a3b_32k_minmax", block_score=2)
# ... and with the low-rank keys of the block scores stored as 8-bit codes
QWEN3_30B_32K_INT8 = QWEN3_30B_32K.with_(name="qwen3_30b_a3b_32k_int8", index_bits=8)

# 1M-token all-sparse layer: every head is a retrieval head, the low-rank keys
# are clustered (16384 centroids, 10 Lloyd iterations, seeds every 64th key),
# each query block takes its top-64 clusters plus a 4096 window.
ALLSPARSE_1M = Workload(
    name="allsparse_1m", n_tokens=1 << 20, n_q_heads=16, n_kv_heads=2,
    head_kind=(HEAD_RETRIEVAL,) * 16, window=4096, topk=64,
    n_clusters=16384, kmeans_iters=10, kmeans_stride=64,
    recipe="needles", n_needles=64)

# The same layer with GQA-group-shared selection: each KV head's 8 retrieval
# heads share one top-64 cluster selection per query block.
ALLSPARSE_1M_GQA = ALLSPARSE_1M.with_(name="allsparse_1m_gqa", group_select=1)

# Adaptive budget (a proposal; the page states only the need): the top-k is a
# budget, and each query block keeps the shortest prefix of it, by score,
# whose softmax share at scale 1/sqrt(r) reaches 0.9.
QWEN3_30B_32K_ADAPTIVE = QWEN3_30B_32K.with_(name="qwen3_30b_a3b_32k_adaptive", topk_mass=0.9)
ALLSPARSE_1M_ADAPTIVE = ALLSPARSE_1M.with_(name="allsparse_1m_adaptive", topk_mass=0.9)

# The TriangleMix layer split: 12 dense shallow layers, 20 triangle layers.
TRIANGLE_LAYER_SPLIT = (12, 20)

WORKLOADS = {w.name: w for w in (
    TINY_HYBRID_2K, QWEN3_30B_32K, QWEN3_30B_32K_MEAN, QWEN3_30B_32K_MINMAX, QWEN3_30B_32K_INT8,
    TRIANGLE_8B_128K, DENSE_8B_128K,
    ORTHROS_8B_128K, ORTHROS_8B_128K_SFT, ALLSPARSE_1M, ALLSPARSE_1M_GQA,
    QWEN3_30B_32K_ADAPTIVE, ALLSPARSE_1M_ADAPTIVE)}


def shrink(w: Workload, n_tokens: int, *, n_clusters: Optional[int] = None,
           window: Optional[int] = None, n_needles: Optional[int] = None) -> Workload:
    """The same head roles and parameters at a smaller sequence length, for
    parity cases the oracle finishes quickly."""
    kw = dict(n_tokens=n_tokens)
    if n_clusters is not None:
        kw["n_clusters"] = n_clusters
    if window is not None:
        kw["window"] = window
    if n_needles is not None:
        kw["n_needles"] = n_needles
    return w.with_(name=f"{w.name}@{n_tokens}", **kw)
