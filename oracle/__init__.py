"""Plain fp64 CPU oracle for head-wise hybrid attention prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this package.  The product path
(``hybrid_attention_prefill_amd``) never imports it and shares no code with
it: the two meet only in the seeded input generator ``synth``.

Everything here is written for a reader checking it against the pages by eye:
numpy in float64, one query block at a time, explicit key sets, no fusion.

Sources (the pages, cited by title and passage):
  [RTPurbo]    "RTPurbo" post, tchannels.org (Анализ данных): retrieval vs
               streaming heads; a cheap 16-dim indexer picks candidates, then
               exact attention in full dimension on that small set.
  [RTPurboV2]  "RTPurboV2" article (th-motor.com mirror): ~15% retrieval heads,
               the rest SWA; low-rank projector D -> r=16; K clustering in the
               low-rank space; top-k critique.
  [TriangleMix] 36kr interview "Agent 的注意力系统", TriangleMix introduction:
               shallow layers dense, deep layers keep the streaming region and
               the last Q-K region; GQA group sharing; block representatives.
  [Orthros]    qingkeai.online "一个 Attention,两种工作模式" (Orthros): all
               tokens SWA, output positions add full cross-attention with a
               scale-offset query.

Readings where the pages are silent (each applies throughout):
  softmax scale 1/sqrt(D); query head h uses KV head h // (Hq/Hkv); window w
  keeps keys i-w < j <= i; Q and K are taken as already rotated (no RoPE);
  top-k ties go to the lower index; k-means ties go to the lower centroid.

Parity status per function is stated in each docstring ("pinned by ...").
"""
from .attention import (  # noqa: F401
    softmax_attention, visible_dense, visible_swa, visible_triangle, attend_rows,
)
from .indexer import (  # noqa: F401
    project, eligible_blocks, block_scores, topk_order, select_blocks,
    eligible_clusters, cluster_scores,
)
from .kmeans import lloyd, assign_step, update_step, kmeans_objective  # noqa: F401
from .prefill import (  # noqa: F401
    head_group, static_key_candidates, retrieval_key_set, layer_prefill, orthros_cross, OracleResult,
)
