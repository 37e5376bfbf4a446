"""ha_prefill_static (no allocation, static device scratch) against ha_prefill
(caller's workspace) through the C ABI: the same kernels on the same inputs,
so outputs, selections and k-means results must be bit-identical.  Several
calls in a row share the GPU's one scratch array, each on a shorter sequence
than the one before, so a call that read stale scratch left by a larger call
would differ."""
import numpy as np
import pytest
import torch

import hybrid_attention_prefill_amd as ha
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def _both(w):
    print(f"\n[case] static scratch vs workspace: {w.name} N={w.n_tokens}", flush=True)
    li = synth.make_layer_inputs(w)
    Q, K, V = _gpu.dev_bf16(li.Q), _gpu.dev_bf16(li.K), _gpu.dev_bf16(li.V)
    P = _gpu.dev_f32(li.P) if li.P is not None else None
    xs = _gpu.dev_f32(li.xa_scale) if li.xa_scale is not None else None
    xo = _gpu.dev_f32(li.xa_offset) if li.xa_offset is not None else None
    d = ha.make_desc(w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, **{
        k: v for k, v in w.desc_dict().items() if k not in ("n_tokens", "n_q_heads", "n_kv_heads", "head_dim")})
    N, Hq, Hkv, D = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
    assert ha.ha_workspace_bytes(d, w.head_kind) <= ha.HA_STATIC_SCRATCH_BYTES

    def outputs():
        O = torch.full((N, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        O_out = torch.full((w.n_out, Hq, D), float("nan"), dtype=torch.float32, device="cuda") if w.n_out else None
        aux = None
        if w.ret_heads:
            nret = len(w.ret_heads)
            aux = dict(sel=torch.full((nret, w.n_qb, max(1, w.topk)), -7, dtype=torch.int32, device="cuda"))
            if w.n_clusters:
                aux["centroids"] = torch.zeros((Hkv, w.n_clusters, 16), dtype=torch.float32, device="cuda")
                aux["assign"] = torch.full((Hkv, N), -7, dtype=torch.int32, device="cuda")
        return O, O_out, aux

    Oa, Oa_out, aux_a = outputs()
    ws = torch.empty(ha.ha_workspace_bytes(d, w.head_kind), dtype=torch.uint8, device="cuda")
    ha.ha_prefill(d, w.head_kind, Q, K, V, P, xs, xo, Oa, Oa_out, aux_a, ws)
    Ob, Ob_out, aux_b = outputs()
    ha.ha_prefill_static(d, w.head_kind, Q, K, V, P, xs, xo, Ob, Ob_out, aux_b)
    torch.cuda.synchronize()
    assert torch.equal(Oa, Ob), f"{w.name}: outputs differ"
    assert torch.isfinite(Ob).all()
    if w.n_out:
        assert torch.equal(Oa_out, Ob_out), f"{w.name}: cross-attention outputs differ"
    if aux_a is not None:
        for k in aux_a:
            assert torch.equal(aux_a[k], aux_b[k]), f"{w.name}: {k} differs"
    print(f"{w.name}: bit-identical", flush=True)


def test_static_scratch_matches_workspace_path_calls_in_a_row():
    base = synth.WORKLOADS["allsparse_1m"]
    cluster = synth.configs.shrink(base, 12288, n_clusters=192, window=512, n_needles=2).with_(kmeans_iters=3)
    for w in (synth.WORKLOADS["qwen3_30b_a3b_32k"],        # block selection, ~20 MB of scratch
              cluster,                                      # k-means + clusters
              synth.configs.shrink(synth.WORKLOADS["orthros_8b_128k"], 16384),   # split-key cross partials
              synth.WORKLOADS["tiny_hybrid_2k"]):            # smallest last
        _both(w)
