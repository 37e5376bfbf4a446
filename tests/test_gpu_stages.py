"""The stage entry points, called one after another the way a caller (and the
benchmark) can use them, give bit-identical outputs to the whole-layer call:
same kernels, same order, the workspace shared between stages."""
import numpy as np
import pytest

import synth
from synth.configs import shrink
from tests import _gpu

pytestmark = pytest.mark.gpu


def _cases():
    q = synth.WORKLOADS["qwen3_30b_a3b_32k"]
    a = synth.WORKLOADS["allsparse_1m"]
    o = synth.WORKLOADS["orthros_8b_128k"]
    small_q = shrink(q, 4096, window=1024)
    small_a = shrink(a, 4096, n_clusters=64, window=256, n_needles=2).with_(kmeans_stride=64, topk=4,
                                                                              kmeans_iters=3)
    return [
        ("tiny", synth.WORKLOADS["tiny_hybrid_2k"]),
        ("blocks", small_q),
        ("blocks_group", small_q.with_(group_select=1)),
        ("blocks_mean", small_q.with_(block_score=1)),
        ("blocks_extremes", small_q.with_(block_score=2)),
        ("blocks_int8", small_q.with_(index_bits=8)),
        ("clusters", small_a),
        ("clusters_group", small_a.with_(group_select=1)),
        ("orthros", shrink(o, 3000).with_(n_out=100)),
    ]


@pytest.mark.parametrize("name,w", _cases(), ids=[c[0] for c in _cases()])
def test_stages_equal_whole_layer(name, w):
    import torch
    import hybrid_attention_prefill_amd as ha
    print(f"\n[case] stages {name} N={w.n_tokens}", flush=True)
    li = synth.make_layer_inputs(w)
    O1, Oo1, _ = _gpu.run_gpu(w, li, return_aux=False)
    Q, K, V = _gpu.dev_bf16(li.Q), _gpu.dev_bf16(li.K), _gpu.dev_bf16(li.V)
    N, Hq, Hkv = w.n_tokens, w.n_q_heads, w.n_kv_heads
    d = ha.make_desc(N, Hq, Hkv, 128, window=w.window, topk=w.topk, force_block0=w.force_block0,
                     n_clusters=w.n_clusters, kmeans_iters=w.kmeans_iters, kmeans_stride=w.kmeans_stride,
                     sink=w.sink, last_q=w.last_q, n_out=w.n_out, group_select=w.group_select,
                     block_score=w.block_score, index_bits=w.index_bits)
    ws = torch.empty(max(256, ha.ha_workspace_bytes(d, w.head_kind)), dtype=torch.uint8, device="cuda")
    O2 = torch.zeros((N, Hq, 128), dtype=torch.float32, device="cuda")
    if w.ret_heads:
        P = _gpu.dev_f32(li.P)
        nret, nqb = len(w.ret_heads), w.n_qb
        qlow = torch.empty((nret, N, 16), dtype=torch.float32, device="cuda")
        klow = torch.empty((Hkv, N, 16), dtype=torch.float32, device="cuda")
        sel = torch.empty((nret, nqb, w.topk), dtype=torch.int32, device="cuda")
        ha.ha_index_project(d, w.head_kind, Q, K, P, qlow, klow)
        if w.n_clusters:
            M = w.n_clusters
            cent = torch.empty((Hkv, M, 16), dtype=torch.float32, device="cuda")
            asg = torch.empty((Hkv, N), dtype=torch.int32, device="cuda")
            off = torch.empty((Hkv, M + 1), dtype=torch.int32, device="cuda")
            mem = torch.empty((Hkv, N), dtype=torch.int32, device="cuda")
            ha.ha_kmeans(d, klow, cent, asg, off, mem, ws)
            ha.ha_select_clusters(d, w.head_kind, qlow, cent, off, mem, sel, ws)
            ha.ha_attn_gather(d, w.head_kind, Q, K, V, sel, off, mem, O2, ws)
        else:
            ha.ha_select_blocks(d, w.head_kind, qlow, klow, sel, ws)
            ha.ha_attn_gather(d, w.head_kind, Q, K, V, sel, None, None, O2, ws)
    if any(k != 1 for k in w.head_kind):
        ha.ha_attn_band(d, w.head_kind, Q, K, V, O2, ws)
    if w.n_out:
        Oo2 = torch.empty((w.n_out, Hq, 128), dtype=torch.float32, device="cuda")
        ha.ha_attn_cross(d, Q, K, V, _gpu.dev_f32(li.xa_scale), _gpu.dev_f32(li.xa_offset), Oo2, ws)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2), f"{name}: max diff {float((O1 - O2).abs().max()):.3e}"
    if w.n_out:
        assert torch.equal(Oo1, Oo2)
