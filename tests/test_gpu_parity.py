"""Parity of the HIP path (through the C ABI) with the fp64 oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails, edge windows."""
import numpy as np
import pytest

import synth
from synth.configs import Workload, HEAD_DENSE, HEAD_RETRIEVAL, HEAD_SWA, HEAD_TRIANGLE
from oracle.prefill import layer_prefill
from tests._util import oracle_arrays
from tests import _gpu

pytestmark = pytest.mark.gpu


def _layer(kinds, N, Hkv=2, **kw):
    return Workload(name="case", n_tokens=N, n_q_heads=len(kinds), n_kv_heads=Hkv, head_kind=tuple(kinds), **kw)


def _compare(w, blocks=None, check_sel=True):
    print(f"\n[case] {w.name} N={w.n_tokens} kinds={w.head_kind} w={w.window} k={w.topk}", flush=True)
    li = synth.make_layer_inputs(w)
    O, O_out, aux = _gpu.run_gpu(w, li)
    q, K, V, P, xs, xo = oracle_arrays(w, li)
    ref = layer_prefill(w, q, K, V, P, xs, xo, blocks=blocks)
    Og = O.cpu().numpy()[ref.rows]
    if w.ret_heads and check_sel:
        sel = aux["sel"].cpu().numpy()
        _gpu.check_group_rows(sel, w)
        klow = aux["klow"].cpu().numpy()
        _gpu.check_lowrank_rows(aux, ref, w)
        k32 = None
        if w.index_bits == 8:
            # 8-bit keys: the oracle quantizes the GPU's validated fp32 keys, so
            # both sides take the float-to-integer step on the same values
            k32 = {g: klow[g] for g in range(w.n_kv_heads)}
            ref = layer_prefill(w, q, K, V, P, xs, xo, blocks=blocks, klow32_override=k32)
        override = {}
        for t, h in enumerate(w.ret_heads):
            override[h] = {}
            for b, (E, s) in ref.scored[h].items():
                _gpu.check_sel(w, sel[t, b], E, s, f"head {h} block {b}")
                override[h][b] = np.array([x for x in sel[t, b] if x >= 0], dtype=np.int64)
        # grade attention given the validated GPU selection
        ref = layer_prefill(w, q, K, V, P, xs, xo, blocks=blocks, sel_override=override, klow32_override=k32)
    _gpu.assert_close_out(Og, ref.O, w.name)
    if w.n_out:
        _gpu.assert_close_out(O_out.cpu().numpy(), ref.O_out, w.name + " O_out")
    return O, ref


@pytest.mark.parametrize("N", [1, 63, 64, 65, 700])
@pytest.mark.parametrize("window", [1, 7, 64, 100, 5000])
def test_swa_heads(N, window):
    _compare(_layer([HEAD_SWA] * 8, N, window=window))


@pytest.mark.parametrize("N", [1, 130, 1000])
def test_dense_heads(N):
    _compare(_layer([HEAD_DENSE] * 4, N, Hkv=1))


@pytest.mark.parametrize("N,sink,window,last", [(1000, 64, 128, 128), (1000, 3, 50, 37), (777, 100, 1, 0),
                                                (500, 0, 64, 500), (256, 64, 2048, 128)])
def test_triangle_heads(N, sink, window, last):
    _compare(_layer([HEAD_TRIANGLE] * 4, N, window=window, sink=sink, last_q=last))


def test_mixed_roles_one_layer():
    kinds = [HEAD_SWA, HEAD_DENSE, HEAD_TRIANGLE, HEAD_SWA, HEAD_TRIANGLE, HEAD_DENSE, HEAD_SWA, HEAD_SWA]
    _compare(_layer(kinds, 900, window=130, sink=10, last_q=70))


def test_gqa_group_sizes():
    _compare(_layer([HEAD_SWA] * 6, 300, Hkv=6, window=40))       # G = 1
    _compare(_layer([HEAD_SWA] * 16, 300, Hkv=2, window=40))      # G = 8: two packs per KV head
    _compare(_layer([HEAD_SWA] * 5, 300, Hkv=1, window=40))       # partial pack


@pytest.mark.parametrize("kind", [HEAD_SWA, HEAD_DENSE, HEAD_TRIANGLE])
def test_band_pack_classes(kind):
    # 7 heads of one role on one KV head: a 4-head pack (64 rows per
    # workgroup) and a 3-head remainder split into 2 heads (128 rows) + 1
    # head (256 rows); N = 333 leaves every class a ragged last tile
    _compare(_layer([kind] * 7, 333, Hkv=1, window=90, sink=5, last_q=40))


def test_band_pack_classes_retrieval_window():
    # 3 retrieval heads + 4 SWA heads on one KV head: the retrieval heads'
    # window pass runs as a 2-head and a 1-head pack
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_SWA, HEAD_SWA, HEAD_RETRIEVAL, HEAD_SWA]
    _compare(_layer(kinds, 700, Hkv=1, window=100, topk=3))


@pytest.mark.parametrize("N,window,topk,f0", [(1000, 100, 3, 0), (1000, 100, 3, 1), (1337, 64, 8, 1),
                                              (700, 1, 2, 0), (640, 50, 0, 1), (640, 50, 100, 0),
                                              (300, 5000, 4, 0)])
def test_retrieval_block_mode(N, window, topk, f0):
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL,
             HEAD_RETRIEVAL]
    _compare(_layer(kinds, N, window=window, topk=topk, force_block0=f0))


@pytest.mark.parametrize("N,window,topk,f0", [(1000, 100, 3, 0), (1337, 64, 8, 1), (700, 1, 2, 0),
                                              (640, 50, 100, 0), (300, 5000, 4, 1)])
def test_group_select_block_mode(N, window, topk, f0):
    # groups of 3 retrieval heads (one pack each) next to streaming heads
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL,
             HEAD_RETRIEVAL]
    _compare(_layer(kinds, N, window=window, topk=topk, force_block0=f0, group_select=1))


@pytest.mark.parametrize("score", [1, 2])
@pytest.mark.parametrize("N,window,topk,f0,gs", [(1000, 100, 3, 0, 0), (1337, 64, 8, 1, 0), (700, 1, 2, 0, 0),
                                                 (640, 50, 100, 0, 0), (300, 5000, 4, 1, 0), (1000, 100, 3, 1, 1)])
def test_block_representative_scores(score, N, window, topk, f0, gs):
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL,
             HEAD_RETRIEVAL]
    _compare(_layer(kinds, N, window=window, topk=topk, force_block0=f0, group_select=gs, block_score=score))


@pytest.mark.parametrize("N,window,topk,f0,gs", [(1000, 100, 3, 0, 0), (1337, 64, 8, 1, 0), (700, 1, 2, 0, 0),
                                                 (640, 50, 100, 0, 0), (1000, 100, 3, 1, 1)])
def test_int8_indexer_keys(N, window, topk, f0, gs):
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL,
             HEAD_RETRIEVAL]
    _compare(_layer(kinds, N, window=window, topk=topk, force_block0=f0, group_select=gs, index_bits=8))


def test_quantize_keys_bit_exact():
    # codes and scales equal the oracle's fp32 quantizer bit for bit: random
    # keys of many magnitudes, all-zero keys, and keys with max |k| = 127
    # (scale 1) holding exact .5 values, which round to even
    import torch
    import hybrid_attention_prefill_amd as ha
    from oracle.indexer import quantize_keys_int8
    rng = np.random.default_rng(11)
    Hkv, N = 2, 3000
    k = (rng.standard_normal((Hkv * N, 16)) * rng.uniform(1e-3, 50, (Hkv * N, 1))).astype(np.float32)
    k[5] = 0.0
    k[7] = 0.0
    k[100] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.5, 0.0, -0.0, 10.5, -10.5, 64.5, 1.0]
    d = ha.make_desc(N, 2, Hkv, 128, window=64, topk=4, index_bits=8)
    codes = torch.empty((Hkv, N, 16), dtype=torch.int8, device="cuda")
    scales = torch.empty((Hkv, N), dtype=torch.float32, device="cuda")
    ha.ha_quantize_keys(d, torch.from_numpy(k.reshape(Hkv, N, 16)).cuda(), codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = quantize_keys_int8(k)
    np.testing.assert_array_equal(scales.cpu().numpy().reshape(-1).view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy().reshape(-1, 16), want_c)
    assert list(want_c[100]) == [127, 0, 2, 2, 0, -2, -2, 126, -126, 4, 0, 0, 10, -10, 64, 1]


@pytest.mark.parametrize("N", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("mode", ["blocks", "group", "mean", "extremes", "int8"])
def test_retrieval_tiny_sequences(N, mode):
    # sequences shorter than, equal to and just past one block: no eligible
    # block at all, then the first one
    kinds = [HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL]
    kw = dict(window=64, topk=3)
    kw.update({"group": dict(group_select=1), "mean": dict(block_score=1), "extremes": dict(block_score=2),
               "int8": dict(index_bits=8)}.get(mode, {}))
    _compare(_layer(kinds, N, Hkv=1, **kw))


def test_group_select_pack_shapes():
    # G = 8, all retrieval: two full packs per group
    _compare(_layer([HEAD_RETRIEVAL] * 16, 900, Hkv=2, window=70, topk=4, group_select=1))
    # G = 6: a full pack and a half-empty one
    _compare(_layer([HEAD_RETRIEVAL] * 6, 900, Hkv=1, window=70, topk=5, force_block0=1, group_select=1))
    # one retrieval head per group: same as per-head selection
    kinds = [HEAD_RETRIEVAL if h % 4 == 1 else HEAD_SWA for h in range(8)]
    _compare(_layer(kinds, 900, window=70, topk=3, group_select=1))


def test_tiny_hybrid_layer_full():
    _compare(synth.WORKLOADS["tiny_hybrid_2k"])


def test_planted_component_layer_reduced():
    w = synth.configs.shrink(synth.WORKLOADS["qwen3_30b_a3b_32k"], 4096, window=1024)
    _compare(w)


@pytest.mark.parametrize("N,n_out", [(1, 1), (3000, 1), (2500, 3), (2500, 15),
                                     # matrix-core path: split key range, one tile, ragged rows
                                     (2500, 16), (130, 100), (3000, 700),
                                     # every position an output position (pre-training)
                                     (1000, 1000), (64, 64)])
def test_orthros_cross(N, n_out):
    w = _layer([HEAD_SWA] * 8, N, window=256, n_out=n_out)
    _compare(w)


def test_orthros_cross_many_rows_wide_groups():
    # G = 20 (five packs of four heads per KV head), a partial last pack (G = 6)
    _compare(_layer([HEAD_SWA] * 20, 900, Hkv=1, window=100, n_out=200))
    _compare(_layer([HEAD_SWA] * 12, 900, Hkv=2, window=100, n_out=77))


def test_deterministic_rerun():
    import torch
    w = synth.WORKLOADS["tiny_hybrid_2k"]
    li = synth.make_layer_inputs(w)
    a = _gpu.run_gpu(w, li)
    b = _gpu.run_gpu(w, li)
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[2]["sel"], b[2]["sel"])


@pytest.mark.parametrize("score", [0, 1, 2])
@pytest.mark.parametrize("f0", [0, 1])
def test_block_selection_exact_ties_keep_lowest_ids(f0, score):
    # every key block holds the same low-rank keys and the window (128) keeps
    # every eligible pair causal, so all eligible blocks score exactly alike
    # (pairs, means and extremes alike): the selection must be the k lowest
    # eligible block ids
    import torch
    import hybrid_attention_prefill_amd as ha
    N, k, w = 4096, 5, 128
    rng = np.random.default_rng(3)
    kl = np.tile(rng.standard_normal((64, 16)).astype(np.float32), (N // 64, 1))
    ql = rng.standard_normal((N, 16)).astype(np.float32)
    kinds = [HEAD_RETRIEVAL] + [HEAD_SWA] * 3
    d = ha.make_desc(N, 4, 1, 128, window=w, topk=k, force_block0=f0, block_score=score)
    klow = torch.from_numpy(kl[None]).cuda()
    qlow = torch.from_numpy(ql[None]).cuda()
    sel = torch.full((1, N // 64, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(256, ha.ha_workspace_bytes(d, kinds)), dtype=torch.uint8, device="cuda")
    ha.ha_select_blocks(d, kinds, qlow, klow, sel, ws)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()[0]
    for b in range(N // 64):
        qe = b * 64 + 63
        E = list(range(f0, (qe - w) // 64 + 1)) if qe - w >= 0 else []
        expect = E[:k] + [-1] * (k - min(k, len(E)))
        assert list(sel[b]) == expect, (b, list(sel[b]), expect)


@pytest.mark.parametrize("M", [256, 2048])
def test_cluster_selection_exact_ties_keep_lowest_ids(M):
    # identical centroids: every eligible cluster scores alike.  With M = 2048
    # each quarter of the clusters holds more candidates than the prefilter's
    # per-wave region, so late blocks take the full select.
    import torch
    import hybrid_attention_prefill_amd as ha
    N, k, w = 4096, 7, 512
    rng = np.random.default_rng(4)
    cent = np.tile(rng.standard_normal((1, 16)).astype(np.float32), (M, 1))
    assign = np.arange(N) % M                       # first member of cluster m is key m
    off = np.r_[0, np.cumsum(np.bincount(assign, minlength=M))].astype(np.int32)
    mem = np.lexsort((np.arange(N), assign)).astype(np.int32)
    kinds = [HEAD_RETRIEVAL] * 4
    d = ha.make_desc(N, 4, 1, 128, window=w, topk=k, n_clusters=M, kmeans_iters=1, kmeans_stride=N // M)
    ql = torch.from_numpy(rng.standard_normal((4, N, 16)).astype(np.float32)).cuda()
    sel = torch.full((4, N // 64, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(ha.ha_workspace_bytes(d, kinds), dtype=torch.uint8, device="cuda")
    ha.ha_select_clusters(d, kinds, ql, torch.from_numpy(cent[None]).cuda(), torch.from_numpy(off[None]).cuda(),
                          torch.from_numpy(mem[None]).cuda(), sel, ws)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    for t in range(4):
        for b in range(N // 64):
            lim = b * 64 + 63 - w
            E = [m for m in range(M) if m <= lim]
            expect = E[:k] + [-1] * (k - min(k, len(E)))
            assert list(sel[t, b]) == expect, (t, b, list(sel[t, b]), expect)


@pytest.mark.parametrize("N,window,topk,mass,scale,f0,gs,score", [
    (1000, 100, 8, 0.5, 0.0, 0, 0, 0), (1337, 64, 12, 0.9, 0.0, 1, 0, 0), (1000, 100, 8, 0.7, 2.0, 0, 1, 0),
    (700, 1, 30, 0.3, 0.5, 0, 0, 0), (640, 50, 100, 0.8, 0.0, 0, 0, 0), (1000, 100, 8, 0.6, 0.0, 0, 0, 1),
    (300, 5000, 4, 0.5, 0.0, 0, 0, 0)])
def test_adaptive_budget_block_mode(N, window, topk, mass, scale, f0, gs, score):
    # adaptive budget: each query block keeps the shortest prefix of its top-k
    # whose softmax share reaches the mass (max-pair scores, group-shared
    # selection, mean representatives; budgets larger than the candidate set)
    kinds = [HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL, HEAD_SWA, HEAD_RETRIEVAL, HEAD_RETRIEVAL,
             HEAD_RETRIEVAL]
    _compare(_layer(kinds, N, window=window, topk=topk, force_block0=f0, group_select=gs, block_score=score,
                    topk_mass=mass, mass_scale=scale))

