"""Cluster mode (k-means of the low-rank keys) on the GPU against the oracle.

Staged, because fp32 and fp64 Lloyd trajectories may part at near-ties:
  1. assignment of iteration t: the oracle's argmin over the GPU's centroids
     of iteration t-1 must equal the GPU's, except where the exact distances
     to the two centroids differ by <= 1e-5 (|k|^2 + |C|^2);
  2. update: the oracle's means of the GPU's assignment match the GPU's
     centroids within 1e-4;
  3. CSR: bit-exact (members of each cluster in ascending position);
  4. selection: tie band as in block mode; output graded with the GPU's
     validated clusters and selection.
"""
import numpy as np
import pytest
import torch

import hybrid_attention_prefill_amd as ha
import synth
from synth import inputs as si
from oracle.kmeans import assign_step, update_step, sq_dist
from oracle.indexer import cluster_scores, eligible_clusters
from oracle.prefill import layer_prefill
from tests import _gpu

pytestmark = pytest.mark.gpu
KM_REL = 1e-5
CENT_ABS = 1e-4     # in units of the keys' rms (1 for the unit-scale inputs)


def cent_tol(X):
    """Centroid-update tolerance: CENT_ABS times the rms of the low-rank keys,
    so that keys scaled far from unit size are held to the same relative bar."""
    return CENT_ABS * float(np.sqrt(np.mean(np.square(np.asarray(X, dtype=np.float64)))))


def _kmeans_gpu(w, klow, iters):
    Hkv, N, M = w.n_kv_heads, w.n_tokens, w.n_clusters
    d = ha.make_desc(N, w.n_q_heads, Hkv, w.head_dim, window=w.window, topk=w.topk, n_clusters=M,
                     kmeans_iters=iters, kmeans_stride=w.kmeans_stride)
    cent = torch.empty((Hkv, M, 16), dtype=torch.float32, device="cuda")
    asg = torch.empty((Hkv, N), dtype=torch.int32, device="cuda")
    off = torch.empty((Hkv, M + 1), dtype=torch.int32, device="cuda")
    mem = torch.empty((Hkv, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(ha.ha_workspace_bytes(d, w.head_kind), dtype=torch.uint8, device="cuda")
    ha.ha_kmeans(d, klow, cent, asg, off, mem, ws)
    torch.cuda.synchronize()
    return cent.cpu().numpy(), asg.cpu().numpy(), off.cpu().numpy(), mem.cpu().numpy()


def check_assign(X, C, gpu_a, keys, what):
    """Oracle argmin over the given centroids vs the GPU's, for the listed keys."""
    X = X[keys].astype(np.float64)
    C = C.astype(np.float64)
    ora = assign_step(X, C)
    ga = gpu_a[keys].astype(np.int64)
    bad = np.nonzero(ora != ga)[0]
    for t in bad:
        dg = sq_dist(X[t:t + 1], C[ga[t]:ga[t] + 1])[0]
        do = sq_dist(X[t:t + 1], C[ora[t]:ora[t] + 1])[0]
        band = KM_REL * (np.dot(X[t], X[t]) + max(np.dot(C[ga[t]], C[ga[t]]), np.dot(C[ora[t]], C[ora[t]])))
        assert abs(dg - do) <= band, f"{what}: key {keys[t]} GPU cluster {ga[t]} vs oracle {ora[t]} ({dg} vs {do})"
    return bad.size


def check_csr(a, off, mem, M, what):
    N = a.size
    cnt = np.bincount(a, minlength=M)
    np.testing.assert_array_equal(off, np.r_[0, np.cumsum(cnt)], err_msg=what)
    expect = np.lexsort((np.arange(N), a))       # by cluster, then position
    np.testing.assert_array_equal(mem, expect, err_msg=what)


def _kmeans_staged(w, li, iters, key_sample=None, key_scale=None):
    Q, K = _gpu.dev_bf16(li.Q) if li.Q is not None else None, _gpu.dev_bf16(li.K)
    P = _gpu.dev_f32(li.P)
    d = ha.make_desc(w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, window=w.window, topk=w.topk)
    klow = torch.empty((w.n_kv_heads, w.n_tokens, 16), dtype=torch.float32, device="cuda")
    ha.ha_index_project(d, w.head_kind, None, K, P, None, klow)
    if key_scale is not None:
        klow *= key_scale      # test input: low-rank keys far from unit scale
    torch.cuda.synchronize()
    X = klow.cpu().numpy()
    prev = None
    for t in range(1, iters + 1):
        C, a, off, mem = _kmeans_gpu(w, klow, t)
        for g in range(w.n_kv_heads):
            Cp = X[g][np.arange(w.n_clusters) * w.kmeans_stride] if prev is None else prev[0][g]
            keys = np.arange(w.n_tokens) if key_sample is None else key_sample
            nb = check_assign(X[g], Cp, a[g], keys, f"iter {t} kv {g}")
            ref = update_step(X[g].astype(np.float64), a[g].astype(np.int64), Cp.astype(np.float64))
            assert np.max(np.abs(ref - C[g])) <= cent_tol(X[g]), f"iter {t} kv {g}: centroid update off"
            check_csr(a[g], off[g], mem[g], w.n_clusters, f"iter {t} kv {g}")
            print(f"iter {t} kv {g}: {nb} near-tie assignment differences")
        prev = (C, a)
    return X, prev


def test_kmeans_small_every_iteration():
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 8192, n_clusters=128, window=512, n_needles=4)
    print(f"\n[case] kmeans N={w.n_tokens} M={w.n_clusters}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    _kmeans_staged(w, li, 4)


def test_kmeans_degenerate_every_key_a_cluster():
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 512, n_clusters=512, window=64, n_needles=0)
    w = w.with_(kmeans_stride=1)
    print(f"\n[case] kmeans identity N={w.n_tokens}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    X, (C, a) = _kmeans_staged(w, li, 2)
    for g in range(w.n_kv_heads):
        np.testing.assert_array_equal(a[g], np.arange(512))
        np.testing.assert_array_equal(C[g], X[g])


def test_kmeans_ragged_chunks_and_empty_clusters():
    # N not a multiple of the histogram chunk; duplicated keys make some
    # clusters empty after the first assignment (lowest-index rule).
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 9000, n_clusters=300, window=256, n_needles=0)
    w = w.with_(kmeans_stride=30)
    print(f"\n[case] kmeans ragged N={w.n_tokens}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    li.K[30] = li.K[0]     # centroid seeds 0 and 1 coincide
    _kmeans_staged(w, li, 3)


def test_kmeans_equal_centroids_in_different_ranges_take_the_lowest_index():
    # Centroid seeds 5, 700 and 1000 coincide (their key rows are equal) and
    # lie in different ones of the 8 centroid ranges the exact assignment
    # pass spreads its keys over; no key near them can be decided by the
    # one-product pass (best and second equal), so the lowest-index rule must
    # hold across ranges.  Iteration 1: no key may go to 700 or 1000, and the
    # three equal keys go to 5.  Iteration 2: 5 has moved to its members'
    # mean, 700 and 1000 are empty and still equal, so no key may go to 1000
    # and the three equal keys (distance 0 to 700) go to 700.
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 16384, n_clusters=1024, window=512, n_needles=0)
    w = w.with_(kmeans_stride=16)
    print(f"\n[case] kmeans equal centroids across ranges N={w.n_tokens} M={w.n_clusters}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    dup = [5 * 16, 700 * 16, 1000 * 16]
    for j in dup[1:]:
        li.K[j] = li.K[dup[0]]
    K = _gpu.dev_bf16(li.K)
    d = ha.make_desc(w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, window=w.window, topk=w.topk)
    klow = torch.empty((w.n_kv_heads, w.n_tokens, 16), dtype=torch.float32, device="cuda")
    ha.ha_index_project(d, w.head_kind, None, K, _gpu.dev_f32(li.P), None, klow)
    torch.cuda.synchronize()
    X = klow.cpu().numpy()
    C1, a1, _, _ = _kmeans_gpu(w, klow, 1)
    _, a2, _, _ = _kmeans_gpu(w, klow, 2)
    for g in range(w.n_kv_heads):
        assert np.array_equal(X[g][dup[0]], X[g][dup[1]]) and np.array_equal(X[g][dup[0]], X[g][dup[2]])
        assert not np.isin(a1[g], [700, 1000]).any(), f"kv {g}: iteration 1 used a higher equal centroid"
        assert (a1[g][dup] == 5).all(), f"kv {g}: {a1[g][dup]}"
        assert np.array_equal(C1[g][700], C1[g][1000])
        assert not (a2[g] == 1000).any(), f"kv {g}: iteration 2 used centroid 1000 over the equal 700"
        # 5 has moved clearly away (other members) in these inputs: the equal
        # keys, at distance 0 from 700, are no near-tie with it
        c = C1[g].astype(np.float64)
        assert np.sum((c[5] - c[700]) ** 2) > 1e-4 * np.dot(c[700], c[700])
        assert (a2[g][dup] == 700).all(), f"kv {g}: {a2[g][dup]}"


@pytest.mark.parametrize("M", [1, 33, 257, 1000])
def test_kmeans_cluster_counts_and_centroid_ranges(M):
    # cluster counts that leave the exact pass one range (1), ranges smaller
    # than a tile (33), a partial last range (257: ranges of 64) and a partial
    # last tile inside the last of 8 ranges (1000: ranges of 128)
    N = 4096 + 7
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], N, n_clusters=M, window=256, n_needles=0)
    w = w.with_(kmeans_stride=N // M)
    print(f"\n[case] kmeans N={w.n_tokens} M={M}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    _kmeans_staged(w, li, 3)


@pytest.mark.parametrize("scale", [1e4, 2.0 ** 14, 1e-3, 2.0 ** -14, 1e20, 1e-20])
def test_kmeans_key_range(scale):
    # Low-rank keys far from unit scale: each KV head is brought into range by
    # a power of two before the fp16 split, so the staged per-iteration check
    # holds at any finite scale (an unscaled split overflows fp16 above 2^15
    # and loses precision in the fp16 subnormals below 2^-14).
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 8192, n_clusters=128, window=512, n_needles=4)
    print(f"\n[case] kmeans N={w.n_tokens} M={w.n_clusters} key scale {scale:g}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    _kmeans_staged(w, li, 3, key_scale=scale)


def test_kmeans_fp64_lloyd_agreement_reduced_1m():
    """Informational (not graded): the GPU's 10-iteration assignment against an
    independent fp64 Lloyd run from the same seeds, on a 1M-shaped layer
    reduced to 32768 keys and 512 centroids (stride 64).  fp32 and fp64
    trajectories may part at near-ties, so agreement below 100% is expected."""
    w = synth.configs.shrink(synth.WORKLOADS["allsparse_1m"], 32768, n_clusters=512, window=1024, n_needles=4)
    print(f"\n[case] kmeans fp64 agreement N={w.n_tokens} M={w.n_clusters} iters={w.kmeans_iters}", flush=True)
    li = synth.make_layer_inputs(w, with_q=False)
    K = _gpu.dev_bf16(li.K)
    d = ha.make_desc(w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, window=w.window, topk=w.topk)
    klow = torch.empty((w.n_kv_heads, w.n_tokens, 16), dtype=torch.float32, device="cuda")
    ha.ha_index_project(d, w.head_kind, None, K, _gpu.dev_f32(li.P), None, klow)
    C, a, _, _ = _kmeans_gpu(w, klow, w.kmeans_iters)
    from oracle.kmeans import lloyd
    from oracle.indexer import project
    Kf = si.bf16_to_f64(li.K)
    for g in range(w.n_kv_heads):
        _, a64, _ = lloyd(project(Kf[:, g], li.P[g].astype(np.float64)), w.n_clusters, w.kmeans_stride,
                          w.kmeans_iters)
        agree = float(np.mean(a64 == a[g]))
        print(f"kv {g}: GPU vs independent fp64 Lloyd, {w.kmeans_iters} iterations: "
              f"{100 * agree:.2f}% of keys in the same cluster")
        assert 0.0 <= agree <= 1.0


def _layer_cluster(w, blocks=None, p_scale=None):
    print(f"\n[case] cluster layer {w.name} N={w.n_tokens} M={w.n_clusters} k={w.topk} w={w.window}"
          f"{'' if p_scale is None else f' P x {p_scale:g}'}", flush=True)
    li = synth.make_layer_inputs(w)
    if p_scale is not None:
        li.P *= np.float32(p_scale)     # low-rank queries and keys at another scale
    O, _, aux = _gpu.run_gpu(w, li)
    q_rows = lambda a, b: si.bf16_to_f64(li.Q[a:b])
    K, V, P = si.bf16_to_f64(li.K), si.bf16_to_f64(li.V), li.P.astype(np.float64)
    C = aux["centroids"].cpu().numpy()
    asg = aux["assign"].cpu().numpy()
    off = aux["csr_off"].cpu().numpy()
    mem = aux["csr_mem"].cpu().numpy()
    sel = aux["sel"].cpu().numpy()
    _gpu.check_group_rows(sel, w)
    for g in range(w.n_kv_heads):
        _gpu.assert_lowrank(aux["klow"][g].cpu().numpy(), K[:, g] @ P[g], f"klow[{g}]")
        check_csr(asg[g], off[g], mem[g], w.n_clusters, f"kv {g}")
        # final centroids are the means of the final assignment
        Xg = aux["klow"][g].cpu().numpy().astype(np.float64)
        ref = update_step(Xg, asg[g].astype(np.int64), C[g].astype(np.float64))
        assert np.max(np.abs(ref - C[g])) <= cent_tol(Xg)
    km = {g: (C[g], asg[g]) for g in range(w.n_kv_heads)}
    blocks = list(range(w.n_qb)) if blocks is None else blocks
    ref = layer_prefill(w, q_rows, K, V, P, blocks=blocks, kmeans_override=km)
    override = {}
    nd = 0
    for t, h in enumerate(w.ret_heads):
        override[h] = {}
        for b, (E, s) in ref.scored[h].items():
            nd += _gpu.check_sel(w, sel[t, b], E, s, f"head {h} block {b}")
            override[h][b] = np.array([x for x in sel[t, b] if x >= 0], dtype=np.int64)
    print(f"selection near-tie differences: {nd}")
    _gpu.check_lowrank_rows(aux, ref, w, klow_rows=[])
    ref = layer_prefill(w, q_rows, K, V, P, blocks=blocks, kmeans_override=km, sel_override=override)
    mx, mean = _gpu.assert_close_out(O.cpu().numpy()[ref.rows], ref.O, w.name)
    print(f"max abs {mx:.3e}, mean abs {mean:.3e}")
    return li, O, ref


@pytest.mark.parametrize("N,M,window,topk", [(4096, 64, 256, 4), (3000, 50, 100, 8), (5000, 128, 64, 0),
                                             (2048, 32, 4096, 3), (2048, 128, 200, 200)])
def test_cluster_layer_small(N, M, window, topk):
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, N, n_clusters=M, window=window, n_needles=2)
    w = w.with_(kmeans_stride=N // M if N // M >= 1 else 1, topk=topk, kmeans_iters=3)
    _layer_cluster(w)


@pytest.mark.parametrize("N,M,window,topk", [(4096, 64, 256, 4), (3000, 50, 100, 8), (2048, 128, 200, 200)])
def test_group_select_cluster_layer(N, M, window, topk):
    base = synth.WORKLOADS["allsparse_1m_gqa"]
    w = synth.configs.shrink(base, N, n_clusters=M, window=window, n_needles=2)
    w = w.with_(kmeans_stride=N // M, topk=topk, kmeans_iters=3)
    _layer_cluster(w)


@pytest.mark.parametrize("N,M,gs", [(64, 4, 0), (65, 4, 1), (130, 8, 0), (200, 3, 1)])
def test_cluster_tiny_sequences(N, M, gs):
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, N, n_clusters=M, window=64, n_needles=1)
    w = w.with_(kmeans_stride=N // M, topk=2, kmeans_iters=2, group_select=gs)
    _layer_cluster(w)


@pytest.mark.parametrize("p_scale", [1e4, 1e-3])
def test_cluster_layer_scaled_projection(p_scale):
    # the whole layer with low-rank vectors 1e4 / 1e-3 times the unit scale
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, 4096, n_clusters=64, window=256, n_needles=2)
    w = w.with_(kmeans_stride=64, topk=4, kmeans_iters=3)
    _layer_cluster(w, p_scale=p_scale)


@pytest.mark.parametrize("N,M,window,topk,mass,gs", [(4096, 64, 256, 8, 0.5, 0), (3000, 50, 100, 12, 0.9, 1),
                                                    (2048, 128, 200, 200, 0.7, 0)])
def test_cluster_layer_adaptive_budget(N, M, window, topk, mass, gs):
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, N, n_clusters=M, window=window, n_needles=2)
    w = w.with_(kmeans_stride=N // M, topk=topk, kmeans_iters=3, topk_mass=mass, group_select=gs)
    _layer_cluster(w)


def test_group_select_cluster_mixed_with_swa_heads():
    base = synth.WORKLOADS["allsparse_1m_gqa"]
    kinds = tuple(1 if h % 3 == 0 else 0 for h in range(16))
    w = synth.configs.shrink(base, 6000, n_clusters=96, window=300, n_needles=2)
    w = w.with_(head_kind=kinds, kmeans_stride=62, topk=6, kmeans_iters=2)
    _layer_cluster(w)


def test_cluster_layer_mixed_with_swa_heads():
    base = synth.WORKLOADS["allsparse_1m"]
    kinds = tuple(1 if h % 3 == 0 else 0 for h in range(16))
    w = synth.configs.shrink(base, 6000, n_clusters=96, window=300, n_needles=2)
    w = w.with_(head_kind=kinds, kmeans_stride=62, topk=6, kmeans_iters=2)
    _layer_cluster(w)


def test_cluster_layer_reduced_allsparse_needles_found():
    base = synth.WORKLOADS["allsparse_1m"]
    w = synth.configs.shrink(base, 32768, n_clusters=512, window=1024, n_needles=16)
    nd = si.needles(w)
    blocks = sorted(set(int(r) // 64 for r in nd.q_row))[:12]
    li, O, ref = _layer_cluster(w, blocks=blocks)
