"""GPU-side helpers for the parity tests: device copies of the seeded inputs,
a run of the C-ABI path, and the comparison rules.

Comparison rules (stated for bf16 inputs with fp32 accumulation):
  outputs     max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3
  low-rank    |gpu - oracle| <= 1e-5 * ||oracle row||_2 per row
  selections  equal sets, except candidates whose oracle score is within
              1e-3 * |tau| of the oracle's k-th best score tau (near ties)
"""
import numpy as np

import hybrid_attention_prefill_amd as ha
from synth import inputs as si

OUT_MAX, OUT_MEAN = 2e-2, 2e-3
LOWRANK_REL = 1e-5
TIE_REL = 1e-3
MASS_DELTA = 1e-3   # adaptive budget: tolerance on the cumulative share at the cut


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def run_gpu(w, li, return_aux=True):
    """The whole layer through ha_prefill on the current stream."""
    import torch
    Q, K, V = dev_bf16(li.Q), dev_bf16(li.K), dev_bf16(li.V)
    P = dev_f32(li.P) if li.P is not None else None
    xs = dev_f32(li.xa_scale) if li.xa_scale is not None else None
    xo = dev_f32(li.xa_offset) if li.xa_offset is not None else None
    res = ha.hybrid_attn_prefill(
        Q, K, V, w.head_kind, w.window, P, topk=w.topk, block=w.q_block, force_block0=w.force_block0,
        n_clusters=w.n_clusters, kmeans_iters=w.kmeans_iters, kmeans_stride=w.kmeans_stride,
        sink=w.sink, last_q=w.last_q, n_out=w.n_out, group_select=w.group_select, block_score=w.block_score,
        index_bits=w.index_bits, topk_mass=w.topk_mass, mass_scale=w.mass_scale, xa_scale=xs, xa_offset=xo,
        return_aux=return_aux and bool(w.ret_heads))
    torch.cuda.synchronize()
    if not isinstance(res, tuple):
        res = (res,)
    O = res[0]
    O_out = res[1] if w.n_out > 0 else None
    aux = res[-1] if (return_aux and w.ret_heads) else None
    return O, O_out, aux


def assert_close_out(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert mx <= OUT_MAX and mean <= OUT_MEAN, f"{what}: max abs {mx:.3g}, mean abs {mean:.3g}"
    return mx, mean


def assert_lowrank(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    nrm = np.linalg.norm(ref, axis=-1, keepdims=True)
    bad = np.abs(gpu - ref) > LOWRANK_REL * np.maximum(nrm, 1e-30)
    assert not bad.any(), f"{what}: {int(bad.sum())} low-rank entries off"


def check_group_rows(sel, w):
    """Group-shared selection: the retrieval heads of a KV group hold equal rows."""
    if not w.group_select:
        return
    G = w.n_q_heads // w.n_kv_heads
    first = {}
    for t, h in enumerate(w.ret_heads):
        g = h // G
        if g in first:
            np.testing.assert_array_equal(sel[t], sel[first[g]], err_msg=f"head {h} vs group {g} row")
        else:
            first[g] = t


def check_selection(gpu_sel, eligible, scores, k, what=""):
    """gpu_sel: GPU row (ascending, -1 padded); eligible/scores: oracle's."""
    g = [int(x) for x in gpu_sel if x >= 0]
    assert g == sorted(g), f"{what}: selection not ascending"
    assert len(set(g)) == len(g), f"{what}: duplicate ids"
    kk = min(k, len(eligible))
    assert len(g) == kk, f"{what}: {len(g)} selected, expected {kk}"
    if kk == 0:
        return 0
    order = np.lexsort((eligible, -scores))
    tau = scores[order[kk - 1]]
    ref = set(int(x) for x in eligible[order[:kk]])
    sc = dict(zip((int(x) for x in eligible), scores))
    diff = ref.symmetric_difference(g)
    for c in diff:
        assert c in sc, f"{what}: block {c} not eligible"
        assert abs(sc[c] - tau) <= TIE_REL * max(abs(tau), 1e-30), \
            f"{what}: block {c} (score {sc[c]:.6g}) differs from the oracle outside the tie band (tau {tau:.6g})"
    return len(diff)


def check_lowrank_rows(aux, ref, w, heads=None, klow_rows=None):
    """Staged parity, stage 1: the GPU's low-rank queries (every row the oracle
    computed) and keys (all rows, or the listed ones) against the oracle's."""
    qlow = aux["qlow"].cpu().numpy()
    klow = aux["klow"].cpu().numpy()
    n = 0
    for t, h in enumerate(w.ret_heads):
        if heads is not None and h not in heads:
            continue
        for b, ql in ref.qlow.get(h, {}).items():
            rows = np.arange(b * w.q_block, min(w.n_tokens, (b + 1) * w.q_block))
            assert_lowrank(qlow[t][rows], ql, f"qlow head {h} block {b}")
            n += rows.size
    for g, kl in ref.klow.items():
        rows = np.arange(w.n_tokens) if klow_rows is None else np.asarray(klow_rows, dtype=np.int64)
        assert_lowrank(klow[g][rows], kl[rows], f"klow[{g}]")
    return n


def fails_tolerance(candidate, ref):
    """True when `candidate` would be rejected against `ref` by the output rule
    (max abs > OUT_MAX or mean abs > OUT_MEAN): the discrimination check that
    the tolerances reject a trivially wrong answer."""
    err = np.abs(np.asarray(candidate, dtype=np.float64) - ref)
    return bool(err.max() > OUT_MAX or err.mean() > OUT_MEAN)


def check_selection_adaptive(gpu_sel, eligible, scores, k, mass, scale, what=""):
    """Adaptive budget: the GPU keeps n of the oracle's top-k budget; n must be
    a cut the oracle's shares allow (the share of the first n reaches the
    mass, that of the first n - 1 does not, both within MASS_DELTA: fp32 and
    fp64 shares differ slightly), and the kept ids a valid top-n (tie band)."""
    g = [int(x) for x in gpu_sel if x >= 0]
    kk = min(k, len(eligible))
    if kk == 0:
        assert not g, f"{what}: selected from an empty candidate set"
        return 0
    order = np.lexsort((eligible, -scores))[:kk]
    sc = np.asarray(scores, dtype=np.float64)[order]
    wts = np.exp(scale * (sc - sc[0]))
    share = np.cumsum(wts) / np.sum(wts)
    n = len(g)
    assert 1 <= n <= kk, f"{what}: {n} kept of a budget of {kk}"
    assert share[n - 1] >= mass - MASS_DELTA, f"{what}: {n} kept reach share {share[n - 1]:.6f} < {mass}"
    assert n == 1 or share[n - 2] < mass + MASS_DELTA, \
        f"{what}: {n - 1} would already reach {share[n - 2]:.6f} >= {mass}"
    return check_selection(gpu_sel, eligible, scores, n, what)


def check_sel(w, gpu_sel, eligible, scores, what=""):
    """The selection rule of workload w: fixed top-k or the adaptive budget."""
    if 0.0 < w.topk_mass < 1.0:
        scale = w.mass_scale if w.mass_scale > 0 else 1.0 / np.sqrt(w.rank)
        return check_selection_adaptive(gpu_sel, eligible, scores, w.topk, w.topk_mass, scale, what)
    return check_selection(gpu_sel, eligible, scores, w.topk, what)

