"""The C-ABI library: it loads without a GPU, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import hybrid_attention_prefill_amd as ha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ha_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree_and_library_exports_all():
    decl = _declared()
    assert set(decl) == set(ha.EXPORTS)
    L = ha.lib()
    for name in decl:
        assert hasattr(L, name), name
    assert L.ha_version() == 6


def test_status_strings():
    for c in range(6):
        assert ha.status_string(c).startswith("HA_")
    assert "unknown" in ha.status_string(99)


def _desc(**kw):
    base = dict(n_tokens=1000, n_q_heads=8, n_kv_heads=2, head_dim=128, window=64)
    base.update(kw)
    n, hq, hkv, d = base.pop("n_tokens"), base.pop("n_q_heads"), base.pop("n_kv_heads"), base.pop("head_dim")
    return ha.make_desc(n, hq, hkv, d, **base)


FAKE = 0x1000  # never dereferenced: every case below fails validation first


def _band(desc, kinds, Q=FAKE, K=FAKE, V=FAKE, O=FAKE):
    return ha.lib().ha_attn_band(ctypes.byref(desc), ha._kinds(kinds), Q, K, V, O, None, 0, None)


@pytest.mark.parametrize("kw,kinds,code", [
    (dict(n_q_heads=6, n_kv_heads=4), [0] * 6, ha.HA_ERR_ARG),          # Hq % Hkv
    (dict(n_tokens=0), [0] * 8, ha.HA_ERR_ARG),
    (dict(head_dim=64), [0] * 8, ha.HA_ERR_UNSUPPORTED),
    (dict(head_dim=0), [0] * 8, ha.HA_ERR_ARG),
    (dict(q_block=32, k_block=32), [0] * 8, ha.HA_ERR_UNSUPPORTED),
    (dict(), [0] * 7 + [9], ha.HA_ERR_ARG),                               # unknown kind
    (dict(window=0), [0] * 8, ha.HA_ERR_ARG),                             # SWA needs w >= 1
    (dict(sink=-1), [2] * 8, ha.HA_ERR_ARG),
    (dict(n_q_heads=512, n_kv_heads=2), [0] * 512, ha.HA_ERR_UNSUPPORTED),
    (dict(n_q_heads=256, n_kv_heads=2), [0] * 256, ha.HA_ERR_UNSUPPORTED),  # head ids are bytes, 0xFF = empty
])
def test_band_rejects(kw, kinds, code):
    assert _band(_desc(**kw), kinds) == code


def test_band_null_pointers():
    d = _desc()
    assert _band(d, [0] * 8, Q=None) == ha.HA_ERR_ARG
    assert _band(d, [0] * 8, O=None) == ha.HA_ERR_ARG
    assert ha.lib().ha_attn_band(None, ha._kinds([0] * 8), FAKE, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_ARG
    assert ha.lib().ha_attn_band(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_ARG


def test_dense_heads_need_no_window():
    # a dense-only layer with window 0 passes validation: the workspace query says so
    assert ha.ha_workspace_bytes(_desc(window=0), [3] * 8) >= 0
    assert ha.ha_workspace_bytes(_desc(window=0), [0] * 8) == 0   # invalid -> 0


def _prefill(desc, kinds, P=FAKE, xs=None, xo=None, Oo=None, ws=None, wsb=0):
    return ha.lib().ha_prefill(ctypes.byref(desc), ha._kinds(kinds), FAKE, FAKE, FAKE, P, xs, xo, FAKE, Oo,
                               None, ws, wsb, None)


def test_prefill_retrieval_argument_checks():
    kinds = [1, 1] + [0] * 6
    d = _desc(topk=8)
    assert _prefill(d, kinds, P=None) == ha.HA_ERR_ARG                       # P required
    assert _prefill(_desc(topk=8, rank=8), kinds) == ha.HA_ERR_UNSUPPORTED
    assert _prefill(_desc(topk=-1), kinds) == ha.HA_ERR_ARG
    assert _prefill(_desc(topk=8, force_block0=2), kinds) == ha.HA_ERR_ARG
    assert _prefill(_desc(topk=100000), kinds) == ha.HA_ERR_UNSUPPORTED
    # workspace: needed, missing -> HA_ERR_WORKSPACE
    need = ha.ha_workspace_bytes(d, kinds)
    assert need > 0
    assert _prefill(d, kinds, ws=None, wsb=0) == ha.HA_ERR_WORKSPACE
    assert _prefill(d, kinds, ws=FAKE, wsb=need - 1) == ha.HA_ERR_WORKSPACE
    assert _prefill(d, kinds, ws=FAKE + 8, wsb=need) == ha.HA_ERR_WORKSPACE  # misaligned


def test_prefill_cluster_argument_checks():
    kinds = [1] * 8
    # M * stride > N
    assert _prefill(_desc(topk=4, n_clusters=100, kmeans_iters=2, kmeans_stride=20), kinds) == ha.HA_ERR_ARG
    # iterations must be >= 1
    assert _prefill(_desc(topk=4, n_clusters=10, kmeans_iters=0, kmeans_stride=2), kinds) == ha.HA_ERR_ARG
    # more clusters than the selection kernel scores in LDS
    big = _desc(n_tokens=1 << 20, topk=4, n_clusters=20000, kmeans_iters=1, kmeans_stride=2)
    assert _prefill(big, kinds) == ha.HA_ERR_UNSUPPORTED
    # block 0 is a block-mode rule
    assert _prefill(_desc(topk=4, n_clusters=10, kmeans_iters=2, kmeans_stride=2, force_block0=1),
                    kinds) == ha.HA_ERR_UNSUPPORTED
    L = ha.lib()
    d = _desc(topk=4, n_clusters=10, kmeans_iters=2, kmeans_stride=2)
    assert L.ha_kmeans(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ha.HA_ERR_ARG
    assert L.ha_kmeans(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_WORKSPACE
    assert L.ha_select_clusters(ctypes.byref(d), ha._kinds(kinds), FAKE, FAKE, None, FAKE, FAKE, None, 0,
                                None) == ha.HA_ERR_ARG


def test_prefill_orthros_argument_checks():
    kinds = [0] * 8
    d = _desc(n_out=1)
    assert _prefill(d, kinds, xs=FAKE, xo=None, Oo=FAKE) == ha.HA_ERR_ARG
    assert _prefill(d, kinds, xs=FAKE, xo=FAKE, Oo=None) == ha.HA_ERR_ARG
    assert _prefill(_desc(n_out=2000), kinds, xs=FAKE, xo=FAKE, Oo=FAKE) == ha.HA_ERR_ARG
    # any group size (G = 17 here) passes the checks; the split-key partials
    # then need a workspace
    d17 = _desc(n_q_heads=34, n_kv_heads=2, n_out=1)
    assert ha.lib().ha_workspace_bytes(ctypes.byref(d17), ha._kinds([0] * 34)) > 0
    assert _prefill(d17, [0] * 34, xs=FAKE, xo=FAKE, Oo=FAKE) == ha.HA_ERR_WORKSPACE


def test_stage_argument_checks():
    L = ha.lib()
    d = _desc(topk=8)
    kinds = ha._kinds([1, 1] + [0] * 6)
    assert L.ha_index_project(ctypes.byref(d), kinds, FAKE, FAKE, None, FAKE, FAKE, None) == ha.HA_ERR_ARG
    assert L.ha_index_project(ctypes.byref(d), ha._kinds([0] * 8), FAKE, FAKE, FAKE, FAKE, FAKE, None) == ha.HA_ERR_ARG
    assert L.ha_select_blocks(ctypes.byref(d), kinds, FAKE, None, FAKE, None, 0, None) == ha.HA_ERR_ARG
    # block representatives need their workspace
    d_rep = _desc(topk=8, block_score=1)
    assert L.ha_select_blocks(ctypes.byref(d_rep), kinds, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_WORKSPACE
    assert L.ha_select_blocks(ctypes.byref(_desc(topk=8, block_score=3)), kinds, FAKE, FAKE, FAKE, None, 0,
                              None) == ha.HA_ERR_ARG
    assert L.ha_attn_gather(ctypes.byref(d), kinds, FAKE, FAKE, FAKE, None, None, None, FAKE, None, 0, None) == ha.HA_ERR_ARG
    dc = _desc(n_out=1)
    assert L.ha_attn_cross(ctypes.byref(dc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_WORKSPACE
    assert L.ha_attn_cross(ctypes.byref(_desc(n_out=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ha.HA_ERR_ARG


def test_binding_raises_on_error():
    with pytest.raises(ha.HAError) as ei:
        ha.ha_attn_band(_desc(head_dim=64), [0] * 8, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.code == ha.HA_ERR_UNSUPPORTED


def test_static_entry_point_rejects_layers_beyond_its_scratch():
    # the 1M cluster-mode layer needs ~2.4 GB of scratch: rejected on the host,
    # before any HIP call (no GPU needed)
    import synth
    w = synth.WORKLOADS["allsparse_1m"]
    d = ha.make_desc(w.n_tokens, w.n_q_heads, w.n_kv_heads, 128, window=w.window, topk=w.topk,
                     n_clusters=w.n_clusters, kmeans_iters=w.kmeans_iters, kmeans_stride=w.kmeans_stride)
    assert ha.ha_workspace_bytes(d, w.head_kind) > ha.HA_STATIC_SCRATCH_BYTES
    rc = ha.lib().ha_prefill_static(ctypes.byref(d), ha._kinds(w.head_kind), FAKE, FAKE, FAKE, FAKE, None, None,
                                    FAKE, None, None, None)
    assert rc == ha.HA_ERR_SCRATCH
    # argument errors come first
    rc = ha.lib().ha_prefill_static(ctypes.byref(d), ha._kinds(w.head_kind), FAKE, FAKE, FAKE, None, None, None,
                                    FAKE, None, None, None)
    assert rc == ha.HA_ERR_ARG
    # the default workloads that fit: every one but the 1M layers
    for name, wl in synth.WORKLOADS.items():
        dd = ha.make_desc(wl.n_tokens, wl.n_q_heads, wl.n_kv_heads, 128, **{
            k: v for k, v in wl.desc_dict().items()
            if k not in ("n_tokens", "n_q_heads", "n_kv_heads", "head_dim")})
        fits = ha.ha_workspace_bytes(dd, wl.head_kind) <= ha.HA_STATIC_SCRATCH_BYTES
        assert fits == (wl.n_tokens < (1 << 20)), name

