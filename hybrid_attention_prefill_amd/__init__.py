"""Head-wise hybrid attention prefill for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libha.so`` (the C ABI in ``include/ha.h``).  It
only marshals arguments: device pointers of torch tensors, the current HIP
stream, and the layer descriptor.  Every step of the computation runs in the
library's HIP kernels; there is no Python or CPU fallback.  Importing works
without a GPU (argument checks run on the host); if the library has not been
built, every call raises.

Names follow the C entry points (``ha_prefill``, ``ha_index_project``, ...)
plus the convenience call ``hybrid_attn_prefill``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libha.so")

HA_SWA, HA_RETRIEVAL, HA_TRIANGLE, HA_DENSE = 0, 1, 2, 3
HA_OK, HA_ERR_ARG, HA_ERR_UNSUPPORTED, HA_ERR_WORKSPACE, HA_ERR_DEVICE, HA_ERR_SCRATCH = range(6)
HA_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("ha_status_string", "ha_version", "ha_workspace_bytes", "ha_prefill", "ha_prefill_static",
           "ha_index_project", "ha_select_blocks", "ha_quantize_keys", "ha_kmeans", "ha_select_clusters",
           "ha_attn_band", "ha_attn_gather", "ha_attn_cross")


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("window", ctypes.c_int32),
        ("rank", ctypes.c_int32), ("q_block", ctypes.c_int32), ("k_block", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("force_block0", ctypes.c_int32),
        ("n_clusters", ctypes.c_int32), ("kmeans_iters", ctypes.c_int32),
        ("kmeans_stride", ctypes.c_int32), ("sink", ctypes.c_int32),
        ("last_q", ctypes.c_int32), ("n_out", ctypes.c_int32),
        ("group_select", ctypes.c_int32), ("block_score", ctypes.c_int32), ("index_bits", ctypes.c_int32),
        ("topk_mass", ctypes.c_float), ("mass_scale", ctypes.c_float),
    ]


class Aux(ctypes.Structure):
    _fields_ = [("sel", ctypes.c_void_p), ("qlow", ctypes.c_void_p), ("klow", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("assign", ctypes.c_void_p),
                ("csr_off", ctypes.c_void_p), ("csr_mem", ctypes.c_void_p)]


class HAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hybrid_attention_prefill_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p = ctypes.c_void_p, ctypes.c_void_p
        dp = ctypes.POINTER(LayerDesc)
        L.ha_status_string.restype = ctypes.c_char_p
        L.ha_status_string.argtypes = [ctypes.c_int]
        L.ha_version.restype = ctypes.c_int
        L.ha_workspace_bytes.restype = ctypes.c_size_t
        L.ha_workspace_bytes.argtypes = [dp, i32p]
        L.ha_prefill.restype = ctypes.c_int
        L.ha_prefill.argtypes = [dp, i32p, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Aux), vp,
                                 ctypes.c_size_t, vp]
        L.ha_prefill_static.restype = ctypes.c_int
        L.ha_prefill_static.argtypes = [dp, i32p, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Aux), vp]
        L.ha_index_project.restype = ctypes.c_int
        L.ha_index_project.argtypes = [dp, i32p, vp, vp, vp, vp, vp, vp]
        L.ha_select_blocks.restype = ctypes.c_int
        L.ha_select_blocks.argtypes = [dp, i32p, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ha_quantize_keys.restype = ctypes.c_int
        L.ha_quantize_keys.argtypes = [dp, vp, vp, vp, vp]
        L.ha_kmeans.restype = ctypes.c_int
        L.ha_kmeans.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ha_select_clusters.restype = ctypes.c_int
        L.ha_select_clusters.argtypes = [dp, i32p, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ha_attn_band.restype = ctypes.c_int
        L.ha_attn_band.argtypes = [dp, i32p, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ha_attn_gather.restype = ctypes.c_int
        L.ha_attn_gather.argtypes = [dp, i32p, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.ha_attn_cross.restype = ctypes.c_int
        L.ha_attn_cross.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().ha_status_string(int(code)).decode()


def _check(code: int):
    if code != HA_OK:
        raise HAError(code, status_string(code))


# ---------------------------------------------------------------------------
# marshalling helpers


def _ptr(x) -> Optional[int]:
    """Device (or host) address of a tensor / raw int; None for None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def make_desc(n_tokens, n_q_heads, n_kv_heads, head_dim=128, *, softmax_scale=0.0, window=0, rank=16,
              q_block=64, k_block=64, topk=0, force_block0=0, n_clusters=0, kmeans_iters=0,
              kmeans_stride=0, sink=0, last_q=0, n_out=0, group_select=0, block_score=0,
              index_bits=0, topk_mass=0.0, mass_scale=0.0) -> LayerDesc:
    return LayerDesc(n_tokens, n_q_heads, n_kv_heads, head_dim, float(softmax_scale or 0.0), window, rank,
                     q_block, k_block, topk, int(force_block0), n_clusters, kmeans_iters, kmeans_stride,
                     sink, last_q, n_out, int(group_select), int(block_score), int(index_bits),
                     float(topk_mass), float(mass_scale))


def _kinds(head_kind: Sequence[int]):
    arr = (ctypes.c_int32 * len(head_kind))(*[int(k) for k in head_kind])
    return arr


def ha_workspace_bytes(desc: LayerDesc, head_kind: Sequence[int]) -> int:
    return int(lib().ha_workspace_bytes(ctypes.byref(desc), _kinds(head_kind)))


def _aux(aux):
    return None if aux is None else Aux(*[_ptr(aux.get(f)) for f, _ in Aux._fields_])


def ha_prefill(desc, head_kind, Q, K, V, P_idx, xa_scale, xa_offset, O, O_out, aux=None,
               workspace=None, ws_bytes=None, stream=None):
    a = _aux(aux)
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_prefill(ctypes.byref(desc), _kinds(head_kind), _ptr(Q), _ptr(K), _ptr(V), _ptr(P_idx),
                            _ptr(xa_scale), _ptr(xa_offset), _ptr(O), _ptr(O_out),
                            ctypes.byref(a) if a is not None else None, _ptr(workspace), int(ws_bytes),
                            _stream(stream)))


def ha_prefill_static(desc, head_kind, Q, K, V, P_idx, xa_scale, xa_offset, O, O_out, aux=None, stream=None):
    """ha_prefill without a workspace: the library's static device scratch."""
    a = _aux(aux)
    _check(lib().ha_prefill_static(ctypes.byref(desc), _kinds(head_kind), _ptr(Q), _ptr(K), _ptr(V), _ptr(P_idx),
                                   _ptr(xa_scale), _ptr(xa_offset), _ptr(O), _ptr(O_out),
                                   ctypes.byref(a) if a is not None else None, _stream(stream)))


def ha_index_project(desc, head_kind, Q, K, P_idx, qlow, klow, stream=None):
    _check(lib().ha_index_project(ctypes.byref(desc), _kinds(head_kind), _ptr(Q), _ptr(K), _ptr(P_idx),
                                  _ptr(qlow), _ptr(klow), _stream(stream)))


def ha_select_blocks(desc, head_kind, qlow, klow, sel, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_select_blocks(ctypes.byref(desc), _kinds(head_kind), _ptr(qlow), _ptr(klow), _ptr(sel),
                                  _ptr(workspace), int(ws_bytes), _stream(stream)))


def ha_quantize_keys(desc, klow, codes, scales, stream=None):
    _check(lib().ha_quantize_keys(ctypes.byref(desc), _ptr(klow), _ptr(codes), _ptr(scales), _stream(stream)))


def ha_kmeans(desc, klow, centroids, assign, csr_off, csr_mem, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_kmeans(ctypes.byref(desc), _ptr(klow), _ptr(centroids), _ptr(assign), _ptr(csr_off),
                           _ptr(csr_mem), _ptr(workspace), int(ws_bytes), _stream(stream)))


def ha_select_clusters(desc, head_kind, qlow, centroids, csr_off, csr_mem, sel, workspace=None, ws_bytes=None,
                       stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_select_clusters(ctypes.byref(desc), _kinds(head_kind), _ptr(qlow), _ptr(centroids),
                                    _ptr(csr_off), _ptr(csr_mem), _ptr(sel), _ptr(workspace), int(ws_bytes),
                                    _stream(stream)))


def ha_attn_band(desc, head_kind, Q, K, V, O, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_attn_band(ctypes.byref(desc), _kinds(head_kind), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                              _ptr(workspace), int(ws_bytes), _stream(stream)))


def ha_attn_gather(desc, head_kind, Q, K, V, sel, csr_off, csr_mem, O, workspace=None, ws_bytes=None,
                   stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_attn_gather(ctypes.byref(desc), _kinds(head_kind), _ptr(Q), _ptr(K), _ptr(V), _ptr(sel),
                                _ptr(csr_off), _ptr(csr_mem), _ptr(O), _ptr(workspace), int(ws_bytes),
                                _stream(stream)))


def ha_attn_cross(desc, Q, K, V, xa_scale, xa_offset, O_out, workspace=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ha_attn_cross(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(xa_scale), _ptr(xa_offset),
                               _ptr(O_out), _ptr(workspace), int(ws_bytes), _stream(stream)))


# ---------------------------------------------------------------------------
# convenience entry point


def hybrid_attn_prefill(Q, K, V, head_kind, window, P_idx=None, topk=0, block=64, *, force_block0=False,
                        n_clusters=0, kmeans_iters=10, kmeans_stride=64, sink=0, last_q=0, n_out=0,
                        group_select=False, block_score=0, index_bits=0, topk_mass=0.0, mass_scale=0.0,
                        xa_scale=None, xa_offset=None,
                        softmax_scale=None, out=None, out_cross=None, workspace=None, return_aux=False):
    """One layer's hybrid attention prefill on the current HIP stream.

    Q [N, Hq, D], K/V [N, Hkv, D] bf16 CUDA tensors; head_kind a sequence of
    HA_* values per query head.  Returns O [N, Hq, D] fp32, plus O_out
    [n_out, Hq, D] when n_out > 0, plus a dict of indexer intermediates when
    return_aux.  Allocation of outputs and workspace is done here with torch;
    everything else is the library's.
    """
    import torch
    N, Hq, D = Q.shape
    Hkv = K.shape[1]
    desc = make_desc(N, Hq, Hkv, D, softmax_scale=softmax_scale or 0.0, window=window, topk=topk,
                     q_block=block, k_block=block, force_block0=int(bool(force_block0)),
                     n_clusters=n_clusters, kmeans_iters=kmeans_iters if n_clusters else 0,
                     kmeans_stride=kmeans_stride if n_clusters else 0, sink=sink, last_q=last_q, n_out=n_out,
                     group_select=int(bool(group_select)), block_score=int(block_score),
                     index_bits=int(index_bits), topk_mass=topk_mass, mass_scale=mass_scale)
    dev = Q.device
    O = out if out is not None else torch.empty((N, Hq, D), dtype=torch.float32, device=dev)
    O_out = None
    if n_out > 0:
        O_out = out_cross if out_cross is not None else torch.empty((n_out, Hq, D), dtype=torch.float32, device=dev)
    ws_need = ha_workspace_bytes(desc, head_kind)
    if ws_need == 0 and workspace is None:
        # invalid descriptor: let the library report the precise error
        ws = None
    else:
        ws = workspace if workspace is not None else torch.empty(ws_need, dtype=torch.uint8, device=dev)
    aux = None
    if return_aux:
        n_ret = sum(1 for k in head_kind if int(k) == HA_RETRIEVAL)
        nqb = (N + block - 1) // block
        aux = dict(sel=torch.empty((n_ret, nqb, max(topk, 0)), dtype=torch.int32, device=dev),
                   qlow=torch.empty((n_ret, N, 16), dtype=torch.float32, device=dev),
                   klow=torch.empty((Hkv, N, 16), dtype=torch.float32, device=dev))
        if n_clusters:
            aux.update(centroids=torch.empty((Hkv, n_clusters, 16), dtype=torch.float32, device=dev),
                       assign=torch.empty((Hkv, N), dtype=torch.int32, device=dev),
                       csr_off=torch.empty((Hkv, n_clusters + 1), dtype=torch.int32, device=dev),
                       csr_mem=torch.empty((Hkv, N), dtype=torch.int32, device=dev))
    ha_prefill(desc, head_kind, Q, K, V, P_idx, xa_scale, xa_offset, O, O_out, aux, ws, None)
    res = [O]
    if n_out > 0:
        res.append(O_out)
    if return_aux:
        res.append(aux)
    return res[0] if len(res) == 1 else tuple(res)
