#!/usr/bin/env python3
"""Benchmark of head-wise hybrid attention prefill on one MI355X.

A step is one pass of the hot path over a suite of single attention layers
(synthetic bf16 inputs, resident in HBM before timing starts):

  qwen3_30b_a3b_32k         5 retrieval heads (rank-16 indexer, top-32 key blocks
                            + window 8192) and 27 SWA heads, N = 32768
  trianglemix_llama8b_128k  TriangleMix layer (sink 64, band 2048, last 128 rows),
                            32 q / 8 kv heads, N = 131072
  dense_llama8b_128k        dense causal layer of the same shape
  orthros_8b_128k           SWA 4096 for all rows + cross-attention for the last row
  allsparse_1m              all 16 heads retrieval, k-means clusters (1M tokens)

Every stage is a call of the C ABI on the current stream with HIP events
between stages; per-layer and per-stage times come from those events.  The
printed JSON line carries the aggregate actual-attention TFLOP/s, per-layer
ms and TFLOP/s, the roofline of the dominant kernel and the fp64 CPU oracle
timed on a bounded sample (rank 0, N=1 only).

  python bench.py [--steps K] [--warmup W] [--workloads a,b] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid-attn prefill ms/layer + TFLOP/s (% MFMA peak) at 128K and 1M tokens"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
DEFAULT_SUITE = ["qwen3_30b_a3b_32k", "trianglemix_llama8b_128k", "dense_llama8b_128k",
                 "orthros_8b_128k", "allsparse_1m"]
COPY_CAL_BYTES = 1 << 30
# HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE,
# KiB per dispatch, scaled by the same counters on a plain 1 GiB copy); valid
# only while the kernel source is the one the counters were taken on.
TRAFFIC = {
    ("dense_llama8b_128k", "attn_band"): {
        "bytes": 20688568621, "source": "hybrid_attention_prefill_amd/csrc/attn.hip",
        "sha256_prefix": "385622c8e0ec6f6e"},
}


def traffic_for(workload, stage):
    import hashlib
    t = TRAFFIC.get((workload, stage))
    if t is None:
        return None
    try:
        with open(os.path.join(ROOT, t["source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return t["bytes"] if sha.startswith(t["sha256_prefix"]) else None


# ---------------------------------------------------------------------------
# exact work accounting (host, from the realised key sets)


def pairs_swa(N, w):
    i = np.arange(N, dtype=np.int64)
    return int(np.minimum(w, i + 1).sum())


def pairs_dense(N):
    return N * (N + 1) // 2


def pairs_triangle(N, sink, w, last):
    i = np.arange(N, dtype=np.int64)
    band = np.minimum(w, i + 1)
    # sink keys j < sink that are not already in the band (j <= i - w)
    extra = np.clip(np.minimum(sink, i - w + 1), 0, None)
    rows = np.where(i >= N - last, i + 1, band + extra)
    return int(rows.sum())


def pairs_retrieval_blocks(N, w, sel_rows, f0, Bk=64, Bq=64):
    """Pairs of one retrieval head: window + selected/forced blocks (keys j <= i-w)."""
    total = pairs_swa(N, w)
    n_qb = sel_rows.shape[0]
    for b in range(n_qb):
        rows = np.arange(b * Bq, min(N, (b + 1) * Bq), dtype=np.int64)
        blocks = [int(c) for c in sel_rows[b] if c >= 0]
        if f0:
            blocks.append(0)
        for c in set(blocks):
            lo = c * Bk
            hi = np.minimum(lo + Bk - 1, rows - w)
            total += int(np.clip(hi - lo + 1, 0, None).sum())
    return total


def pairs_retrieval_clusters(N, w, sel_rows, csr_off, csr_mem, Bq=64):
    """Pairs of one retrieval head in cluster mode: window + members j <= i-w
    of the selected clusters, from the CSR (members ascending per cluster).
    For rows [qs, qe] of a block and a cluster with C(x) = #members <= x and
    S(x) = sum of members <= x:
      pairs = n*C(qs-w) + (qe-w+1)*(C(qe-w) - C(qs-w)) - (S(qe-w) - S(qs-w))."""
    total = pairs_swa(N, w)
    n_qb, k = sel_rows.shape
    M = csr_off.size - 1
    clus = np.repeat(np.arange(M, dtype=np.int64), np.diff(csr_off))
    keyv = clus * (N + 1) + csr_mem.astype(np.int64)          # ascending
    csum = np.r_[0, np.cumsum(csr_mem.astype(np.int64))]
    b = np.repeat(np.arange(n_qb, dtype=np.int64), k)
    m = sel_rows.reshape(-1).astype(np.int64)
    ok = m >= 0
    b, m = b[ok], m[ok]
    qs = b * Bq
    qe = np.minimum(N, qs + Bq) - 1
    n = qe - qs + 1

    def CS(x):
        xx = np.maximum(x, -1)
        pos = np.searchsorted(keyv, m * (N + 1) + xx, side="right")
        lo = csr_off[m]
        pos = np.maximum(pos, lo)
        return pos - lo, csum[pos] - csum[lo]

    c1, s1 = CS(qs - w)
    c2, s2 = CS(qe - w)
    total += int((n * c1 + (qe - w + 1) * (c2 - c1) - (s2 - s1)).sum())
    return total


def layer_work(w, sel=None, csr=None):
    """(actual attention pairs, dense-equivalent pairs) summed over heads."""
    N = w.n_tokens
    act = 0
    for h, k in enumerate(w.head_kind):
        if k == 0:
            act += pairs_swa(N, w.window)
        elif k == 3:
            act += pairs_dense(N)
        elif k == 2:
            act += pairs_triangle(N, w.sink, w.window, w.last_q)
        else:
            t = w.ret_heads.index(h)
            if w.n_clusters:
                g = h // (w.n_q_heads // w.n_kv_heads)
                act += pairs_retrieval_clusters(N, w.window, sel[t], csr[0][g], csr[1][g])
            else:
                act += pairs_retrieval_blocks(N, w.window, sel[t], w.force_block0)
    # cross-attention rows p = N - n_out .. N - 1 see keys 0..p
    act += w.n_q_heads * (w.n_out * (N - w.n_out) + w.n_out * (w.n_out + 1) // 2)
    return act, w.n_q_heads * pairs_dense(N)


# ---------------------------------------------------------------------------


class Layer:
    def __init__(self, w, dev_inputs, torch, ha):
        self.w = w
        self.ha = ha
        self.torch = torch
        N, Hq, Hkv, D = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
        self.Q, self.K, self.V, self.P, self.xs, self.xo = dev_inputs
        dev = self.Q.device
        self.desc = ha.make_desc(N, Hq, Hkv, D, window=w.window, topk=w.topk, force_block0=w.force_block0,
                                 n_clusters=w.n_clusters, kmeans_iters=w.kmeans_iters,
                                 kmeans_stride=w.kmeans_stride, sink=w.sink, last_q=w.last_q, n_out=w.n_out,
                                 group_select=w.group_select, block_score=w.block_score,
                                 index_bits=w.index_bits)
        self.kinds = list(w.head_kind)
        self.O = torch.empty((N, Hq, D), dtype=torch.float32, device=dev)
        self.O_out = torch.empty((w.n_out, Hq, D), dtype=torch.float32, device=dev) if w.n_out else None
        nret = len(w.ret_heads)
        self.qlow = torch.empty((nret, N, 16), dtype=torch.float32, device=dev) if nret else None
        self.klow = torch.empty((Hkv, N, 16), dtype=torch.float32, device=dev) if nret else None
        self.sel = torch.empty((nret, w.n_qb, max(1, w.topk)), dtype=torch.int32, device=dev) if nret else None
        nb = ha.ha_workspace_bytes(self.desc, self.kinds)
        self.ws = torch.empty(max(256, nb), dtype=torch.uint8, device=dev)
        self.has_band = any(k != 1 for k in self.kinds)
        if w.n_clusters:
            M = w.n_clusters
            self.cent = torch.empty((Hkv, M, 16), dtype=torch.float32, device=dev)
            self.assign = torch.empty((Hkv, N), dtype=torch.int32, device=dev)
            self.csr_off = torch.empty((Hkv, M + 1), dtype=torch.int32, device=dev)
            self.csr_mem = torch.empty((Hkv, N), dtype=torch.int32, device=dev)

    def stages(self):
        ha, w = self.ha, self.w
        st = []
        if w.ret_heads:
            st.append(("index_project", lambda: ha.ha_index_project(self.desc, self.kinds, self.Q, self.K, self.P,
                                                                     self.qlow, self.klow)))
            if w.n_clusters:
                st.append(("kmeans", lambda: ha.ha_kmeans(self.desc, self.klow, self.cent, self.assign,
                                                          self.csr_off, self.csr_mem, self.ws)))
                st.append(("select_clusters", lambda: ha.ha_select_clusters(
                    self.desc, self.kinds, self.qlow, self.cent, self.csr_off, self.csr_mem, self.sel, self.ws)))
                st.append(("attn_gather", lambda: ha.ha_attn_gather(
                    self.desc, self.kinds, self.Q, self.K, self.V, self.sel, self.csr_off, self.csr_mem,
                    self.O, self.ws)))
            else:
                st.append(("select_blocks", lambda: ha.ha_select_blocks(self.desc, self.kinds, self.qlow,
                                                                         self.klow, self.sel, self.ws)))
                st.append(("attn_gather", lambda: ha.ha_attn_gather(self.desc, self.kinds, self.Q, self.K, self.V,
                                                                     self.sel, None, None, self.O, self.ws)))
        if self.has_band:
            st.append(("attn_band", lambda: ha.ha_attn_band(self.desc, self.kinds, self.Q, self.K, self.V,
                                                             self.O, self.ws)))
        if w.n_out:
            st.append(("attn_cross", lambda: ha.ha_attn_cross(self.desc, self.Q, self.K, self.V, self.xs, self.xo,
                                                               self.O_out, self.ws)))
        return st


def dev_inputs_for(w, cache, torch, log):
    import synth
    key = (w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.recipe, w.n_needles,
           w.window if w.recipe == "needles" else None, w.seed)
    if key in cache:
        base = cache[key]
    else:
        t = time.time()
        li = synth.make_layer_inputs(w.with_(n_out=0))
        dev = torch.device("cuda")

        def bf(b):
            return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
        base = (bf(li.Q), bf(li.K), bf(li.V))
        del li
        cache[key] = base
        log(f"inputs {w.name}: {time.time() - t:.1f}s")
    P = xs = xo = None
    if w.ret_heads:
        P = torch.from_numpy(synth.inputs.gen_proj(w)).cuda()
    if w.n_out:
        s, o = synth.inputs.gen_scale_offset(w)
        xs, xo = torch.from_numpy(s).cuda(), torch.from_numpy(o).cuda()
    return base + (P, xs, xo)


def cpu_baseline(names, log, budget_s=20.0):
    """The fp64 oracle, as it stands, on one query block per layer of the suite
    (the last block of each, so every row sees its full key set); rate =
    oracle attention FLOPs / oracle seconds."""
    import synth
    from synth import inputs as si
    from oracle.prefill import layer_prefill
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    flops = 0.0
    secs = 0.0
    done = []
    for name in names:
        w = synth.WORKLOADS[name]
        if w.n_clusters:
            continue   # k-means over 1M keys does not fit the sampling budget
        K = si.bf16_to_f64(si.gen_k(w))
        V = si.bf16_to_f64(si.gen_v(w))
        P = si.gen_proj(w).astype(np.float64) if w.ret_heads else None
        xs = xo = None
        if w.n_out:
            s, o = si.gen_scale_offset(w)
            xs, xo = s.astype(np.float64), o.astype(np.float64)
        b = w.n_qb - 1
        t = time.time()
        res = layer_prefill(w, lambda a, c: si.bf16_to_f64(si.gen_q(w, a, c)), K, V, P, xs, xo, blocks=[b],
                            out_rows=[w.n_out - 1] if w.n_out else None)
        dt = time.time() - t
        # attention pairs the oracle evaluated for that block (+ the cross row)
        act = 0
        rows = res.rows
        for h, k in enumerate(w.head_kind):
            if k == 0:
                act += int(np.minimum(w.window, rows + 1).sum())
            elif k == 3:
                act += int((rows + 1).sum())
            elif k == 2:
                act += int((rows + 1).sum()) if rows[0] >= w.n_tokens - w.last_q else \
                    int(np.minimum(w.window, rows + 1).sum())
            else:
                act += int(np.minimum(w.window, rows + 1).sum()) + 64 * 64 * len(res.sel[h][b])
        act += w.n_q_heads * w.n_tokens if w.n_out else 0   # the last output row: all N keys
        flops += 4.0 * w.head_dim * act
        secs += dt
        done.append(f"{name}: block {b} all heads" + (", last output row" if w.n_out else ""))
        log(f"cpu oracle {name}: {dt:.1f}s")
        if secs > budget_s:
            break
    return {"value": flops / secs / 1e12 if secs > 0 else None, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "sample": "; ".join(done) + f"; {secs:.1f}s of fp64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workloads", type=str, default=",".join(DEFAULT_SUITE))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain device copy of 1 GiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(each layer's kernels run on one GPU's share; see the sharding notes in the design document).",
              file=sys.stderr)
        sys.exit(2)

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import torch
    import hybrid_attention_prefill_amd as ha
    import synth
    ha.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 1 GiB device-to-device copy done")
    names = [n for n in args.workloads.split(",") if n]
    cache = {}
    layers = []
    for n in names:
        w = synth.WORKLOADS[n]
        layers.append(Layer(w, dev_inputs_for(w, cache, torch, log), torch, ha))
    plan = [(L, name, fn) for L in layers for name, fn in L.stages()]
    stream = torch.cuda.current_stream()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)] for _ in range(args.steps)]

    def step(ev):
        if ev is not None:
            ev[0].record(stream)
        for t, (L, name, fn) in enumerate(plan):
            fn()
            if ev is not None:
                ev[t + 1].record(stream)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    log("warm-up done")
    stage_ms = np.zeros(len(plan))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for ev in events:
        stage_ms += np.array([ev[t].elapsed_time(ev[t + 1]) for t in range(len(plan))])
    ms_step = (t1 - t0) * 1e3 / args.steps
    stage_ms /= args.steps
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step")

    per_layer = {}
    tot_act = tot_dense = 0.0
    for L in layers:
        w = L.w
        sel = L.sel.cpu().numpy() if w.ret_heads else None
        csr = (L.csr_off.cpu().numpy(), L.csr_mem.cpu().numpy()) if w.n_clusters else None
        act, dense = layer_work(w, sel, csr)
        ms = float(sum(stage_ms[t] for t, (LL, _, _) in enumerate(plan) if LL is L))
        stg = {name: round(float(stage_ms[t]), 4) for t, (LL, name, _) in enumerate(plan) if LL is L}
        fl_act = None if act is None else 4.0 * w.head_dim * act
        fl_dense = 4.0 * w.head_dim * dense
        per_layer[w.name] = {
            "ms": round(ms, 4), "stages_ms": stg,
            "actual_tflops": None if fl_act is None else round(fl_act / ms / 1e9, 2),
            "dense_equiv_tflops": round(fl_dense / ms / 1e9, 2),
            "mfma_frac_actual": None if fl_act is None else round(fl_act / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "attn_pairs": act,
        }
        if fl_act is not None:
            tot_act += fl_act
        tot_dense += fl_dense

    # dominant kernel: the longest single-kernel stage
    best = max(range(len(plan)), key=lambda t: stage_ms[t])
    L, sname, _ = plan[best]
    w = L.w
    roof = None
    if sname in ("attn_band", "attn_gather"):
        if sname == "attn_band":
            act = sum(pairs_swa(w.n_tokens, w.window) if k == 0 else pairs_dense(w.n_tokens) if k == 3 else
                      pairs_triangle(w.n_tokens, w.sink, w.window, w.last_q) if k == 2 else 0
                      for k in w.head_kind)
        else:
            act = per_layer[w.name]["attn_pairs"] - sum(
                pairs_swa(w.n_tokens, w.window) for k in w.head_kind if k == 0)
        achieved = 4.0 * w.head_dim * act / (stage_ms[best] * 1e-3) / 1e12
        tr = traffic_for(w.name, sname)
        roof = {"kernel": f"{sname} ({w.name})", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": tr, "avg_ms": round(float(stage_ms[best]), 4),
                "work": "4*D FLOPs per (query, key) pair of the realised key sets"}

    value = tot_act / (ms_step * 1e-3) / 1e12 if tot_act else None
    out = {
        "metric": METRIC, "value": None if value is None else round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs shaped like the pages' workloads; random-init indexer)",
        "config": {"workload": "suite:" + "+".join(names), "layers_per_step": len(layers),
                   "value_is": "actual attention FLOPs of all layers / wall time of the step"},
        "layers": per_layer,
        "dense_equiv_tflops": round(tot_dense / (ms_step * 1e-3) / 1e12, 2),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(names, log)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
