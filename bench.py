#!/usr/bin/env python3
"""Benchmark of the LSA indexer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads decode_1m,prefill_1m,decode_10m,prefill_10m]

A step is one ``lsa_select`` call over a workload's batch of query heads
(query projection, centroid descent, gather-and-score, top-k, assembly), with
the key cache and its index already resident in HBM.  The first workload is
the headline (``value``, ``roofline``); the others are reported in full under
``workloads``.  Each key cache (1M, 10M) is generated, uploaded and indexed
once for the workloads that share it.

Decode steps rotate over a pool of seeded query batches (``--pool``, batch 0
is the workload's own), so consecutive steps select different leaves and the
rows one pass of the pool reads exceed the 256 MB Infinity Cache: ``value``,
the stage times and ``roofline`` are these cold figures.  The same figures
for batch 0 repeated (its rows stay on chip) are reported under ``warm``.

``value`` comes from the wall time of K steps with nothing else in the
stream; the per-stage kernel times come from a second run with HIP events
that the library records around every stage on its own launch stream.  The
index build and the full-scan baseline (``lsa_flat_select``) are timed in the
same run, together with tree-vs-flat recall.

``roofline`` describes the dominant kernel of the step:
  * decode (per-query-head path): the gather-and-score kernel against HBM,
    algorithmic bytes per launch = keys scored x bytes per key row;
  * prefill (node-major path): the main pass of the leaf-major gather
    against the bf16 matrix-core peak, algorithmic flops per launch = keys
    scored x 2 x latent dim; the centroid descent is reported the same way
    under ``centroid_scoring``.
``cpu_baseline`` times the CPU oracle on a bounded sample of the headline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer query-heads/s and keys-scored/s at 1M/10M keys; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3                 # fp32 vector FMA: 256 CUs x 128 FMA/clk x 2 x 2.4 GHz
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "hierarchical_key_indexer_amd", "csrc", f)
                  for f in ("select.hip", "select_device.h", "prefill.hip", "lsa_device.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them on
    the stream it launches on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        """Milliseconds between two recorded events, None if they were never
        recorded (a stage the call did not run; the failed query's error is
        cleared so that it does not surface in the next HIP call)."""
        ms = ctypes.c_float()
        if self.hip.hipEventSynchronize(b) != 0 or self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            self.hip.hipGetLastError()
            return None
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_steps(fn, steps, hip, stages, abi):
    """Run fn() `steps` times; return (wall ms per step, {stage: ms per step,
    None for a stage the call does not run})."""
    import torch
    ev = {st: (hip.create(steps), hip.create(steps)) for st in stages}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for st in stages:
            abi.set_profile_events(st, ev[st][0][i], ev[st][1][i])
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    out = {}
    for st in stages:
        abi.set_profile_events(st, None, None)
        ms = [hip.elapsed_ms(a, b) for a, b in zip(*ev[st])]
        out[st] = None if any(m is None for m in ms) else sum(ms) / steps
        hip.destroy(ev[st][0] + ev[st][1])
    return wall, out


def graph_replay(step, steps, qheads):
    """The same step captured once in a graph and replayed `steps` times (the
    library only enqueues kernels, so a call is capturable)."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        return {"ms_per_step": ms, "query_heads_per_s": qheads / (ms * 1e-3)}
    except Exception as e:  # reported, never fatal to the bench line
        return {"error": f"{type(e).__name__}: {e}"}


def cpu_baseline(wl, keys, W, queries, pos):
    """The CPU oracle, untuned, on KV head 0 of the workload: its index build
    (reported, not in the value) and the selection of that head's G query
    heads for every token (sampled to at most 64 query heads), repeated
    until about ten seconds of selection have been timed."""
    import numpy as np
    from oracle import lsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    desc = O.IndexDesc.of(wl)
    t = time.perf_counter()
    oidx = O.build_index(keys, W, desc, heads=[0])
    build_s = time.perf_counter() - t
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    pairs = [(tt, hq) for tt in range(wl.n_tokens) for hq in range(wl.group)]
    if len(pairs) > 64:
        rng = np.random.default_rng(0)
        pairs = [pairs[i] for i in sorted(rng.choice(len(pairs), 64, replace=False))]
    # the same selection is repeated until it has run for about ten seconds
    reps, sel_s = 0, 0.0
    while sel_s < 10.0:
        t = time.perf_counter()
        O.select(oidx, queries, pos, prm, pairs=pairs)
        sel_s += time.perf_counter() - t
        reps += 1
    return {
        "value": reps * len(pairs) / sel_s, "unit": "query-heads/s", "cores": blas_threads, "kind": "oracle",
        "sample": (f"KV head 0 of {wl.name} (N={wl.n_keys}): oracle select of {len(pairs)} query heads, "
                   f"{reps} times in {sel_s:.1f} s, on the oracle's own index of that head (index build "
                   f"{build_s:.1f} s, not in the value); float64 numpy, BLAS threads={blas_threads}, "
                   f"host cpus={os.cpu_count()}"),
        "build_s_one_head": build_s,
    }


def pca_leg(abi, desc, kd, reps=3):
    """The training-free latent map of the workload's keys: the device
    covariance (two kernels, timed with events on the stream they run on) and
    the host eigenvectors."""
    import numpy as np
    import torch
    d, hk = desc.d_head, desc.n_kv_heads
    cov = torch.empty((hk, d, d), dtype=torch.float64, device="cuda")
    ws = torch.empty(abi.pca_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    abi.lsa_pca_covariance(desc, kd, cov, ws)      # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        abi.lsa_pca_covariance(desc, kd, cov, ws)
    e1.record()
    torch.cuda.synchronize()
    cov_ms = e0.elapsed_time(e1) / reps
    c = cov.cpu().numpy()
    t = time.perf_counter()
    W, lam = abi.lsa_pca_map(desc, c)
    eig_ms = (time.perf_counter() - t) * 1e3
    flops = 2.0 * desc.n_keys * hk * d * d          # every product of the d x d sums
    return {"covariance_ms": cov_ms, "eigensolve_ms": eig_ms, "kernels": "pca_gram_kernel + pca_reduce_kernel",
            "bound": "alu", "algorithmic_flops": flops, "achieved_TFLOPs": flops / (cov_ms * 1e-3) / 1e12,
            "peak_TFLOPs": FP32_PEAK_TFLOPS, "frac": flops / (cov_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
            "variance_kept": float(lam.sum() / np.trace(c, axis1=1, axis2=2).sum())}


def attention_leg(abi, desc, wl, qd, kd, idx, reps=20):
    """Exact sparse attention over the rows a select call returned (the step
    after the indexer): seeded bf16 values made on the device, keys and
    queries of the workload, scale 1/sqrt(d); timed with events on the stream
    it runs on.  Bytes: one key row and one value row per listed key."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(20261030)
    vals = torch.randn(tuple(kd.shape), generator=g, device="cuda",
                       dtype=torch.bfloat16 if wl.key_dtype == "bf16" else torch.float32)
    T, Hq, width = idx.shape
    out = torch.empty((T, Hq, desc.d_head), dtype=torch.float32, device="cuda")
    scale = 1.0 / float(desc.d_head) ** 0.5
    ws = torch.empty(max(abi.sparse_attention_workspace_bytes(desc, width, T, Hq), 1), dtype=torch.uint8,
                     device="cuda")
    abi.lsa_sparse_attention(desc, qd, kd, vals, idx, scale, out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        abi.lsa_sparse_attention(desc, qd, kd, vals, idx, scale, out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    valid = (idx >= 0) & (idx < desc.n_keys)
    listed = int(valid.sum().item())
    elt = 2 if wl.key_dtype == "bf16" else 4
    row_bytes = listed * 2 * desc.d_head * elt + idx.numel() * 4
    # rows of one KV head share keys (GQA, neighbouring tokens): the distinct
    # (KV head, key) pairs are what HBM has to deliver at least
    kvh = (torch.arange(Hq, device=idx.device) // (Hq // desc.n_kv_heads)).view(1, Hq, 1).long()
    uniq = int(torch.unique((kvh * desc.n_keys + idx.long())[valid]).numel())
    unique_bytes = uniq * 2 * desc.d_head * elt + idx.numel() * 4
    del vals
    return {"ms_per_call": ms, "rows": T * Hq, "keys_per_row": listed / (T * Hq), "kernel": "sparse_attention_kernel",
            "bound": "hbm", "distinct_kv_rows": uniq, "bytes": unique_bytes,
            "achieved_GBs": unique_bytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": unique_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "per_row_bytes": row_bytes,
            "note": "bytes: each distinct (KV head, key) K and V row once plus the index rows; per_row_bytes "
                    "counts every row's own reads, which rows sharing keys serve from the caches"}


def recall_rows(tree_out, flat_out, sink, k):
    """Per query head |tree top-k & flat top-k| / |flat top-k|, computed on
    the device from the two output tensors [T, Hq, width]."""
    import numpy as np
    import torch
    a = tree_out[:, :, sink:sink + k].reshape(-1, k).long()
    b = flat_out[:, :, sink:sink + k].reshape(-1, k).long()
    bs, _ = torch.sort(b, dim=1)
    pos = torch.searchsorted(bs, a).clamp(max=k - 1)
    hit = (torch.gather(bs, 1, pos) == a) & (a >= 0)
    nb = (b >= 0).sum(1).clamp(min=1)
    return np.asarray((hit.sum(1).double() / nb.double()).cpu())


def keys_scored_of(li, leaves_t, wl):
    """Keys scored by a select call: the members of every selected leaf."""
    import numpy as np
    counts = li.leaf_counts()                                  # [Hkv, P_L]
    lv = leaves_t.cpu().numpy().reshape(wl.n_tokens * wl.n_q_heads, -1)
    heads = np.tile(np.arange(wl.n_q_heads) // wl.group, wl.n_tokens)
    hh = np.broadcast_to(heads[:, None], lv.shape)
    ok = lv >= 0
    return int(counts[hh[ok], lv[ok]].sum())


def centroid_dots(wl):
    """Centroid dot products per query head: F_1 + b F_2 + b^2 F_3 + ..."""
    dots, kept = 0, 1
    for f in wl.fanout:
        dots += kept * f
        kept *= min(wl.b, f)
    return dots


def decode_record(wl, li, keys, hip, args, pool_n, abi):
    """A decode workload (per-query-head path).  Steps rotate over a pool of
    seeded query batches (batch 0 is the workload's own), so consecutive steps
    select different leaves and the rows one pass of the pool reads exceed the
    256 MB Infinity Cache: the cold figures.  The warm figures repeat batch 0
    (its rows stay on chip between steps)."""
    import numpy as np
    import torch
    from hierarchical_key_indexer_amd.indexer import keys_to_device
    from synth import gen_positions, gen_queries
    T, Hq = wl.n_tokens, wl.n_q_heads
    prm = abi.SelectParams.make(wl.b, wl.k, wl.sink, wl.window)
    row_bytes = wl.d_latent * (2 if wl.latent_dtype == "bf16" else 4) + 4
    pd = torch.from_numpy(gen_positions(wl)).cuda()
    pool = []
    for i in range(pool_n):
        wq = wl if i == 0 else wl.scaled(query_id=1000 + 100 * wl.query_id + i)
        qd = keys_to_device(gen_queries(wq, keys))
        out = li.alloc_select_outputs(T, Hq, prm, scores=True, leaves=True)
        li.select(qd, pd, prm, leaves=True, out=out)
        pool.append((qd, out, keys_scored_of(li, out[2], wl)))
    torch.cuda.synchronize()
    ks = [b[2] for b in pool]
    outs = li.alloc_select_outputs(T, Hq, prm, scores=True)
    state = {"i": 0}

    def cold_step():
        qd = pool[state["i"] % pool_n][0]
        state["i"] += 1
        li.select(qd, pd, prm, leaves=False, out=(outs[0], outs[1], None))

    def warm_step():
        li.select(pool[0][0], pd, prm, leaves=False, out=(outs[0], outs[1], None))

    def keys_of(i0, n):
        return sum(ks[(i0 + j) % pool_n] for j in range(n)) / n

    for _ in range(args.warmup):
        cold_step()
    torch.cuda.synchronize()
    i0 = state["i"]
    t0 = time.perf_counter()
    for _ in range(args.steps):
        cold_step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    keys_step = keys_of(i0, args.steps)
    stages = [abi.STAGE_DESCEND, abi.STAGE_GATHER, abi.STAGE_MERGE]
    n_ev = max(1, min(args.steps, 20))
    i0 = state["i"]
    _, cold = timed_steps(cold_step, n_ev, hip, stages, abi)
    cold_bytes = keys_of(i0, n_ev) * row_bytes
    for _ in range(3):
        warm_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        warm_step()
    torch.cuda.synchronize()
    warm_ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    _, warm = timed_steps(warm_step, n_ev, hip, stages, abi)
    warm_bytes = ks[0] * row_bytes
    gather_ms = cold[abi.STAGE_GATHER]
    roof = {"bound": "hbm", "achieved": cold_bytes / (gather_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # decode plans split the descent over the kept level-1 nodes when the
    # per-parent beam keeps at most 16 of them and no fanout exceeds 64
    split = wl.b <= 16 and max(wl.fanout) <= 64
    roof["traffic"] = load_traffic(wl.name, "gather_split" if split else "gather")
    roof["kernel"] = "gather_split_kernel" if split else "gather_kernel"
    roof["algorithmic_bytes_per_launch"] = cold_bytes
    roof["kernel_ms"] = gather_ms
    roof["timing"] = (f"cold: steps rotate over {pool_n} query batches whose rows total "
                      f"{sum(ks) * row_bytes / 1e6:.0f} MB, so a step's rows are not left on chip by the last one")
    rec = {
        "value": T * Hq / (ms_step * 1e-3), "unit": "query-heads/s", "ms_per_step": ms_step,
        "keys_scored_per_s": keys_step / (ms_step * 1e-3), "keys_scored_per_step": keys_step,
        "roofline": roof, "select_path": "per-query-head",
        "stages_ms": {n: cold.get(st) for n, st in (("descend", abi.STAGE_DESCEND), ("gather", abi.STAGE_GATHER),
                                                    ("merge", abi.STAGE_MERGE))},
        "query_pool": {"batches": pool_n, "rows_bytes_per_pass": sum(ks) * row_bytes,
                       "keys_scored_per_batch": ks},
        "warm": {"ms_per_step": warm_ms_step, "value": T * Hq / (warm_ms_step * 1e-3),
                 "gather_ms": warm[abi.STAGE_GATHER],
                 "gather_GBs_l2_miss": warm_bytes / (warm[abi.STAGE_GATHER] * 1e-3) / 1e9,
                 "stages_ms": {n: warm.get(st) for n, st in (("descend", abi.STAGE_DESCEND),
                               ("gather", abi.STAGE_GATHER), ("merge", abi.STAGE_MERGE))},
                 "note": "batch 0 repeated: its rows stay in the Infinity Cache, so this is L2-miss bandwidth, "
                         "not HBM"},
        "graph_replay": graph_replay(warm_step, args.steps, T * Hq),
    }
    if not args.no_flat:
        fout = li.alloc_select_outputs(T, Hq, prm, scores=True, flat=True)
        for _ in range(3):
            li.flat_select(pool[0][0], pd, prm, out=fout)
        fsteps = args.flat_steps or max(5, min(args.steps, 20))
        fstate = {"i": 0}

        def fstep():
            li.flat_select(pool[fstate["i"] % pool_n][0], pd, prm, out=fout)
            fstate["i"] += 1

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(fsteps):
            fstep()
        torch.cuda.synchronize()
        flat_ms = (time.perf_counter() - t0) * 1e3 / fsteps
        _, fst = timed_steps(fstep, max(1, min(fsteps, 10)), hip, [abi.STAGE_FLAT], abi)
        flat_kernel_ms = fst[abi.STAGE_FLAT]
        rec_all = []
        for qd, out, _ in pool:
            li.flat_select(qd, pd, prm, out=fout)
            rec_all.append(recall_rows(out[0], fout[0], wl.sink, wl.k))
        rec_all = np.concatenate(rec_all)
        flat_bytes = T * wl.n_kv_heads * wl.n_keys * row_bytes
        rec["flat"] = {
            "ms_per_call": flat_ms, "query_heads_per_s": T * Hq / (flat_ms * 1e-3),
            "keys_scored_per_s": T * Hq * wl.n_keys / (flat_ms * 1e-3),
            "kernel": "flat_kernel", "kernel_ms": flat_kernel_ms,
            "achieved_GBs": flat_bytes / (flat_kernel_ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": flat_bytes / (flat_kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": load_traffic(wl.name, "flat"),
        }
        rec["recall_at_k_vs_flat"] = {"mean": float(rec_all.mean()), "p5": float(np.percentile(rec_all, 5)),
                                      "rows": int(rec_all.size)}
        rec["speedup_vs_flat"] = flat_ms / ms_step
    if not args.no_upkeep:
        rec["upkeep"] = upkeep_leg(wl, li, [b[0] for b in pool], hip, args, abi, ms_step)
    rec["_rows"] = pool[0][1][0]
    rec["_queries"] = pool[0][0]
    return rec


def upkeep_leg(wl, li, qpool, hip, args, abi, base_ms, n_app=4096):
    """Incremental upkeep: n_app keys that arrive after the cache appended to
    the index (one call of n_app tokens, and single-token calls as a decode
    loop makes them), then decode steps over the index plus the appended keys
    at the last position, rotating over the same query batches."""
    import numpy as np
    import torch
    from hierarchical_key_indexer_amd.indexer import keys_to_device
    from synth import gen_keys_range
    N, T, Hq = wl.n_keys, wl.n_tokens, wl.n_q_heads
    later = keys_to_device(gen_keys_range(wl, N, N + n_app))
    buf = torch.empty(abi.append_pool_bytes(li.desc, n_app), dtype=torch.uint8, device="cuda")
    abi.lsa_append_keys(li.desc, li.index, later, 0, buf, n_app)          # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        abi.lsa_append_keys(li.desc, li.index, later, 0, buf, n_app)
    e1.record()
    torch.cuda.synchronize()
    batch_ms = e0.elapsed_time(e1) / reps
    ones = 200
    e0.record()
    for i in range(ones):
        abi.lsa_append_keys(li.desc, li.index, later[i:i + 1], i, buf, n_app)
    e1.record()
    torch.cuda.synchronize()
    one_ms = e0.elapsed_time(e1) / ones
    prm = abi.SelectParams.make(wl.b, wl.k, wl.sink, wl.window)
    ws = torch.empty(abi.select_appended_workspace_bytes(li.desc, prm, T, Hq), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, Hq, wl.sink + wl.k + wl.window), dtype=torch.int32, device="cuda")
    sc = torch.empty((T, Hq, wl.k), dtype=torch.float32, device="cuda")
    pd = torch.full((T,), N + n_app - 1, dtype=torch.int32, device="cuda")
    state = {"i": 0}

    def step():
        q = qpool[state["i"] % len(qpool)]
        state["i"] += 1
        abi.lsa_select_appended(li.desc, li.index, buf, n_app, n_app, q, pd, prm, idx, sc, None, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    assert abi.device_status(ws) == abi.LSA_OK
    del later, buf, ws
    return {
        "appended_keys": n_app, "append_batch_ms": batch_ms,
        "appended_key_heads_per_s": n_app * wl.n_kv_heads / (batch_ms * 1e-3),
        "append_one_token_us": one_ms * 1e3,
        "select_with_appended_ms_per_step": ms, "select_without_ms_per_step": base_ms,
        "query_heads_per_s": T * Hq / (ms * 1e-3),
        "note": "keys of the positions after the cache, one latent projection and one root-to-leaf routing per "
                "(key, KV head); select runs on the index plus every appended key, at position N + 4095",
    }


def prefill_record(wl, li, keys, hip, args, abi):
    """A prefill chunk (node-major path): one batch of T tokens x Hq heads."""
    import numpy as np
    import torch
    from hierarchical_key_indexer_amd.indexer import keys_to_device
    from synth import gen_positions, gen_queries
    T, Hq = wl.n_tokens, wl.n_q_heads
    prm = abi.SelectParams.make(wl.b, wl.k, wl.sink, wl.window)
    qd = keys_to_device(gen_queries(wl, keys))
    pd = torch.from_numpy(gen_positions(wl)).cuda()
    out = li.alloc_select_outputs(T, Hq, prm, scores=True, leaves=True)
    li.select(qd, pd, prm, leaves=True, out=out)
    torch.cuda.synchronize()
    keys_scored = keys_scored_of(li, out[2], wl)
    node_major = abi.select_path(li.desc, prm, T, Hq) == abi.PATH_NODE_MAJOR
    step = lambda: li.select(qd, pd, prm, leaves=False, out=(out[0], out[1], None))  # noqa: E731
    steps = args.prefill_steps
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    stages = [abi.STAGE_DESCEND, abi.STAGE_SAMPLE, abi.STAGE_GATHER, abi.STAGE_MERGE]
    _, st = timed_steps(step, steps, hip, stages, abi)
    gather_ms = st[abi.STAGE_GATHER]
    flops = keys_scored * 2 * wl.d_latent
    roof = {"bound": "mfma", "achieved": flops / (gather_ms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(wl.name, "pf_gather")
    roof["kernel"] = "pf_gather (main pass)"
    roof["algorithmic_flops_per_launch"] = flops
    roof["kernel_ms"] = gather_ms
    cflops = T * Hq * centroid_dots(wl) * 2 * wl.d_latent
    dms = st[abi.STAGE_DESCEND]
    rec = {
        "value": T * Hq / (ms_step * 1e-3), "unit": "query-heads/s", "ms_per_step": ms_step,
        "keys_scored_per_s": keys_scored / (ms_step * 1e-3), "keys_scored_per_step": keys_scored,
        "roofline": roof, "select_path": "node-major" if node_major else "per-query-head",
        "stages_ms": {n: st.get(s_) for n, s_ in (("descend", abi.STAGE_DESCEND), ("sample", abi.STAGE_SAMPLE),
                                                  ("gather", abi.STAGE_GATHER), ("merge", abi.STAGE_MERGE))},
        "centroid_scoring": {"flops_per_call": cflops, "ms": dms, "achieved_TFLOPs": cflops / (dms * 1e-3) / 1e12,
                             "frac_of_mfma_peak": cflops / (dms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                             "includes": "query projection, per-level MFMA scoring with exact top-b, child lists"},
    }
    if not args.no_flat:
        fout = li.alloc_select_outputs(T, Hq, prm, scores=True, flat=True)
        li.flat_select(qd, pd, prm, out=fout)
        fstep = lambda: li.flat_select(qd, pd, prm, out=fout)  # noqa: E731
        fsteps = 2
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(fsteps):
            fstep()
        torch.cuda.synchronize()
        flat_ms = (time.perf_counter() - t0) * 1e3 / fsteps
        fstages = [abi.STAGE_PROJECT, abi.STAGE_SAMPLE, abi.STAGE_FLAT, abi.STAGE_MERGE]
        _, fst = timed_steps(fstep, fsteps, hip, fstages, abi)
        scan_ms = fst[abi.STAGE_FLAT]
        fflops = T * Hq * wl.n_keys * 2 * wl.d_latent
        rc = recall_rows(out[0], fout[0], wl.sink, wl.k)
        rec["flat"] = {
            "ms_per_call": flat_ms, "query_heads_per_s": T * Hq / (flat_ms * 1e-3),
            "keys_scored_per_s": T * Hq * wl.n_keys / (flat_ms * 1e-3),
            "path": "row-tiled (matrix cores)", "kernel": "fs_scan_kernel", "kernel_ms": scan_ms,
            "algorithmic_flops_per_launch": fflops,
            "achieved_TFLOPs": fflops / (scan_ms * 1e-3) / 1e12,
            "frac_of_mfma_peak": fflops / (scan_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "stages_ms": {n: fst.get(s_) for n, s_ in (("project", abi.STAGE_PROJECT), ("sample", abi.STAGE_SAMPLE),
                                                       ("scan", abi.STAGE_FLAT), ("merge", abi.STAGE_MERGE))},
            "traffic": load_traffic(wl.name, "fs_scan"),
        }
        rec["recall_at_k_vs_flat"] = {"mean": float(rc.mean()), "p5": float(np.percentile(rc, 5)),
                                      "rows": int(rc.size)}
        rec["speedup_vs_flat"] = flat_ms / ms_step
        del fout
    rec["_rows"] = out[0]
    rec["_queries"] = qd
    return rec


def config_of(wl):
    return {"workload": wl.name, "n_keys": wl.n_keys, "kv_heads": wl.n_kv_heads, "q_heads": wl.n_q_heads,
            "tokens": wl.n_tokens, "d_head": wl.d_head, "d_latent": wl.d_latent, "fanout": list(wl.fanout),
            "b": wl.b, "k": wl.k, "sink": wl.sink, "window": wl.window}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="decode_1m,prefill_1m,decode_10m,prefill_10m",
                    help="comma list; the first is the headline (value, roofline), the others are reported "
                         "under 'workloads'")
    ap.add_argument("--pool", type=int, default=16, help="query batches the decode steps rotate over")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--flat-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat", action="store_true")
    ap.add_argument("--no-pca", action="store_true", help="skip the training-free latent map leg")
    ap.add_argument("--no-attention", action="store_true", help="skip the sparse attention leg")
    ap.add_argument("--no-upkeep", action="store_true", help="skip the incremental-upkeep leg (decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the indexer shards by KV head "
              f"with no exchange, and this benchmark runs on one GPU.", flush=True)
        sys.exit(2)

    import torch

    from hierarchical_key_indexer_amd import _abi
    from hierarchical_key_indexer_amd.indexer import LatentIndex, keys_to_device
    from synth import gen_keys, gen_W, get_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _abi.load()
    hip = HipEvents()
    names = [n for n in args.workloads.split(",") if n]
    wls = [get_workload(n) for n in names]
    headline = wls[0]
    records = {}
    # one key cache at a time: its workloads share the cache and its index
    caches = []
    for wl in wls:
        if wl.cache_id not in caches:
            caches.append(wl.cache_id)
    extra = {}
    for cid in caches:
        group = [wl for wl in wls if wl.cache_id == cid]
        base = group[0]
        log(f"cache {cid} ({base.n_keys} keys x {base.n_kv_heads} KV heads): generating inputs")
        t = time.perf_counter()
        keys, W = gen_keys(base), gen_W(base)
        log(f"inputs ready in {time.perf_counter() - t:.1f} s")
        kd, Wd = keys_to_device(keys), torch.from_numpy(W).cuda()
        desc = _abi.IndexDesc.of(base)
        li = LatentIndex(desc)
        li.build(kd, Wd)                             # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        li.build(kd, Wd)
        e1.record()
        torch.cuda.synchronize()
        build_ms = e0.elapsed_time(e1)
        li.release_build_workspace()
        log(f"index build {build_ms:.1f} ms")
        for wl in group:
            log(f"{wl.name}: timing select ({wl.n_tokens} tokens x {wl.n_q_heads} query heads)")
            if wl.n_tokens == 1:
                rec = decode_record(wl, li, keys, hip, args, args.pool, _abi)
            else:
                rec = prefill_record(wl, li, keys, hip, args, _abi)
            rec["config"] = config_of(wl)
            rec["build_ms"] = build_ms
            rec["index_bytes"] = int(li.index.numel())
            if wl is headline:
                if not args.no_pca:
                    rec["pca_map"] = pca_leg(_abi, desc, kd)
                    log(f"training-free latent map: covariance {rec['pca_map']['covariance_ms']:.2f} ms")
                if not args.no_attention:
                    log("exact sparse attention over the selected rows")
                    rec["sparse_attention"] = attention_leg(_abi, desc, wl, rec["_queries"], kd, rec["_rows"],
                                                            reps=20 if wl.n_tokens == 1 else 2)
                if not args.no_cpu_baseline:
                    log("timing the CPU oracle on a bounded sample")
                    from synth import gen_positions, gen_queries
                    extra["cpu_baseline"] = cpu_baseline(wl, keys, W, gen_queries(wl, keys), gen_positions(wl))
            rec.pop("_rows")
            rec.pop("_queries")
            records[wl.name] = rec
            torch.cuda.empty_cache()
        del li, kd, Wd, keys
        torch.cuda.empty_cache()

    h = records[headline.name]
    result = {
        "metric": METRIC, "value": h["value"], "unit": "query-heads/s", "n_gpus": 1,
        "steps": args.steps if headline.n_tokens == 1 else args.prefill_steps, "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if headline.latent_dtype == "bf16" else "f32",
        "data": "synthetic (seeded; keys around Gaussian centers, queries = noisy cached keys)",
        "config": h.pop("config"),
    }
    for k_, v_ in h.items():
        if k_ not in ("value", "unit", "ms_per_step"):
            result[k_] = v_
    result["workloads"] = {n: r for n, r in records.items() if n != headline.name}
    result.update(extra)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
