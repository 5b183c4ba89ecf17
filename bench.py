#!/usr/bin/env python3
"""Benchmark of the LSA indexer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_1m]

A step is one ``lsa_select`` call over the workload's batch of query heads
(query projection, centroid descent, gather-and-score, top-k, assembly), with
the key cache and its index already resident in HBM.  ``value`` comes from the
wall time of K steps with nothing else in the stream; the per-stage kernel
times come from a second, shorter run with HIP events around every stage.  The index build and the
full-scan baseline (``lsa_flat_select``) are timed in the same run and
reported beside it, together with tree-vs-flat recall.

Prints one JSON line.  ``roofline`` describes the dominant kernel of the step,
timed with HIP events that the library records on its own launch stream:
  * per-query-head path (decode): the gather-and-score kernel against HBM,
    algorithmic bytes per launch = keys scored x bytes per key row;
  * node-major path (prefill batches): the main pass of the leaf-major gather
    against the bf16 matrix-core peak, algorithmic flops per launch = keys
    scored x 2 x latent dim (one dot product per scored key); the centroid
    descent is reported the same way under ``centroid_scoring``.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload.
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
        recorded (a stage the call did not run)."""
        if self.hip.hipEventSynchronize(b) != 0:
            return None
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
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
    listed = int(((idx >= 0) & (idx < desc.n_keys)).sum().item())
    nbytes = listed * 2 * desc.d_head * (2 if wl.key_dtype == "bf16" else 4) + idx.numel() * 4
    del vals
    return {"ms_per_call": ms, "rows": T * Hq, "keys_per_row": listed / (T * Hq), "kernel": "sparse_attention_kernel",
            "bound": "hbm", "bytes": nbytes, "achieved_GBs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_1m")
    ap.add_argument("--flat-steps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat", action="store_true")
    ap.add_argument("--no-pca", action="store_true", help="skip the training-free latent map leg")
    ap.add_argument("--no-attention", action="store_true", help="skip the sparse attention leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the indexer shards by KV head "
              f"with no exchange, and multi-GPU runs are not part of this build.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from hierarchical_key_indexer_amd import _abi
    from hierarchical_key_indexer_amd.indexer import LatentIndex, keys_to_device
    from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _abi.load()
    hip = HipEvents()
    wl = get_workload(args.workload)
    log(f"workload {wl.name}: generating inputs")
    t = time.perf_counter()
    keys, W = gen_keys(wl), gen_W(wl)
    queries, pos = gen_queries(wl, keys), gen_positions(wl)
    log(f"inputs ready in {time.perf_counter() - t:.1f} s")
    kd, Wd = keys_to_device(keys), torch.from_numpy(W).cuda()
    qd, pd = keys_to_device(queries), torch.from_numpy(pos).cuda()
    desc = _abi.IndexDesc.of(wl)
    li = LatentIndex(desc)
    # index build (not part of the step): first call warms up, then timed
    li.build(kd, Wd)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    li.build(kd, Wd)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    li.release_build_workspace()
    log(f"index build {build_ms:.1f} ms")
    pca = None
    if not args.no_pca:
        pca = pca_leg(_abi, desc, kd)
        log(f"training-free latent map: covariance {pca['covariance_ms']:.2f} ms, "
            f"eigenvectors {pca['eigensolve_ms']:.0f} ms on the host")

    prm = _abi.SelectParams.make(wl.b, wl.k, wl.sink, wl.window)
    out = li.alloc_select_outputs(wl.n_tokens, wl.n_q_heads, prm, scores=True, leaves=True)
    li.select(qd, pd, prm, leaves=True, out=out)
    torch.cuda.synchronize()
    # keys scored per call: members of every selected leaf
    counts = li.leaf_counts()
    leaves = out[2].cpu().numpy()
    heads_of = np.arange(wl.n_q_heads) // wl.group
    keys_scored = int(sum(counts[heads_of[hq]][leaves[t_, hq][leaves[t_, hq] >= 0]].sum()
                          for t_ in range(wl.n_tokens) for hq in range(wl.n_q_heads)))
    row_bytes = wl.d_latent * (2 if wl.latent_dtype == "bf16" else 4) + 4

    for _ in range(args.warmup):
        li.select(qd, pd, prm, leaves=False, out=(out[0], out[1], None))
    torch.cuda.synchronize()
    node_major = _abi.select_path(desc, prm, wl.n_tokens, wl.n_q_heads) == _abi.PATH_NODE_MAJOR
    log(f"timing {args.steps} select steps ({'node-major' if node_major else 'per-query-head'} path)")
    step = lambda: li.select(qd, pd, prm, leaves=False, out=(out[0], out[1], None))  # noqa: E731
    # the value: wall time of K steps with no events in the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-stage kernel time (events around each stage) in a second, shorter run
    stages = [_abi.STAGE_DESCEND, _abi.STAGE_GATHER, _abi.STAGE_MERGE] + ([_abi.STAGE_SAMPLE] if node_major else [])
    _, stage_ms = timed_steps(step, max(1, min(args.steps, 20)), hip, stages, _abi)
    graph = graph_replay(step, args.steps, wl.n_tokens * wl.n_q_heads)
    gather_ms = stage_ms[_abi.STAGE_GATHER]
    qheads = wl.n_tokens * wl.n_q_heads
    tree_idx = out[0].cpu().numpy()

    if node_major:
        flops = keys_scored * 2 * wl.d_latent
        roof = {"bound": "mfma", "achieved": flops / (gather_ms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = load_traffic(wl.name, "pf_gather")
        roof["kernel"] = "pf_gather (main pass)"
        roof["algorithmic_flops_per_launch"] = flops
        roof["kernel_ms"] = gather_ms
        # centroid dots per query head: F_1 + b F_2 + b^2 F_3 + ...
        dots, kept = 0, 1
        for f in wl.fanout:
            dots += kept * f
            kept *= min(wl.b, f)
        cflops = qheads * dots * 2 * wl.d_latent
        dms = stage_ms[_abi.STAGE_DESCEND]
        centroid = {"flops_per_call": cflops, "ms": dms, "achieved_TFLOPs": cflops / (dms * 1e-3) / 1e12,
                    "frac_of_mfma_peak": cflops / (dms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "includes": "query projection, per-level MFMA scoring with exact top-b, child lists"}
    else:
        gather_bytes = keys_scored * row_bytes
        roof = {"bound": "hbm", "achieved": gather_bytes / (gather_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = load_traffic(wl.name, "gather")
        roof["kernel"] = "gather_kernel"
        roof["algorithmic_bytes_per_launch"] = gather_bytes
        roof["kernel_ms"] = gather_ms
        centroid = None

    result = {
        "metric": METRIC, "value": qheads / (ms_step * 1e-3), "unit": "query-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.latent_dtype == "bf16" else "f32",
        "data": "synthetic (seeded; keys around Gaussian centers, queries = noisy cached keys)",
        "config": {"workload": wl.name, "n_keys": wl.n_keys, "kv_heads": wl.n_kv_heads, "q_heads": wl.n_q_heads,
                   "tokens": wl.n_tokens, "d_head": wl.d_head, "d_latent": wl.d_latent, "fanout": list(wl.fanout),
                   "b": wl.b, "k": wl.k, "sink": wl.sink, "window": wl.window},
        "keys_scored_per_s": keys_scored / (ms_step * 1e-3),
        "keys_scored_per_step": keys_scored,
        "roofline": roof,
        "select_path": "node-major" if node_major else "per-query-head",
        "stages_ms": {name: stage_ms.get(st) for name, st in (("descend", _abi.STAGE_DESCEND),
                      ("sample", _abi.STAGE_SAMPLE), ("gather", _abi.STAGE_GATHER), ("merge", _abi.STAGE_MERGE))},
        "build_ms": build_ms,
        "index_bytes": int(li.index.numel()),
        "graph_replay": graph,
    }
    if centroid is not None:
        result["centroid_scoring"] = centroid

    if not args.no_flat and node_major:
        # The full scan of the whole chunk on the matrix cores (row-tiled):
        # every key scored against every query head, with the same output
        # rows as the tree.
        fout = li.alloc_select_outputs(wl.n_tokens, wl.n_q_heads, prm, scores=True, flat=True)
        li.flat_select(qd, pd, prm, out=fout)
        fstep = lambda: li.flat_select(qd, pd, prm, out=fout)  # noqa: E731
        fsteps = args.flat_steps or 3
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(fsteps):
            fstep()
        torch.cuda.synchronize()
        flat_ms = (time.perf_counter() - t0) * 1e3 / fsteps
        fstages = [_abi.STAGE_PROJECT, _abi.STAGE_SAMPLE, _abi.STAGE_FLAT, _abi.STAGE_MERGE]
        _, fst = timed_steps(fstep, fsteps, hip, fstages, _abi)
        scan_ms = fst[_abi.STAGE_FLAT]
        fflops = qheads * wl.n_keys * 2 * wl.d_latent
        rec = recall_rows(out[0], fout[0], wl.sink, wl.k)
        result["flat"] = {
            "ms_per_call": flat_ms, "query_heads_per_s": qheads / (flat_ms * 1e-3),
            "keys_scored_per_s": qheads * wl.n_keys / (flat_ms * 1e-3),
            "path": "row-tiled (matrix cores)", "kernel": "fs_scan_kernel", "kernel_ms": scan_ms,
            "algorithmic_flops_per_launch": fflops,
            "achieved_TFLOPs": fflops / (scan_ms * 1e-3) / 1e12,
            "frac_of_mfma_peak": fflops / (scan_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "stages_ms": {name: fst.get(st) for name, st in (("project", _abi.STAGE_PROJECT),
                          ("sample", _abi.STAGE_SAMPLE), ("scan", _abi.STAGE_FLAT), ("merge", _abi.STAGE_MERGE))},
            "traffic": load_traffic(wl.name, "fs_scan"),
        }
        result["recall_at_k_vs_flat"] = {"mean": float(rec.mean()), "p5": float(np.percentile(rec, 5)),
                                         "rows": int(rec.size)}
        result["speedup_vs_flat"] = flat_ms / ms_step
    elif not args.no_flat:
        fsteps = args.flat_steps or max(5, min(args.steps, 50))
        fout = li.alloc_select_outputs(wl.n_tokens, wl.n_q_heads, prm, scores=True, flat=True)
        for _ in range(3):
            li.flat_select(qd, pd, prm, out=fout)
        fstep = lambda: li.flat_select(qd, pd, prm, out=fout)  # noqa: E731
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(fsteps):
            fstep()
        torch.cuda.synchronize()
        flat_ms = (time.perf_counter() - t0) * 1e3 / fsteps
        _, fst = timed_steps(fstep, max(1, min(fsteps, 10)), hip, [_abi.STAGE_FLAT], _abi)
        flat_kernel_ms = fst[_abi.STAGE_FLAT]
        flat_idx = fout[0].cpu().numpy()
        s0, k = wl.sink, wl.k
        rec = []
        for t_ in range(wl.n_tokens):
            for hq in range(wl.n_q_heads):
                a = tree_idx[t_, hq, s0:s0 + k]
                b = flat_idx[t_, hq, s0:s0 + k]
                a, b = set(a[a >= 0].tolist()), set(b[b >= 0].tolist())
                rec.append(len(a & b) / max(1, len(b)))
        flat_bytes = wl.n_tokens * wl.n_kv_heads * wl.n_keys * row_bytes
        result["flat"] = {
            "ms_per_call": flat_ms, "query_heads_per_s": qheads / (flat_ms * 1e-3),
            "keys_scored_per_s": qheads * wl.n_keys / (flat_ms * 1e-3),
            "kernel": "flat_kernel", "kernel_ms": flat_kernel_ms,
            "achieved_GBs": flat_bytes / (flat_kernel_ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": flat_bytes / (flat_kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": load_traffic(wl.name, "flat"),
        }
        result["recall_at_k_vs_flat"] = {"mean": float(np.mean(rec)), "p5": float(np.percentile(rec, 5))}
        result["speedup_vs_flat"] = flat_ms / ms_step

    if pca is not None:
        result["pca_map"] = pca
    if not args.no_attention:
        log("exact sparse attention over the selected rows")
        result["sparse_attention"] = attention_leg(_abi, desc, wl, qd, kd, out[0],
                                                   reps=20 if wl.n_tokens == 1 else 2)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, keys, W, queries, pos)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
