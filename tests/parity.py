"""Comparison of the HIP path's outputs with the CPU oracle, to the stated
tolerances.

* scores: |s_gpu - s_ref| <= 1e-3 * sum_i |q~_i k~_i| (fp32 accumulation of a
  64-term dot product errs by about 4e-6 of that scale, so a failure is a bug);
* key sets: equal, except for swaps whose oracle score lies within
  1e-3 * scale of the oracle's k-th score; sink and window segments exact;
* leaf sets: the GPU's descent must be a valid top-b choice at every level
  (every kept child scores >= every dropped sibling, up to the same
  tolerance); key sets are then compared against the oracle's key stage run on
  the GPU's leaves, so one legitimate near-tie swap cannot cascade.
"""
from __future__ import annotations

import numpy as np

from oracle import lsa_oracle as O

TOL = 1e-3


def log(msg: str) -> None:
    """Progress line that names the running case (flushed at once)."""
    print(msg, flush=True)


def check_leaves(hidx, fanout, qlat, b, beam, gpu_leaves):
    """The GPU leaf set is a valid descent (per-parent or global top-b at
    every level, ties up to TOL of the score scale).  Returns the leaf list."""
    leaves = np.array(sorted(int(x) for x in gpu_leaves if x >= 0), dtype=np.int64)
    assert len(set(leaves.tolist())) == len(leaves), "duplicate leaves"
    L = len(fanout)
    if beam == "global":
        # the frontier above the leaves comes from the oracle's own descent;
        # the GPU's leaves must be a valid top-b of that frontier's children
        frontier = O.descend(hidx, fanout[:-1], qlat, b, beam) if L > 1 else np.zeros(1, dtype=np.int64)
        f = fanout[-1]
        cnt = np.diff(hidx.offsets[-1])
        kids = (frontier[:, None] * f + np.arange(f)[None, :]).ravel()
        kids = kids[cnt[kids] > 0]
        assert set(leaves.tolist()) <= set(kids.tolist()), "leaves outside the frontier's children"
        _valid_top(hidx.cscore[-1], kids, set(leaves.tolist()), qlat, b, L)
        return leaves
    # ancestors of the kept leaves at every level (level L = the leaves)
    anc = [None] * (L + 1)
    anc[L] = leaves
    for lev in range(L - 1, -1, -1):
        anc[lev] = np.unique(anc[lev + 1] // fanout[lev])
    assert anc[0].tolist() in ([0], []), "leaves from more than one root"
    for lev in range(1, L + 1):
        f = fanout[lev - 1]
        cnt = np.diff(hidx.offsets[lev - 1])
        kept = set(anc[lev].tolist())
        for p in anc[lev - 1]:
            kids = np.arange(p * f, (p + 1) * f)
            kids = kids[cnt[kids] > 0]
            _valid_top(hidx.cscore[lev - 1], kids, kept, qlat, b, lev)
    return leaves


def _valid_top(cscore, kids, kept, qlat, b, lev):
    """``kept`` holds min(b, |kids|) of ``kids``, and none of the dropped ones
    scores above a kept one by more than the tolerance."""
    sc = cscore[kids] @ qlat
    scale = O.dot_scale(qlat, cscore[kids])
    mine = np.array([k in kept for k in kids])
    assert mine.sum() == min(b, len(kids)), f"level {lev}: kept {mine.sum()} of {len(kids)} children, b={b}"
    if mine.all() or not mine.any():
        return
    worst_kept = np.min(sc[mine] + TOL * scale[mine])
    best_dropped = np.max(sc[~mine] - TOL * scale[~mine])
    assert worst_kept >= best_dropped, f"level {lev}: a dropped child beats a kept one beyond tolerance"


def check_row(gpu_row, gpu_scores, res, p, prm: O.SelectParams, what=""):
    """One output row (and its scores) against the oracle's per-query result
    ``res`` (from O.select_one on the same leaf set)."""
    sink, k, window = prm.sink, prm.k, prm.window
    s, w, _ = O.segments(p, sink, window)
    assert gpu_row[:sink].tolist() == s + [-1] * (sink - len(s)), f"{what}: sink segment"
    assert gpu_row[sink + k:].tolist() == w + [-1] * (window - len(w)), f"{what}: window segment"
    top = np.asarray(gpu_row[sink:sink + k])
    n_ref = len(res["top_idx"])
    valid = top[top >= 0]
    assert len(valid) == n_ref, f"{what}: {len(valid)} selected, oracle {n_ref}"
    assert np.all(top[n_ref:] == -1), f"{what}: padding"
    assert np.all(np.diff(valid) > 0), f"{what}: not ascending / duplicates"
    cand = dict(zip(res["cand_idx"].tolist(), range(len(res["cand_idx"]))))
    missing = [j for j in valid.tolist() if j not in cand]
    assert not missing, f"{what}: selected keys outside the candidate set: {missing[:5]}"
    ci = np.array([cand[j] for j in valid.tolist()], dtype=np.int64)
    ref_s = res["cand_scores"][ci]
    scale = res["cand_scale"][ci]
    if gpu_scores is not None:
        gs = np.asarray(gpu_scores[:len(valid)], dtype=np.float64)
        bad = np.abs(gs - ref_s) > TOL * scale
        assert not bad.any(), f"{what}: {bad.sum()} scores off, e.g. gpu {gs[bad][:3]} ref {ref_s[bad][:3]}"
        assert np.all(np.isneginf(np.asarray(gpu_scores[len(valid):]))), f"{what}: score padding"
    g, o = set(valid.tolist()), set(res["top_idx"].tolist())
    if g != o:
        tau = res["kth"]
        assert np.isfinite(tau), f"{what}: sets differ with fewer candidates than k"
        for j in g ^ o:
            c = cand[j]
            assert abs(res["cand_scores"][c] - tau) <= TOL * res["cand_scale"][c], \
                f"{what}: key {j} differs (score {res['cand_scores'][c]}, k-th {tau})"
    return len(g ^ o)


def compare_select(oidx, queries, q_pos, prm, gpu_idx, gpu_scores, gpu_leaves=None, pairs=None, flat=False,
                   log=None, appended=None):
    """Compare GPU rows with the oracle for the given (t, hq) pairs (all by
    default); ``appended`` (one O.Appended per KV head) adds keys appended
    after the build.  Returns the number of tolerated near-tie swaps."""
    desc = oidx.desc
    T, Hq = queries.shape[0], queries.shape[1]
    g = Hq // desc.n_kv_heads
    pairs = pairs if pairs is not None else [(t, hq) for t in range(T) for hq in range(Hq)]
    swaps = 0
    for (t, hq) in pairs:
        h = hq // g
        p = int(q_pos[t])
        qlat = O.query_latent(queries[t, hq], oidx.heads[h], desc.key_dtype, desc.latent_dtype)
        leaves = None
        if not flat:
            if gpu_leaves is not None:
                leaves = check_leaves(oidx.heads[h], desc.fanout, qlat, prm.b, prm.beam, gpu_leaves[t, hq])
            else:
                leaves = None
        res = O.select_one(oidx, h, qlat, p, prm, flat=flat, leaves=leaves,
                           appended=None if appended is None else appended[h])
        swaps += check_row(gpu_idx[t, hq], None if gpu_scores is None else gpu_scores[t, hq], res, p, prm,
                           what=f"(t={t}, hq={hq}, p={p})")
    if log:
        log(f"compared {len(pairs)} query heads, {swaps} near-tie swaps")
    return swaps


def csr_from_assignment(leaf_of_key: np.ndarray, n_leaves: int):
    """CSR of an assignment, by definition: counts, offsets, stable order."""
    counts = np.bincount(leaf_of_key, minlength=n_leaves)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(leaf_of_key, kind="stable")
    return offsets, perm


def check_build(gidx, keys, W, desc: O.IndexDesc, sample=None, log=None):
    """Properties of a GPU-built index (read back from its blob) that must
    hold whatever the k-means trajectory: latent within 1 ulp of the oracle's
    projection, CSR bit-exact from the GPU's own assignment, every key at its
    nearest centroid (GPU centroids, float64 distances) within 1e-4."""
    rng = np.random.default_rng(123)
    for h, hh in enumerate(gidx.heads):
        n = desc.n_keys
        assert np.array_equal(np.sort(hh.perm), np.arange(n)), "perm is not a bijection"
        rows = np.arange(n) if sample is None or sample >= n else np.sort(rng.choice(n, sample, replace=False))
        keys_h = keys[hh.perm[rows], h, :]
        ref = O.latent_keys(keys_h, W[h], desc.key_dtype, desc.latent_dtype)
        got = hh.csr_latent[rows]
        # fp32 accumulation of d_head products errs by at most about
        # d_head * 2^-24 * sum_i |k_i W_i| (< 1e-5 of that scale), before the
        # one rounding to the latent dtype (one ulp of the exact value)
        sc = np.abs(O.stored_to_f64(keys_h, desc.key_dtype)) @ np.abs(W[h].astype(np.float64))
        if desc.latent_dtype == "bf16":
            ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
        else:
            ulp = np.zeros_like(ref)
        assert np.all(np.abs(got - ref) <= ulp * 1.0000001 + 1e-5 * sc), "latent beyond 1 ulp + accumulation bound"
        lat = np.empty_like(hh.csr_latent)
        lat[hh.perm] = hh.csr_latent
        for lev in range(desc.n_levels):
            nodes = desc.nodes(lev + 1)
            off, perm = csr_from_assignment(hh.assign[lev], nodes)
            assert np.array_equal(off, hh.offsets[lev]), f"head {h} level {lev + 1}: offsets"
            if lev == desc.n_levels - 1:
                assert np.array_equal(perm, hh.perm), f"head {h}: perm is not the stable CSR order"
            f = desc.fanout[lev]
            mcount = np.array([n]) if lev == 0 else np.diff(hh.offsets[lev - 1])
            cent = hh.centroids[lev].reshape(-1, f, lat.shape[1])
            ks = np.arange(n) if sample is None or sample >= n else np.sort(rng.choice(n, sample, replace=False))
            for c0 in range(0, len(ks), 2048):
                kk = ks[c0:c0 + 2048]
                x = lat[kk]
                node = hh.assign[lev][kk]
                pk = node // f
                nv = np.minimum(mcount[pk], f)
                d2 = ((x[:, None, :] - cent[pk]) ** 2).sum(-1)               # [m, F]
                d2[np.arange(f)[None, :] >= nv[:, None]] = np.inf
                best = d2.min(axis=1)
                mine = d2[np.arange(len(kk)), node % f]
                ok = mine <= best * (1 + 1e-4) + 1e-6 * (x * x).sum(-1)
                assert ok.all(), f"head {h} level {lev + 1}: {np.sum(~ok)} keys not at their nearest centroid"
    if log:
        log("build properties hold")


def fixed_point_step(lat_all: np.ndarray, n_keys: int) -> float:
    """Quantisation step of the GPU build's fixed-point centroid sums, from
    the rule include/lsa.h states: every |latent| < 2^e (e the smallest such
    exponent, at least -126), at most 2^c members with 2^c >= N, and step
    2^-(61 - c - e) (the shift clamped to [-100, 100])."""
    m = float(np.max(np.abs(lat_all))) if lat_all.size else 0.0
    e = max(int(np.frexp(m)[1]), -126) if m > 0 else -126
    c = int(np.ceil(np.log2(n_keys))) if n_keys > 1 else 0
    while (1 << c) < n_keys:
        c += 1
    shift = min(100, max(-100, 61 - c - e))
    return float(np.ldexp(1.0, -shift))


def check_lloyd_update(gidx, desc: O.IndexDesc, step: float, log=None, tie_rel=2e-5):
    """One Lloyd round (kmeans_iters = 1), at every level of every head: the
    stored centroids are the update that follows the first assignment.

    For every parent, its members are read from the index's own partition of
    the level above (ascending key order).  The oracle draws the parent's
    initial centroids (seeded Forgy), assigns each member to the nearest one in
    float64 and takes each child's member mean.  An initialised child must then
    hold that mean rounded to fp32, within the fixed-point step of the sums
    (``step``) plus one fp32 ulp; a child that received no member keeps its
    initial centroid exactly; a void child stays zero.  A member whose two
    nearest initial centroids lie within ``tie_rel`` of each other, relative to
    S = |x|^2 + |mu_a|^2 + |mu_b|^2, may go either way in fp32, so the two
    children it touches are not compared.  The GPU evaluates |mu|^2 - 2 x.mu
    with fp32 sums of at most 64 and 33 products; the standard bound
    gamma_n sum|a_i b_i| puts the error of a difference of two such distances
    below 99 * 2^-24 * S = 5.9e-6 S, so 2e-5 S leaves a margin.  Returns
    (children compared, children skipped)."""
    assert desc.kmeans_iters == 1
    compared = skipped = 0
    for h, hh in enumerate(gidx.heads):
        lat = np.empty_like(hh.csr_latent)
        lat[hh.perm] = hh.csr_latent
        for lev, f in enumerate(desc.fanout):
            if lev == 0:
                members = [np.arange(desc.n_keys)]
            else:
                order = np.argsort(hh.assign[lev - 1], kind="stable")
                cuts = np.searchsorted(hh.assign[lev - 1][order], np.arange(desc.nodes(lev) + 1))
                members = [order[cuts[p]:cuts[p + 1]] for p in range(desc.nodes(lev))]
            got = hh.centroids[lev]
            for p, mem in enumerate(members):
                pos = O.kmeans_init_positions(desc.seed, h, lev + 1, p, len(mem), f)
                nv = len(pos)
                g = got[p * f:(p + 1) * f]
                assert np.all(g[nv:] == 0.0), f"head {h} level {lev + 1} node {p}: void child not zero"
                if nv == 0:
                    continue
                x = lat[mem]
                init = O.round_f32(x[np.asarray(pos)])
                xx = np.einsum("ij,ij->i", x, x)
                d2 = O.sq_dists(x, init, xx)
                a = np.argmin(d2, axis=1)
                unsure = np.zeros(nv, dtype=bool)
                if nv > 1:
                    part = np.partition(d2, 1, axis=1)
                    mm = np.einsum("ij,ij->i", init, init)
                    second = np.argsort(d2, axis=1, kind="stable")[:, 1]
                    near = (part[:, 1] - part[:, 0]) <= tie_rel * (xx + mm[a] + mm[second])
                    unsure[a[near]] = True
                    unsure[second[near]] = True
                cnt, sums = O.member_means(x, a, nv)
                for c in range(nv):
                    if unsure[c]:
                        skipped += 1
                        continue
                    compared += 1
                    if cnt[c] == 0:
                        assert np.array_equal(g[c], init[c]), \
                            f"head {h} level {lev + 1} node {p} child {c}: empty child moved"
                        continue
                    mean = sums[c] / cnt[c]
                    tol = step + np.spacing(np.abs(mean).astype(np.float32)).astype(np.float64)
                    bad = np.abs(g[c] - mean) > tol
                    assert not bad.any(), (f"head {h} level {lev + 1} node {p} child {c}: centroid is not the "
                                           f"member mean (max err {np.max(np.abs(g[c] - mean)):.3g})")
    if log:
        log(f"Lloyd update: {compared} children equal their member means, {skipped} skipped at near-ties")
    return compared, skipped


def check_appended(oidx, keys_new, W, desc: O.IndexDesc, gpu_leaf, gpu_lat, log=None):
    """Keys appended on the GPU (pool leaves [Hkv][A], latents [Hkv][A][dl])
    against the oracle: latents within one ulp plus the fp32 accumulation
    bound (as for the build), and every routing step valid: at each level
    the child taken holds keys and its squared distance (float64, stored
    centroids) is the smallest among the non-empty siblings up to 1e-4
    relative (fp32 distances may swap near-ties).  Returns the number of
    keys whose leaf differs from the oracle's own routing."""
    diffs = 0
    for h, hh in enumerate(oidx.heads):
        ref = O.latent_keys(keys_new[:, h, :], W[h], desc.key_dtype, desc.latent_dtype)
        sc = np.abs(O.stored_to_f64(keys_new[:, h, :], desc.key_dtype)) @ np.abs(W[h].astype(np.float64))
        ulp = (np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8) if desc.latent_dtype == "bf16"
               else np.zeros_like(ref))
        got = gpu_lat[h]
        assert np.all(np.abs(got - ref) <= ulp * 1.0000001 + 1e-5 * sc), f"head {h}: appended latent"
        for i, x in enumerate(got):
            leaf = int(gpu_leaf[h][i])
            assert leaf >= 0, f"head {h} key {i}: not appended"
            node, path = leaf, []
            for lev in range(desc.n_levels - 1, -1, -1):
                path.append((lev, node))
                node //= desc.fanout[lev]
            for lev, kid in reversed(path):
                f = desc.fanout[lev]
                par = kid // f
                kids = par * f + np.arange(f)
                ne = np.diff(hh.offsets[lev])[kids] > 0
                assert ne[kid - par * f], f"head {h} key {i}: routed into an empty node"
                d2 = ((hh.centroids[lev][kids] - x) ** 2).sum(-1)
                best = d2[ne].min()
                assert d2[kid - par * f] <= best * (1 + 1e-4) + 1e-6 * float(x @ x), \
                    f"head {h} key {i} level {lev + 1}: not the nearest non-empty child"
            diffs += leaf != O.route_key(hh, desc.fanout, x)
    if log:
        log(f"appended keys: latents and routes hold, {diffs} near-tie routes differ from the oracle's")
    return diffs
