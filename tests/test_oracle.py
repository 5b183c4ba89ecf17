"""Pins of the CPU oracle against facts that do not come from the oracle itself:
published known answers, library routines, textbook properties, exhaustive
brute force on tiny inputs and the invariants the method fixes.  CPU only."""
import itertools
import os
import struct

import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import workloads as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.5, 3.0e38, 1e-40]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_single_rounding_and_ties():
    # halfway between 1 and 1 + 2^-7 -> ties to even (1.0)
    assert O.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # halfway between 1 + 2^-7 and 1 + 2^-6 -> even mantissa is 1 + 2^-6
    assert O.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above halfway: one rounding from float64 must round up (rounding
    # through fp32 first would land on the tie and go down to 1.0)
    assert O.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert O.round_bf16(np.array([np.pi]))[0] == 3.140625


def test_bf16_storage_round_trip():
    vals = O.round_bf16(np.random.default_rng(2).standard_normal(1000))
    assert np.array_equal(O.bf16_bits_to_f64(O.f64_to_bf16_bits(vals)), vals)


def test_synth_bf16_storage_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(50000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S.f32_to_bf16_bits(x), ref)


# --------------------------------------------------------------------------
# splitmix64 and the seeded init
# --------------------------------------------------------------------------

def test_splitmix64_known_answers():
    with open(os.path.join(GOLDEN, "splitmix64_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for r in rows:
        g = O.SplitMix64(int(r[0]))
        assert [g.next() for _ in r[1:]] == [int(v) for v in r[1:]]


@pytest.mark.parametrize("m,f", [(1, 4), (3, 4), (4, 4), (5, 4), (1000, 64), (65, 64), (65536, 256)])
def test_kmeans_init_distinct_and_in_range(m, f):
    a = O.kmeans_init_positions(77, 3, 2, 5, m, f)
    assert len(a) == min(m, f)
    assert len(set(a)) == len(a)
    assert all(0 <= u < m for u in a)
    if m <= f:
        assert a == list(range(m))
    assert a == O.kmeans_init_positions(77, 3, 2, 5, m, f)
    if m > f:
        assert a != O.kmeans_init_positions(77, 3, 2, 6, m, f)


def test_kmeans_init_first_draw_is_splitmix_of_node_seed():
    # the first chosen ordinal is the first output of the node's stream mod m
    seed, h, lev, node, m = 123, 1, 2, 7, 1 << 20
    tag = ((h * 16 + lev) << 32) + node
    start = seed ^ O.SplitMix64(tag).next()
    assert O.kmeans_init_positions(seed, h, lev, node, m, 4)[0] == O.SplitMix64(start).next() % m


# --------------------------------------------------------------------------
# Lloyd k-means
# --------------------------------------------------------------------------

def _blobs(n, f, d, seed, spread=0.05):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((f, d)) * 4
    lab = rng.integers(0, f, n)
    return O.round_f32(centers[lab] + spread * rng.standard_normal((n, d))), lab


def test_lloyd_textbook_1d():
    x = np.array([[0.0], [1.0], [10.0], [11.0]])
    c, a, nv = O.lloyd(x, 2, 5, [0, 1])
    assert nv == 2
    assert sorted(c[:, 0].tolist()) == [0.5, 10.5]
    assert a[0] == a[1] and a[2] == a[3] and a[0] != a[2]


def test_lloyd_objective_non_increasing():
    rng = np.random.default_rng(4)
    x = O.round_f32(rng.standard_normal((3000, 8)))
    init = O.kmeans_init_positions(9, 0, 1, 0, len(x), 16)
    prev = np.inf
    for t in range(0, 12):
        c, a, _ = O.lloyd(x, 16, t, init)
        j = O.lloyd_objective(x, c, a)
        assert j <= prev * (1 + 1e-9)
        prev = j


def test_lloyd_matches_sklearn():
    km = pytest.importorskip("sklearn.cluster")
    x, _ = _blobs(4096, 16, 32, 5, spread=0.7)
    init = O.kmeans_init_positions(11, 0, 1, 0, len(x), 16)
    c, a, _ = O.lloyd(x, 16, 10, init)
    ref = km.KMeans(n_clusters=16, init=x[init], n_init=1, max_iter=10, tol=0.0,
                    algorithm="lloyd").fit(x)
    assert np.bincount(a, minlength=16).min() > 0          # no empty cluster (sklearn relocates those)
    assert np.mean(ref.labels_ == a) >= 0.999
    assert np.allclose(ref.cluster_centers_, c, rtol=0, atol=1e-5)


def test_lloyd_empty_cluster_keeps_centroid_and_void_children():
    # two far points, three children: member-count < fanout => the third child is void
    x = np.array([[0.0, 0.0], [5.0, 5.0]])
    c, a, nv = O.lloyd(x, 3, 3, O.kmeans_init_positions(1, 0, 1, 0, 2, 3))
    assert nv == 2 and sorted(a.tolist()) == [0, 1] and np.all(c[2] == 0)
    # a duplicate init point: the higher-index duplicate never wins a tie and
    # keeps its initial centroid while empty
    x = np.array([[0.0], [0.0], [9.0]])
    c, a, _ = O.lloyd(x, 3, 4, [0, 1, 2])
    assert a.tolist() == [0, 0, 2] and c[1, 0] == 0.0


def test_centroid_score_is_member_mean_score_when_converged():
    # closed form: q . mu_c = mean_{j in c} q . x_j when mu_c is the mean of c
    x, _ = _blobs(2000, 8, 16, 6, spread=0.02)
    init = O.kmeans_init_positions(3, 0, 1, 0, len(x), 8)
    c, a, _ = O.lloyd(x, 8, 20, init)
    c2, a2, _ = O.lloyd(x, 8, 21, init)
    assert np.array_equal(a, a2)                        # converged
    q = np.random.default_rng(7).standard_normal(16)
    for cl in range(8):
        m = x[a == cl]
        assert abs(c[cl] @ q - np.mean(m @ q)) <= 1e-6 * (np.abs(m) @ np.abs(q)).mean()


# --------------------------------------------------------------------------
# index build: CSR invariants
# --------------------------------------------------------------------------

def _small_wl(fanout, n=600, kv=2, group=2, iters=4, latent="bf16", key="bf16", dl=16, centers=40, t=8,
              b=2, k=7, sink=4, window=16):
    return S.get_workload("decode_1m").scaled(
        name="small", n_keys=n, n_kv_heads=kv, group=group, d_latent=dl, key_dtype=key,
        latent_dtype=latent, fanout=tuple(fanout), kmeans_iters=iters, n_centers=centers,
        n_tokens=t, b=b, k=k, sink=sink, window=window)


def _build(wl):
    keys = S.gen_keys(wl)
    W = S.gen_W(wl)
    idx = O.build_index(keys, W, O.IndexDesc.of(wl))
    return keys, W, idx


@pytest.mark.parametrize("fanout", [(16,), (4, 4), (8, 8), (4, 3, 5)])
def test_csr_invariants(fanout):
    wl = _small_wl(fanout)
    keys, W, idx = _build(wl)
    for h, hh in enumerate(idx.heads):
        n = wl.n_keys
        assert sorted(hh.perm.tolist()) == list(range(n))
        for lev, off in enumerate(hh.offsets):
            pn = idx.desc.nodes(lev + 1)
            assert len(off) == pn + 1 and off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
            # every key sits in the range of its node at this level
            pos = np.empty(n, dtype=np.int64)
            pos[hh.perm] = np.arange(n)
            node = hh.assign[lev]
            assert np.all((off[node] <= pos) & (pos < off[node + 1]))
            if lev > 0:  # a node's range is the union of its children's ranges
                f = wl.fanout[lev]
                assert np.array_equal(hh.offsets[lev - 1], off[::f])
        off = hh.offsets[-1]
        for leaf in range(len(off) - 1):
            seg = hh.perm[off[leaf]:off[leaf + 1]]
            assert np.all(np.diff(seg) > 0)                      # ascending within a leaf
        lat = O.latent_keys(keys[:, h, :], W[h], wl.key_dtype, wl.latent_dtype)
        assert np.array_equal(hh.csr_latent, lat[hh.perm])


def test_build_assignments_are_nearest_centroid():
    wl = _small_wl((8, 8), n=2000)
    keys, W, idx = _build(wl)
    for h, hh in enumerate(idx.heads):
        lat = O.latent_keys(keys[:, h, :], W[h], wl.key_dtype, wl.latent_dtype)
        for lev, f in enumerate(wl.fanout):
            node = hh.assign[lev]
            parent = node // f
            for p in np.unique(parent):
                mem = np.nonzero(parent == p)[0]
                kids = np.arange(p * f, (p + 1) * f)
                kids = kids[hh.valid[lev][kids]]
                # brute-force distances, pure definition
                d2 = ((lat[mem][:, None, :] - hh.centroids[lev][kids][None]) ** 2).sum(-1)
                best = d2.min(axis=1)
                mine = ((lat[mem] - hh.centroids[lev][node[mem]]) ** 2).sum(-1)
                assert np.all(mine <= best * (1 + 1e-12) + 1e-12)


# --------------------------------------------------------------------------
# selection: brute force, invariants, tree == flat
# --------------------------------------------------------------------------

def _brute_select(hh, fanout, qlat, p, prm):
    """Pure-Python brute force: a leaf is selected iff along its path each node
    ranks within the top-b of its non-empty siblings by (score desc, id asc)."""
    def score(vec):
        return sum(float(a) * float(b) for a, b in zip(vec, qlat))

    counts = [np.diff(o) for o in hh.offsets]
    nleaf = len(hh.offsets[-1]) - 1
    selected = []
    for leaf in range(nleaf):
        ok = True
        node = leaf
        for lev in range(len(fanout) - 1, -1, -1):
            f = fanout[lev]
            par = node // f
            sib = [par * f + c for c in range(f) if counts[lev][par * f + c] > 0]
            if node not in sib:
                ok = False
                break
            me = (score(hh.cscore[lev][node]), node)
            rank = sum(1 for s in sib if (score(hh.cscore[lev][s]) > me[0]) or
                       (score(hh.cscore[lev][s]) == me[0] and s < node))
            if rank >= prm.b:
                ok = False
                break
            node = par
        if ok:
            selected.append(leaf)
    lo, hi = prm.sink, p - prm.window
    cand = []
    for leaf in selected:
        for r in range(hh.offsets[-1][leaf], hh.offsets[-1][leaf + 1]):
            j = int(hh.perm[r])
            if lo <= j <= hi:
                cand.append((-score(hh.csr_latent[r]), j))
    top = sorted(cand)[:prm.k]
    return sorted(selected), sorted(j for _, j in top)


def _int_index(fanout, n, dl, seed):
    """An index over small-integer latents, so dot products are exact and
    equal scores (ties) are common."""
    rng = np.random.default_rng(seed)
    desc = O.IndexDesc(n, 1, 8, dl, "f32", "f32", tuple(fanout), 0, 0)
    leaves = desc.nodes(len(fanout))
    # about a third of the leaves stay empty, and so does the whole subtree of
    # the last top-level node, so the empty-bucket rule is exercised
    allowed = np.nonzero(rng.random(leaves) > 0.35)[0]
    allowed = allowed[allowed < leaves - leaves // fanout[0]] if len(fanout) > 1 else allowed
    leaf_of = rng.choice(allowed, n)
    perm = np.lexsort((np.arange(n), leaf_of))
    cnt = np.bincount(leaf_of, minlength=leaves)
    offs, cents, cs = [], [], []
    for lev in range(len(fanout)):
        pn = desc.nodes(lev + 1)
        group = leaves // pn
        c = cnt.reshape(pn, group).sum(1)
        offs.append(np.concatenate([[0], np.cumsum(c)]))
        cen = rng.integers(-2, 3, (pn, dl)).astype(np.float64)
        cents.append(cen)
        cs.append(cen)
    lat = rng.integers(-2, 3, (n, dl)).astype(np.float64)
    hh = O.HeadIndex(W=np.zeros((8, dl)), centroids=cents, cscore=cs, offsets=offs, valid=[None] * len(fanout),
                     perm=perm, csr_latent=lat[perm], assign=[None] * len(fanout))
    return O.OracleIndex(desc=desc, heads=[hh]), rng


@pytest.mark.parametrize("fanout", [(16,), (4, 4), (8, 8)])
def test_exhaustive_brute_force_tiny(fanout):
    n = 512
    idx, rng = _int_index(fanout, n, 6, seed=sum(fanout))
    hh = idx.heads[0]
    ps = sorted(set([0, 1, 3, 4, 5, 16, 17, 20, 21, 255, 511] + rng.integers(0, n, 9).tolist()))
    qs = [rng.integers(-2, 3, 6).astype(np.float64) for _ in range(3)]
    for qlat in qs:
        for b in range(1, fanout[0] + 1):
            for k, sink, window in itertools.product((1, 7, 64), (0, 4), (0, 16)):
                prm = O.SelectParams(b=b, k=k, sink=sink, window=window)
                for p in ps:
                    res = O.select_one(idx, 0, qlat, p, prm)
                    leaves, top = _brute_select(hh, idx.desc.fanout, qlat, p, prm)
                    assert sorted(res["leaves"].tolist()) == leaves
                    assert res["top_idx"].tolist() == top, (b, k, sink, window, p)


def test_global_beam_brute_force():
    idx, rng = _int_index((4, 4), 256, 5, seed=11)
    hh = idx.heads[0]
    for _ in range(20):
        qlat = rng.integers(-2, 3, 5).astype(np.float64)
        for b in (1, 2, 3, 5):
            got = O.descend(hh, (4, 4), qlat, b, "global")
            # brute force: level 1 top-b roots, then top-b over all their non-empty children
            cnt1, cnt2 = np.diff(hh.offsets[0]), np.diff(hh.offsets[1])
            s1 = [(-(hh.cscore[0][c] @ qlat), c) for c in range(4) if cnt1[c] > 0]
            l1 = [c for _, c in sorted(s1)[:b]]
            s2 = [(-(hh.cscore[1][p * 4 + c] @ qlat), p * 4 + c) for p in l1 for c in range(4) if cnt2[p * 4 + c] > 0]
            assert got.tolist() == [c for _, c in sorted(s2)[:b]]


def _check_row_invariants(row, p, prm, n_cand_top):
    s, w, _ = O.segments(p, prm.sink, prm.window)
    assert row[:prm.sink].tolist() == s + [-1] * (prm.sink - len(s))
    assert row[prm.sink + prm.k:].tolist() == w + [-1] * (prm.window - len(w))
    top = row[prm.sink:prm.sink + prm.k]
    valid = top[top >= 0]
    assert len(valid) == n_cand_top and np.all(top[len(valid):] == -1)
    assert np.all(np.diff(valid) > 0)
    allv = row[row >= 0]
    assert allv.max(initial=-1) <= p and len(set(allv.tolist())) == len(allv)
    assert np.all((valid >= prm.sink) & (valid <= p - prm.window))


@pytest.mark.parametrize("fanout,b", [((16,), 16), ((4, 4), 4), ((8, 8), 8), ((4, 3, 5), 5)])
def test_tree_with_all_buckets_equals_flat(fanout, b):
    wl = _small_wl(fanout, n=700, k=33, b=b, t=16)
    keys, W, idx = _build(wl)
    q = S.gen_queries(wl, keys)
    pos = np.linspace(0, wl.n_keys - 1, wl.n_tokens).astype(np.int32)
    prm = O.SelectParams(b=b, k=wl.k, sink=wl.sink, window=wl.window)
    tr, ts, _, _ = O.select(idx, q, pos, prm)
    fr, fs, _, res = O.flat_select(idx, q, pos, prm)
    for key in tr:
        assert np.array_equal(tr[key], fr[key])
        assert np.array_equal(ts[key], fs[key])
        _check_row_invariants(tr[key], int(pos[key[0]]), prm, min(prm.k, len(res[key]["cand_idx"])))


def test_output_invariants_and_flat_is_exact_topk():
    wl = _small_wl((8, 8), n=1500, k=40, b=3, t=24)
    keys, W, idx = _build(wl)
    q = S.gen_queries(wl, keys)
    pos = np.concatenate([[0, 1, 3, 4, 10, 20, 21, 22], np.linspace(23, wl.n_keys - 1, 16)]).astype(np.int32)
    prm = O.SelectParams(b=wl.b, k=wl.k, sink=wl.sink, window=wl.window)
    rows, _, leaves, res = O.select(idx, q, pos, prm)
    frows, _, _, fres = O.flat_select(idx, q, pos, prm)
    g = wl.group
    for (t, hq), row in rows.items():
        p = int(pos[t])
        _check_row_invariants(row, p, prm, min(prm.k, len(res[(t, hq)]["cand_idx"])))
        # flat: an explicit definition -- every key of C(p) scored, best k kept
        h = hq // g
        lat = O.latent_keys(keys[:, h, :], W[h], wl.key_dtype, wl.latent_dtype)
        qlat = res[(t, hq)]["qlat"]
        cand = [(-(float(lat[j] @ qlat)), j) for j in range(prm.sink, p - prm.window + 1)]
        want = sorted(j for _, j in sorted(cand)[:prm.k])
        got = frows[(t, hq)][prm.sink:prm.sink + prm.k]
        assert got[got >= 0].tolist() == want
        # tree candidates are a subset of C(p) and the tree top-k is a top-k of them
        assert len(leaves[(t, hq)]) <= prm.b ** len(wl.fanout)


def test_global_and_per_parent_agree_on_one_level():
    wl = _small_wl((16,), n=500, b=4, k=20)
    keys, W, idx = _build(wl)
    q = S.gen_queries(wl, keys)
    pos = np.full(wl.n_tokens, wl.n_keys - 1, dtype=np.int32)
    a = O.select(idx, q, pos, O.SelectParams(4, 20, 4, 16, "per_parent"))[0]
    b = O.select(idx, q, pos, O.SelectParams(4, 20, 4, 16, "global"))[0]
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_fewer_candidates_than_k_pads():
    wl = _small_wl((4,), n=64, b=1, k=64, window=8, sink=2)
    keys, W, idx = _build(wl)
    q = S.gen_queries(wl, keys)
    pos = np.array([12] * wl.n_tokens, dtype=np.int32)
    prm = O.SelectParams(1, 64, 2, 8)
    rows, sc, _, res = O.select(idx, q, pos, prm)
    for key, row in rows.items():
        n = len(res[key]["cand_idx"])
        assert n < 64
        assert np.all(row[2 + n:2 + 64] == -1) and np.all(np.isneginf(sc[key][n:]))


# --------------------------------------------------------------------------
# blob layout
# --------------------------------------------------------------------------

def test_blob_header_fields_and_round_trip():
    wl = _small_wl((4, 3, 5), n=300)
    keys, W, idx = _build(wl)
    blob = O.index_blob(idx)
    lay = O.blob_layout(idx.desc)
    assert blob[:4].tobytes() == b"LSA1"
    (ver,) = struct.unpack_from("<I", blob, 4)
    (n,) = struct.unpack_from("<q", blob, 8)
    i32 = struct.unpack_from("<12i", blob, 16)
    seed, total, offw, offp, offl = struct.unpack_from("<5Q", blob, 64)
    cents = struct.unpack_from("<4Q", blob, 104)
    assert ver == 1 and n == 300 and i32[:6] == (2, 128, 16, 1, 1, 3) and i32[6:10] == (4, 3, 5, 0)
    assert total == len(blob) and offw == 256 and offp == lay["perm"] and offl == lay["latent"]
    assert cents[0] == lay["cent1"] and cents[3] == 0 and seed == wl.seed
    assert all(v % 256 == 0 for k_, v in lay.items())
    back = O.index_from_blob(blob, idx.desc)
    for a, b in zip(idx.heads, back.heads):
        assert np.array_equal(a.perm, b.perm) and np.array_equal(a.csr_latent, b.csr_latent)
        for lev in range(3):
            assert np.array_equal(a.offsets[lev], b.offsets[lev])
            assert np.array_equal(a.centroids[lev], b.centroids[lev])
            assert np.array_equal(a.cscore[lev], b.cscore[lev])
            assert np.array_equal(a.assign[lev], b.assign[lev])


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------

def test_generator_chunks_regenerate():
    wl = S.get_workload("decode_1m").scaled(n_keys=S.CHUNK + 5000, n_kv_heads=2)
    a = S.gen_keys_head_f32(wl, 1, S.CHUNK - 10, S.CHUNK + 10)
    b = S.gen_keys_head_f32(wl, 1, 0, S.CHUNK + 20)[S.CHUNK - 10:S.CHUNK + 10]
    assert np.array_equal(a, b)
    full = S.gen_keys(wl)
    assert full.dtype == np.uint16 and full.shape == (S.CHUNK + 5000, 2, 128)
    assert np.array_equal(full[S.CHUNK - 10:S.CHUNK + 10, 1], S.f32_to_bf16_bits(a))


def test_generator_distributions():
    wl = S.get_workload("decode_10m").scaled(n_keys=200000, n_kv_heads=1)
    x = S.gen_keys_head_f32(wl, 0)
    W = S.gen_W(wl)
    assert W.shape == (1, 128, 64) and abs(W.std() - 1 / np.sqrt(128)) < 2e-3
    # outliers are N(0, I): about 10% of keys sit far from every center
    c = S._centers(wl, 0)
    assert x.shape == (200000, 128) and c.shape == (65536, 128)
    q = S.gen_queries(wl.scaled(n_tokens=3), S.gen_keys(wl))
    assert q.shape == (3, 4, 128) and q.dtype == np.uint16


def test_lloyd_update_checker_accepts_the_definition_and_catches_wrong_updates():
    """The checker the GPU build is held to (tests/parity.check_lloyd_update)
    accepts the oracle's own one-round index and fails an index whose update
    was skipped, moved to another subset's mean, or nudged by more than the
    fixed-point step: a no-op or wrong update kernel cannot pass it."""
    from tests.parity import check_lloyd_update, fixed_point_step
    wl = S.get_workload("decode_1m").scaled(n_keys=3000, n_kv_heads=2, group=1, n_centers=40, fanout=(8, 8),
                                            kmeans_iters=1)
    keys, W = S.gen_keys(wl), S.gen_W(wl)
    desc = O.IndexDesc.of(wl)
    blob = O.index_blob(O.build_index(keys, W, desc))

    def fresh():
        return O.index_from_blob(blob.copy(), desc)

    idx = fresh()
    step = fixed_point_step(np.stack([hh.csr_latent for hh in idx.heads]), desc.n_keys)
    compared, skipped = check_lloyd_update(idx, desc, step)
    assert compared > 0.9 * (compared + skipped) and compared > 100

    # no update: the initial centroids stay
    idx0 = O.index_from_blob(O.index_blob(O.build_index(keys, W, O.IndexDesc.of(wl.scaled(kmeans_iters=0)))),
                             O.IndexDesc.of(wl.scaled(kmeans_iters=0)))
    bad = fresh()
    bad.heads[0].centroids[0] = idx0.heads[0].centroids[0].copy()
    with pytest.raises(AssertionError):
        check_lloyd_update(bad, desc, step)
    # a child moved to its neighbour's mean
    bad = fresh()
    c = bad.heads[1].centroids[1]
    c[[3, 4]] = c[[4, 3]]
    with pytest.raises(AssertionError):
        check_lloyd_update(bad, desc, step)
    # a nudge well beyond the fixed-point step and one fp32 ulp
    bad = fresh()
    bad.heads[0].centroids[1][10, 5] += 1e-3
    with pytest.raises(AssertionError):
        check_lloyd_update(bad, desc, step)


def test_fixed_point_step_rule():
    """The step follows |x| < 2^e and N <= 2^c: shift = 61 - c - e."""
    from tests.parity import fixed_point_step
    assert fixed_point_step(np.array([3.0]), 1 << 20) == 2.0 ** -(61 - 20 - 2)
    assert fixed_point_step(np.array([4.0]), (1 << 20) + 1) == 2.0 ** -(61 - 21 - 3)
    assert fixed_point_step(np.array([0.0]), 10) == 2.0 ** -100
    assert fixed_point_step(np.array([-1e30]), 10_000_000) == 2.0 ** -(61 - 24 - 100)


def test_one_head_readback_matches_the_full_blob():
    """The helper that reads one KV head of a device blob (used at 10M keys,
    where the whole blob is too large to decode) gives that head exactly as
    the reader of the full blob does; run here on a host tensor."""
    import types

    import torch

    from tests.gpu_helpers import one_head_index
    wl = S.get_workload("decode_1m").scaled(n_keys=1500, n_kv_heads=3, group=1, n_centers=20, fanout=(4, 8),
                                            kmeans_iters=2)
    keys, W = S.gen_keys(wl), S.gen_W(wl)
    desc = O.IndexDesc.of(wl)
    blob = O.index_blob(O.build_index(keys, W, desc))
    full = O.index_from_blob(blob, desc)
    li = types.SimpleNamespace(index=torch.from_numpy(blob))
    for h in range(3):
        one = one_head_index(li, desc, h).heads[0]
        ref = full.heads[h]
        assert np.array_equal(one.W, ref.W) and np.array_equal(one.perm, ref.perm)
        assert np.array_equal(one.csr_latent, ref.csr_latent)
        for lev in range(2):
            assert np.array_equal(one.centroids[lev], ref.centroids[lev])
            assert np.array_equal(one.cscore[lev], ref.cscore[lev])
            assert np.array_equal(one.offsets[lev], ref.offsets[lev])
            assert np.array_equal(one.assign[lev], ref.assign[lev])


def test_generator_later_keys_extend_the_cache():
    """Keys past the cache come from the same sequential streams: a longer
    cache's first N keys equal the cache, and its tail is gen_keys_range."""
    wl = S.get_workload("decode_10m").scaled(n_keys=(1 << 20) - 100, n_kv_heads=2, n_centers=64)
    base = S.gen_keys(wl)
    longer = S.gen_keys(wl.scaled(n_keys=(1 << 20) + 300))
    assert np.array_equal(longer[:wl.n_keys], base)
    assert np.array_equal(S.gen_keys_range(wl, wl.n_keys, wl.n_keys + 400), longer[wl.n_keys:])
    assert np.array_equal(S.gen_keys_range(wl, 1000, 1500), base[1000:1500])
