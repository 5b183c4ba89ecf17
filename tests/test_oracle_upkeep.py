"""Pins of the oracle's incremental index upkeep (keys appended after the
build, at positions N, N + 1, ...): the routing rule against the build's own
assignment and against a pure-Python brute force, and selection with
appended keys against its definition (the index with every appended key
placed in its leaf), checked by exhaustive brute force on tiny trees."""
import itertools

import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import workloads as S
from tests.test_oracle import _brute_select, _build, _int_index, _small_wl


def _brute_route(hh, fanout, x):
    """Pure-Python routing: at every level the non-empty child with the
    smallest squared distance, the lowest id on a tie."""
    node = 0
    for lev, f in enumerate(fanout):
        best = None
        for c in range(f):
            kid = node * f + c
            if hh.offsets[lev][kid + 1] == hh.offsets[lev][kid]:
                continue
            d = sum((float(a) - float(b)) ** 2 for a, b in zip(x, hh.centroids[lev][kid]))
            if best is None or d < best[0]:
                best = (d, kid)
        node = best[1]
    return node


@pytest.mark.parametrize("fanout", [(16,), (4, 4), (4, 3, 5)])
def test_routing_existing_keys_reproduces_the_build(fanout):
    """A key appended with the latent of an indexed key reaches the leaf the
    build's final assignment gave that key: its assigned child is nearest
    among the initialised children, holds the key, so is nearest among the
    non-empty ones too."""
    wl = _small_wl(fanout, n=900, iters=3)
    keys, W, idx = _build(wl)
    app = O.append_keys(idx, keys)
    for h, hh in enumerate(idx.heads):
        assert np.array_equal(app[h].leaf, hh.assign[-1]), f"head {h}"


@pytest.mark.parametrize("fanout", [(16,), (4, 4), (8, 8)])
def test_routing_matches_brute_force_with_ties(fanout):
    idx, rng = _int_index(fanout, 300, 5, seed=3 + sum(fanout))
    hh = idx.heads[0]
    for _ in range(200):
        x = rng.integers(-3, 4, 5).astype(np.float64)
        assert O.route_key(hh, fanout, x) == _brute_route(hh, fanout, x)


def _appended_int(idx, rng, a, dl):
    hh = idx.heads[0]
    lat = rng.integers(-2, 3, (a, dl)).astype(np.float64)
    leaf = np.array([O.route_key(hh, idx.desc.fanout, x) for x in lat], dtype=np.int64)
    return [O.Appended(latent=lat, leaf=leaf)]


@pytest.mark.parametrize("fanout", [(16,), (4, 4), (8, 8)])
def test_select_with_appended_keys_brute_force(fanout):
    """Exhaustive over b, k, sink, window and positions (before, among and
    after the appended keys): selection with the appended pool equals the
    pure-Python brute force on the index the definition builds."""
    n, a, dl = 300, 60, 6
    idx, rng = _int_index(fanout, n, dl, seed=7 * sum(fanout))
    app = _appended_int(idx, rng, a, dl)
    full = O.index_with_appended(idx, app)
    assert full.desc.n_keys == n + a
    ps = sorted(set([0, 5, 17, 40, 200, n - 1, n, n + 1, n + 16, n + 17, n + a - 1] +
                    rng.integers(0, n + a, 6).tolist()))
    for qlat in [rng.integers(-2, 3, dl).astype(np.float64) for _ in range(3)]:
        for b in range(1, fanout[0] + 1):
            for k, sink, window in itertools.product((1, 7, 64), (0, 4), (0, 16)):
                prm = O.SelectParams(b=b, k=k, sink=sink, window=window)
                for p in ps:
                    res = O.select_one(idx, 0, qlat, p, prm, appended=app[0])
                    leaves, top = _brute_select(full.heads[0], fanout, qlat, p, prm)
                    assert sorted(res["leaves"].tolist()) == leaves
                    assert res["top_idx"].tolist() == top, (b, k, sink, window, p)
                    ref = O.select_one(full, 0, qlat, p, prm)
                    assert np.array_equal(res["top_idx"], ref["top_idx"])
                    assert np.array_equal(res["top_scores"], ref["top_scores"])


@pytest.mark.parametrize("fanout,b", [((16,), 16), ((4, 4), 4), ((4, 3, 5), 5)])
def test_appended_tree_with_all_buckets_equals_flat(fanout, b):
    wl = _small_wl(fanout, n=700, k=33, b=b, t=6)
    keys, W, idx = _build(wl)
    more = S.gen_keys(wl.scaled(cache_id=wl.cache_id + 50, n_keys=80))
    app = O.append_keys(idx, more[:50])
    app = O.append_keys(idx, more[50:], prev=app)          # two calls: the pool grows in order
    assert all(len(x.leaf) == 80 for x in app)
    q = S.gen_queries(wl, keys)
    pos = np.array([700 + 79, 700 + 40, 700, 699, 300, 20], dtype=np.int32)
    prm = O.SelectParams(b, wl.k, wl.sink, wl.window)
    tr, ts, _, _ = O.select(idx, q, pos, prm, appended=app)
    fr, fs, _, _ = O.flat_select(idx, q, pos, prm, appended=app)
    for key in tr:
        assert np.array_equal(tr[key], fr[key]) and np.array_equal(ts[key], fs[key])
    # and the same rows as the index the definition builds
    full = O.index_with_appended(idx, app)
    dr, ds, _, _ = O.select(full, q, pos, prm)
    for key in tr:
        assert np.array_equal(tr[key], dr[key]) and np.array_equal(ts[key], ds[key])


def test_appended_keys_inside_the_window_are_not_candidates():
    wl = _small_wl((4, 4), n=400, k=500, b=4, t=1, sink=2, window=10)
    keys, W, idx = _build(wl)
    more = S.gen_keys(wl.scaled(cache_id=wl.cache_id + 60, n_keys=30))
    app = O.append_keys(idx, more)
    prm = O.SelectParams(4, 500, 2, 10)
    q = S.gen_queries(wl, keys)
    p = 400 + 29
    res = O.select_one(idx, 0, O.query_latent(q[0, 0], idx.heads[0], "bf16", "bf16"), p, prm, flat=True,
                       appended=app[0])
    assert set(res["top_idx"].tolist()) == set(range(2, p - 10 + 1))      # every candidate, none in the window
