"""GPU parity of the incremental index upkeep: keys appended after the build
(lsa_append_keys) and selection over the index plus the appended keys
(lsa_select_appended), through the C ABI, against the oracle's reading
(oracle.append_keys / select_one with ``appended``)."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _abi, _blob_of, _dev, _li, _params, gpu_build, gpu_select, one_head_index
from tests.parity import check_appended, compare_select, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi().load()


class Pool:
    """A device append pool and the keys appended to it so far."""

    def __init__(self, li, desc_o, cap):
        A = _abi()
        self.li, self.desc, self.cap, self.n = li, desc_o, cap, 0
        self.buf = torch.full((A.append_pool_bytes(li.desc, cap),), 0xF9, dtype=torch.uint8, device="cuda")

    def append(self, keys_new):
        _abi().lsa_append_keys(self.li.desc, self.li.index, _dev(keys_new), self.n, self.buf, self.cap)
        self.n += keys_new.shape[0]

    def read(self):
        """(leaf [Hkv][cap] int64, latent [Hkv][cap][dl] float64) of every slot."""
        d = self.desc
        b = self.buf.cpu().numpy()
        leaf = b[:d.n_kv_heads * self.cap * 4].view(np.int32).reshape(d.n_kv_heads, self.cap).astype(np.int64)
        off = (d.n_kv_heads * self.cap * 4 + 255) // 256 * 256
        cnt = d.n_kv_heads * self.cap * d.d_latent
        if d.latent_dtype == "bf16":
            lat = O.bf16_bits_to_f64(b[off:off + 2 * cnt].view(np.uint16))
        else:
            lat = b[off:off + 4 * cnt].view(np.float32).astype(np.float64)
        return leaf, lat.reshape(d.n_kv_heads, self.cap, d.d_latent)

    def appended(self):
        leaf, lat = self.read()
        return [O.Appended(latent=lat[h, :self.n], leaf=leaf[h, :self.n]) for h in range(self.desc.n_kv_heads)]

    def select(self, queries, pos, prm):
        A = _abi()
        T, Hq = queries.shape[0], queries.shape[1]
        p = _params(prm)
        ws = torch.empty(A.select_appended_workspace_bytes(self.li.desc, p, T, Hq), dtype=torch.uint8, device="cuda")
        idx = torch.empty((T, Hq, prm.sink + prm.k + prm.window), dtype=torch.int32, device="cuda")
        sc = torch.empty((T, Hq, prm.k), dtype=torch.float32, device="cuda")
        nl = prm.b if prm.beam == "global" else prm.b ** self.desc.n_levels
        lv = torch.empty((T, Hq, nl), dtype=torch.int32, device="cuda")
        A.lsa_select_appended(self.li.desc, self.li.index, self.buf, self.cap, self.n, _dev(queries),
                              torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda(), p, idx, sc, lv, ws)
        torch.cuda.synchronize()
        assert A.device_status(ws) == A.LSA_OK
        return idx.cpu().numpy(), sc.cpu().numpy(), lv.cpu().numpy()


def _cache(wl, extra):
    """The first N keys index; the next ``extra`` keys (same distribution,
    same generator stream) arrive later."""
    allk = gen_keys(wl.scaled(n_keys=wl.n_keys + extra))
    return allk[:wl.n_keys], allk[wl.n_keys:]


CASES = {
    "2lvl_bf16_g4": get_workload("decode_1m").scaled(n_keys=20000, n_kv_heads=2, group=4, n_centers=200,
                                                     kmeans_iters=3, fanout=(16, 16), b=4, k=128, sink=4,
                                                     window=64, n_tokens=5),
    "1lvl_f32_dl32": get_workload("tiny_flat_65k").scaled(n_keys=8000, n_centers=60, fanout=(64,), b=5, k=100,
                                                          window=32, n_tokens=5, kmeans_iters=3),
    "3lvl_global": get_workload("decode_1m").scaled(n_keys=30000, n_kv_heads=1, group=2, n_centers=300,
                                                    kmeans_iters=3, fanout=(4, 5, 6), b=3, k=64, sink=0,
                                                    window=16, n_tokens=4),
}


@pytest.mark.parametrize("case", list(CASES))
def test_append_then_select_matches_the_oracle(case):
    wl = CASES[case]
    log(f"[upkeep] case={case} N={wl.n_keys} fanout={wl.fanout}")
    keys, later = _cache(wl, 70)
    W = gen_W(wl)
    desc = O.IndexDesc.of(wl)
    oidx = O.build_index(keys, W, desc)
    li = _li(desc, O.index_blob(oidx))
    pool = Pool(li, desc, 100)
    for a, b in ((0, 5), (5, 6), (6, 70)):          # three calls, one of a single token (a decode step)
        pool.append(later[a:b])
    torch.cuda.synchronize()
    leaf, lat = pool.read()
    assert np.all(leaf[:, 70:] == np.int64(np.uint32(0xF9F9F9F9).astype(np.int32))), "slots past the last append"
    app = pool.appended()
    check_appended(oidx, later, W, desc, [x.leaf for x in app], [x.latent for x in app], log=log)
    N, n = wl.n_keys, pool.n
    queries = gen_queries(wl.scaled(n_tokens=6), keys)
    pos = np.array([N + n - 1, N + n - 2, N + 10, N, N - 1, 3000], dtype=np.int32)
    beams = ("per_parent", "global") if case != "3lvl_global" else ("global", "per_parent")
    for beam in beams:
        prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window, beam)
        gi, gs, gl = pool.select(queries, pos, prm)
        compare_select(oidx, queries, pos, prm, gi, gs, gl, log=log, appended=app)
    # with nothing appended, the same rows as lsa_select
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    empty = Pool(li, desc, 100)
    p0 = np.minimum(pos, N - 1)
    ei, es, el = empty.select(queries, p0, prm)
    ri, rs, rl = gpu_select(li, queries, p0, prm)
    assert np.array_equal(ei, ri) and np.array_equal(es.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(el, rl)


def test_appending_indexed_keys_reproduces_the_gpu_build():
    """Routing uses the build's own assignment arithmetic: a key appended with
    an indexed key's value reaches, bit for bit, the leaf the GPU build gave
    that key."""
    wl = CASES["2lvl_bf16_g4"]
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    li = gpu_build(desc, keys, W)
    gidx = O.index_from_blob(_blob_of(li), desc)
    pool = Pool(li, desc, 600)
    pick = np.random.default_rng(3).choice(wl.n_keys, 600, replace=False)
    pool.append(np.ascontiguousarray(keys[pick]))
    torch.cuda.synchronize()
    leaf, lat = pool.read()
    for h in range(desc.n_kv_heads):
        assert np.array_equal(leaf[h], gidx.heads[h].assign[-1][pick]), f"head {h}"
        want = np.empty_like(gidx.heads[h].csr_latent)
        want[gidx.heads[h].perm] = gidx.heads[h].csr_latent
        assert np.array_equal(lat[h], want[pick]), f"head {h}: latent differs from the build's"


def test_append_to_a_mismatched_index_marks_the_slots():
    wl = CASES["2lvl_bf16_g4"]
    keys, later = _cache(wl, 4)
    desc = O.IndexDesc.of(wl)
    li = _li(desc, O.index_blob(O.build_index(keys, gen_W(wl), desc)))
    li.index[0] = ord("X")
    pool = Pool(li, desc, 8)
    pool.append(later)
    torch.cuda.synchronize()
    leaf, _ = pool.read()
    assert np.all(leaf[:, :4] == -1)


@pytest.mark.timeout(600)
def test_decode_1m_with_appended_keys():
    """The 1M decode workload, index built on the GPU, then 512 decode steps'
    keys appended (in calls of 1 and of 255 and 256 tokens): rows of KV heads
    0 and 7 (query heads 0-3 and 28-31) against the oracle on those heads'
    read-back index with the GPU's appended keys."""
    wl = get_workload("decode_1m")
    log("[upkeep 1M] generating keys")
    keys, later = _cache(wl, 512)
    W = gen_W(wl)
    desc = O.IndexDesc.of(wl)
    li = gpu_build(desc, keys, W)
    li.release_build_workspace()
    pool = Pool(li, desc, 4096)
    pool.append(later[:1])
    pool.append(later[1:256])
    pool.append(later[256:])
    torch.cuda.synchronize()
    N, n = wl.n_keys, pool.n
    queries = gen_queries(wl.scaled(n_tokens=2), keys)
    pos = np.array([N + n - 1, N + 300], dtype=np.int32)
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    log("[upkeep 1M] GPU select with 512 appended keys")
    gi, gs, gl = pool.select(queries, pos, prm)
    app = pool.appended()
    g = wl.group
    for h in (0, 7):
        oh = one_head_index(li, desc, h)
        check_appended(oh, later[:, h:h + 1], W[h:h + 1], oh.desc, [app[h].leaf], [app[h].latent], log=log)
        sl = slice(h * g, (h + 1) * g)
        compare_select(oh, np.ascontiguousarray(queries[:, sl]), pos, prm, gi[:, sl], gs[:, sl], gl[:, sl], log=log,
                       appended=[app[h]])
