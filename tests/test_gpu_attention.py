"""lsa_sparse_attention on the GPU against the oracle's exact sparse attention.

Tolerance, from the fp32 arithmetic: a score is a dot of d fp32 products, off
by at most ds = (d + 2) u scale sum_i |q_i k_i| (u = 2^-24); the weights
exp(s_j - max) are then off by a relative 2 ds + 4u, and the normalised sum by
at most (4 max ds + (width + 32) u) sum_j w_j |v_j| per dim (w the oracle's
weights; the (width + 32) u term covers the fp32 sums of p_j v_j and, for a
row split over workgroups, the rescaling of its parts).
The test allows twice that, entry by entry."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from tests.parity import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_key_indexer_amd import _abi as A
    A.load()


def _store(x, dtype):
    if dtype == "bf16":
        return O.f64_to_bf16_bits(O.round_bf16(x))
    return x.astype(np.float32)


def _dev(a):
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _bound(q, k, v, idx, scale, G):
    u = 2.0 ** -24
    T, Hq, d = q.shape
    width = idx.shape[2]
    out = np.zeros((T, Hq, d))
    for t in range(T):
        for hq in range(Hq):
            h = hq // G
            r = idx[t, hq]
            sel = r[(r >= 0) & (r < k.shape[0])]
            if sel.size == 0:
                continue
            s = scale * (k[sel, h] @ q[t, hq])
            w = np.exp(s - s.max())
            w /= w.sum()
            ds = (d + 2) * u * abs(scale) * (np.abs(k[sel, h]) @ np.abs(q[t, hq])).max()
            out[t, hq] = (4 * ds + (width + 32) * u) * (w @ np.abs(v[sel, h]))
    return out


CASES = [  # N, T, Hkv, G, d, width, dtype
    (5_000, 3, 2, 4, 128, 300, "bf16"),
    (2_000, 2, 1, 2, 64, 257, "f32"),
    (3_000, 1, 2, 1, 256, 1_000, "bf16"),
    (3_000, 2, 1, 1, 256, 40, "f32"),
    (100, 4, 1, 4, 128, 1, "bf16"),
    (200_000, 1, 8, 4, 128, 2_564, "bf16"),     # a 1M-decode row shape: sink 4 + k 2048 + window 512
    (20_000, 32, 8, 4, 128, 700, "bf16"),       # 1024 rows: one workgroup per row, no split
]


@pytest.mark.parametrize("N,T,Hkv,G,d,width,dtype", CASES)
def test_attention_matches_oracle(N, T, Hkv, G, d, width, dtype):
    from hierarchical_key_indexer_amd import _abi as A
    log(f"[attention] N={N} T={T} Hkv={Hkv} G={G} d={d} width={width} {dtype}")
    rng = np.random.default_rng(N + width)
    Hq = Hkv * G
    keys = _store(rng.standard_normal((N, Hkv, d)), dtype)
    vals = _store(rng.standard_normal((N, Hkv, d)), dtype)
    qs = _store(rng.standard_normal((T, Hq, d)), dtype)
    idx = rng.integers(0, N, size=(T, Hq, width)).astype(np.int32)
    # padding, out-of-range entries, duplicates and an empty row
    idx[:, :, ::7] = -1
    if width > 3:
        idx[0, 0, 1] = N + 5
        idx[0, 0, 2] = idx[0, 0, 3]
    if T > 1:
        idx[1, Hq - 1, :] = -1
    scale = 1.0 / np.sqrt(d)
    desc = A.IndexDesc.make(N, Hkv, d, 32, dtype, dtype, (4,), 1, 0)
    out = torch.empty((T, Hq, d), dtype=torch.float32, device="cuda")
    A.lsa_sparse_attention(desc, _dev(qs), _dev(keys), _dev(vals), _dev(idx), scale, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = O.sparse_attention(qs, keys, vals, idx, dtype, scale)
    bound = 2 * _bound(O.stored_to_f64(qs, dtype), O.stored_to_f64(keys, dtype), O.stored_to_f64(vals, dtype),
                       idx, scale, G)
    err = np.abs(got - want)
    assert np.all(err <= bound + 1e-30), f"worst ratio {np.max(err / (bound + 1e-30)):.3g}"
    if T > 1:
        assert np.all(got[1, Hq - 1] == 0.0)


def test_attention_validation():
    from hierarchical_key_indexer_amd import _abi as A
    lib = A.load()
    desc = A.IndexDesc.make(100, 1, 128, 32, "bf16", "bf16", (4,), 1, 0)
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    assert lib.lsa_sparse_attention(desc, p, p, p, p, 0, 1, 1, 1.0, p, p, 1 << 16, None) == A.LSA_ERR_UNSUPPORTED
    assert lib.lsa_sparse_attention(desc, p, p, p, p, 40000, 1, 1, 1.0, p, p, 1 << 16, None) == \
        A.LSA_ERR_UNSUPPORTED
    assert lib.lsa_sparse_attention(desc, None, p, p, p, 4, 1, 1, 1.0, p, p, 1 << 16, None) == A.LSA_ERR_INVALID_ARG
    assert lib.lsa_sparse_attention(desc, p, p, p, p, 4, 1, 1, float("nan"), p, p, 1 << 16, None) == \
        A.LSA_ERR_INVALID_ARG
    # a split row needs its workspace
    assert A.sparse_attention_workspace_bytes(desc, 2564, 1, 1) > 0
    assert lib.lsa_sparse_attention(desc, p, p, p, p, 2564, 1, 1, 1.0, p, p, 16, None) == A.LSA_ERR_BUFFER_TOO_SMALL
    # query heads not a multiple of the KV heads
    desc2 = A.IndexDesc.make(100, 2, 128, 32, "bf16", "bf16", (4,), 1, 0)
    assert lib.lsa_sparse_attention(desc2, p, p, p, p, 4, 1, 3, 1.0, p, p, 1 << 16, None) == A.LSA_ERR_INVALID_ARG


@pytest.mark.parametrize("tokens", [1, 48])
def test_attention_over_select_rows(tokens):
    # the two entry points chained as a caller would: lsa_select's rows feed
    # lsa_sparse_attention; the oracle attends over the same rows
    from hierarchical_key_indexer_amd import _abi as A
    from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
    from tests.gpu_helpers import _dev as dev_keys, _li, _params
    wl = get_workload("decode_1m").scaled(n_keys=30000, n_kv_heads=2, group=4, n_centers=300, n_tokens=tokens,
                                          kmeans_iters=3, fanout=(16, 16), b=4, k=256, window=64)
    log(f"[attention] select rows: N={wl.n_keys} T={tokens}")
    keys, W = gen_keys(wl), gen_W(wl)
    desc_o = O.IndexDesc.of(wl)
    li = _li(desc_o, O.index_blob(O.build_index(keys, W, desc_o)))
    queries, pos = gen_queries(wl, keys), gen_positions(wl)
    qd = dev_keys(queries)
    pd = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda()
    prm = _params(O.SelectParams(wl.b, wl.k, wl.sink, wl.window))
    idx, _, _ = li.select(qd, pd, prm, scores=False)
    rng = np.random.default_rng(11)
    vals = _store(rng.standard_normal(keys.shape), "bf16")
    out = torch.empty((tokens, wl.n_q_heads, wl.d_head), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(wl.d_head)
    A.lsa_sparse_attention(li.desc, qd, dev_keys(keys), _dev(vals), idx, scale, out)
    torch.cuda.synchronize()
    rows = idx.cpu().numpy()
    assert (rows >= 0).any()
    got = out.cpu().numpy().astype(np.float64)
    want = O.sparse_attention(queries, keys, vals, rows, "bf16", scale)
    bound = 2 * _bound(O.stored_to_f64(queries, "bf16"), O.stored_to_f64(keys, "bf16"),
                       O.stored_to_f64(vals, "bf16"), rows, scale, wl.group)
    err = np.abs(got - want)
    assert np.all(err <= bound + 1e-30), f"worst ratio {np.max(err / (bound + 1e-30)):.3g}"
