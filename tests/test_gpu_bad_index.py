"""A select call whose descriptor does not match the blob it is handed must
not read past the blob's header: the first kernel compares the header with
what the descriptor implies, leaves LSA_ERR_BAD_INDEX in the workspace's
status word, and every output row comes back all -1 (scores -inf, leaves -1).
Each mismatch here keeps every read the descriptor could imply inside the
buffer, so a missing check would show as wrong rows, never as a fault.  All
four select paths are covered; a valid call on the same workspace afterwards
reports LSA_OK and matches the oracle."""
import dataclasses

import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _abi, _dev, _li, _params
from tests.parity import compare_select, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("prefill_1m").scaled(n_keys=20000, n_kv_heads=2, group=4, n_centers=200, n_tokens=64,
                                           kmeans_iters=3, fanout=(16, 16), b=4, k=64, sink=4, window=32)
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    oidx = O.build_index(keys, W, desc)
    blob = O.index_blob(oidx)
    queries = gen_queries(wl, keys)
    pos = gen_positions(wl)
    return wl, desc, oidx, blob, queries, pos


def _desc(d: O.IndexDesc):
    A = _abi()
    return A.IndexDesc.make(d.n_keys, d.n_kv_heads, d.d_head, d.d_latent, d.key_dtype, d.latent_dtype, d.fanout,
                            d.kmeans_iters, d.seed)


def _call(desc_o, blob_t, queries, pos, prm, flat):
    """One select call through the C ABI on a fresh workspace filled with
    0xA5 bytes; returns (status word, rows, scores, leaves)."""
    A = _abi()
    d = _desc(desc_o)
    p = _params(prm)
    T, Hq = queries.shape[0], queries.shape[1]
    nbytes = (A.flat_workspace_bytes if flat else A.select_workspace_bytes)(d, p, T, Hq)
    ws = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    qd = _dev(queries)
    pd = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda()
    width = prm.sink + prm.k + prm.window
    idx = torch.zeros((T, Hq, width), dtype=torch.int32, device="cuda")
    sc = torch.zeros((T, Hq, prm.k), dtype=torch.float32, device="cuda")
    lv = None
    if flat:
        A.lsa_flat_select(d, blob_t, qd, pd, p, idx, sc, ws)
    else:
        lv = torch.zeros((T, Hq, prm.b ** desc_o.n_levels), dtype=torch.int32, device="cuda")
        A.lsa_select(d, blob_t, qd, pd, p, idx, sc, lv, ws)
    torch.cuda.synchronize()
    return (A.device_status(ws), idx.cpu().numpy(), sc.cpu().numpy(),
            None if lv is None else lv.cpu().numpy())


PATHS = {  # (tokens, flat): decode-sized batches take the per-query-head kernels,
    "tree_per_query_head": (3, False),   # 256+ query heads per KV head the matrix-core ones
    "flat_per_query_head": (3, True),
    "tree_node_major": (64, False),
    "flat_row_tiled": (64, True),
}


@pytest.mark.parametrize("path", list(PATHS))
def test_mismatched_index_is_refused_on_the_device(small, path):
    wl, desc, oidx, blob, queries, pos = small
    T, flat = PATHS[path]
    # positions below every n_keys used here, so no row is invalid for its position alone
    q, p = queries[-T:], pos[-T:] - 200
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    A = _abi()
    want_path = A.PATH_ROW_TILED if flat else (A.PATH_NODE_MAJOR if T == 64 else A.PATH_PER_QUERY_HEAD)
    got_path = (A.flat_select_path if flat else A.select_path)(_desc(desc), _params(prm), T, wl.n_q_heads)
    if T == 64:
        assert got_path == want_path, f"{path}: the batch takes path {got_path}"
    else:
        assert got_path == A.PATH_PER_QUERY_HEAD
    good = torch.from_numpy(blob).cuda()
    magic = good.clone()
    magic[0] = ord("X")
    flagged = good.clone()
    flagged[60] = 1                                  # build status word: a non-finite latent
    fewer = dataclasses.replace(desc, n_keys=desc.n_keys - 100)   # a smaller blob: reads stay inside
    cases = {"descriptor n_keys": (fewer, good), "magic": (desc, magic), "build status": (desc, flagged)}
    for what, (dsc, bt) in cases.items():
        log(f"[bad index] {path}: mismatched {what}")
        st, idx, sc, lv = _call(dsc, bt, q, p, prm, flat)
        assert st == A.LSA_ERR_BAD_INDEX, f"{path}, {what}: status {st}"
        assert np.all(idx == -1), f"{path}, {what}: rows not all -1"
        assert np.all(np.isneginf(sc)), f"{path}, {what}: scores not -inf"
        if lv is not None:
            assert np.all(lv == -1), f"{path}, {what}: leaves not -1"
    st, idx, sc, lv = _call(desc, good, q, p, prm, flat)
    assert st == A.LSA_OK
    compare_select(oidx, q, p, prm, idx, sc, lv, flat=flat, log=log)


def test_build_of_non_finite_keys_marks_the_index_bad():
    """A key whose latent is not finite: the build sets the header's status
    word, and select refuses the index."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("decode_1m").scaled(n_keys=3000, n_kv_heads=2, group=2, n_centers=30, fanout=(8, 8),
                                          kmeans_iters=2, b=3, k=50, sink=4, window=32, n_tokens=2)
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    li = _li(desc)
    li.build(_dev(keys), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    assert int(li.index[60:64].view(torch.int32).item()) == 0
    bad = keys.copy()
    bad[1234, 1, 7] = 0x7F80                         # +inf in bf16
    li.build(_dev(bad), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    assert int(li.index[60:64].view(torch.int32).item()) == 1
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    st, idx, _, _ = _call(desc, li.index, gen_queries(wl, keys), gen_positions(wl), prm, False)
    assert st == _abi().LSA_ERR_BAD_INDEX and np.all(idx == -1)
