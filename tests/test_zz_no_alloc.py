"""lsa_select_noalloc (the library's static device scratch, no workspace
argument) against lsa_select (caller workspace) through the C ABI: two calls
in a row on one GPU, the second with a smaller batch, each bit for bit equal
to lsa_select's rows, scores and leaves, and lsa_select itself checked
against the oracle."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _abi, _dev, _li, _params
from tests.parity import compare_select, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _outs(T, Hq, prm, nl):
    width = prm.sink + prm.k + prm.window
    return (torch.full((T, Hq, width), -7, dtype=torch.int32, device="cuda"),
            torch.zeros((T, Hq, prm.k), dtype=torch.float32, device="cuda"),
            torch.full((T, Hq, nl), -7, dtype=torch.int32, device="cuda"))


def test_noalloc_select_equals_select_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    A = _abi()
    A.load()
    wl = get_workload("decode_1m").scaled(n_keys=30000, n_kv_heads=2, group=4, n_centers=300, fanout=(16, 16),
                                          kmeans_iters=3, b=4, k=128, sink=4, window=64, n_tokens=6)
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    oidx = O.build_index(keys, W, desc)
    li = _li(desc, O.index_blob(oidx))
    queries, pos = gen_queries(wl, keys), gen_positions(wl)
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    p = _params(prm)
    nl = prm.b ** desc.n_levels
    for T in (6, 2):                                 # the second call is smaller
        q, ps = queries[:T], pos[:T]
        qd = _dev(q)
        pd = torch.from_numpy(np.ascontiguousarray(ps, dtype=np.int32)).cuda()
        log(f"[no-alloc] {T} tokens x {wl.n_q_heads} query heads")
        ref = _outs(T, wl.n_q_heads, prm, nl)
        ws = torch.empty(A.select_workspace_bytes(li.desc, p, T, wl.n_q_heads), dtype=torch.uint8, device="cuda")
        A.lsa_select(li.desc, li.index, qd, pd, p, *ref, ws)
        got = _outs(T, wl.n_q_heads, prm, nl)
        A.lsa_select_noalloc(li.desc, li.index, qd, pd, p, *got)
        torch.cuda.synchronize()
        ri, rs, rl = (x.cpu().numpy() for x in ref)
        gi, gs, gl = (x.cpu().numpy() for x in got)
        compare_select(oidx, q, ps, prm, ri, rs, rl, log=log)
        assert np.array_equal(gi, ri), f"T={T}: rows differ"
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), f"T={T}: scores differ"
        assert np.array_equal(gl, rl), f"T={T}: leaves differ"
