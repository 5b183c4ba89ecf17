"""lsa_select and lsa_flat_select inside a captured graph.

Every entry point only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation), so a call can be captured and
replayed.  Each case captures one call, then replays it three times with
eager work between the replays (the outputs are overwritten), and checks
every replay bit for bit against the eager call: the per-query-head path
(decode), the node-major path and the row-tiled full scan (prefill-sized
batches)."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _abi, _dev, _li, _params
from tests.parity import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hierarchical_key_indexer_amd import _abi as A
    A.load()


DECODE = get_workload("decode_1m").scaled(n_keys=20000, n_kv_heads=2, group=4, n_centers=200, n_tokens=1,
                                          kmeans_iters=4, fanout=(16, 16), b=4, k=64, window=32)
PREFILL = get_workload("prefill_1m").scaled(n_keys=20000, n_kv_heads=2, group=4, n_centers=200, n_tokens=64,
                                            kmeans_iters=4, fanout=(16, 16), b=4, k=64, window=32)
CASES = {"decode_tree": (DECODE, False), "prefill_tree": (PREFILL, False), "prefill_full_scan": (PREFILL, True)}


@pytest.mark.parametrize("case", list(CASES))
def test_call_replays_in_a_graph(case):
    wl, flat = CASES[case]
    A = _abi()
    log(f"[graph] case={case} N={wl.n_keys} T={wl.n_tokens} Hq={wl.n_q_heads}")
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    li = _li(desc, O.index_blob(O.build_index(keys, W, desc)))
    q = _dev(gen_queries(wl, keys))
    pos = gen_positions(wl)
    p = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda()
    prm = _params(O.SelectParams(wl.b, wl.k, wl.sink, wl.window))
    if flat:
        assert A.flat_select_path(li.desc, prm, wl.n_tokens, wl.n_q_heads) == A.PATH_ROW_TILED
    else:
        want = A.PATH_NODE_MAJOR if wl.n_tokens > 1 else A.PATH_PER_QUERY_HEAD
        assert A.select_path(li.desc, prm, wl.n_tokens, wl.n_q_heads) == want

    def call(out):
        if flat:
            li.flat_select(q, p, prm, out=out)
        else:
            li.select(q, p, prm, out=out)

    eager = li.alloc_select_outputs(wl.n_tokens, wl.n_q_heads, prm, scores=True, flat=flat)
    call(eager)                                     # also sizes the cached workspace
    torch.cuda.synchronize()
    want_idx, want_sc = eager[0].cpu().numpy(), eager[1].cpu().numpy()
    assert (want_idx >= 0).any()

    out = li.alloc_select_outputs(wl.n_tokens, wl.n_q_heads, prm, scores=True, flat=flat)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    for rep in range(3):
        out[0].fill_(-7)
        out[1].fill_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out[0].cpu().numpy(), want_idx), f"replay {rep}: indices"
        assert np.array_equal(out[1].cpu().numpy().view(np.uint32), want_sc.view(np.uint32)), f"replay {rep}: scores"
