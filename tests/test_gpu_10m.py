"""GPU parity at 10M keys: one KV head (4 query heads) of the 10M-token cache
at its real shape (N = 10,000,000, 64 x 64 x 64 leaf buckets, 10 Lloyd
rounds, 10% outlier keys), against the oracle's own index of that head.
Decode is compared in full; the 8192-token prefill chunk on sampled query
heads; the GPU build by the properties of its final state."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _blob_of, _li, gpu_build, gpu_select
from tests.parity import check_build, compare_select, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def head10m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("decode_10m").scaled(n_kv_heads=1)
    log("[10m one head] generating 10M keys")
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    log("[10m one head] oracle index build (10 Lloyd rounds, 3 levels)")
    oidx = O.build_index(keys, W, desc, progress=log)
    log("[10m one head] oracle index ready")
    li = _li(desc, O.index_blob(oidx))
    return wl, keys, W, desc, oidx, li


@pytest.mark.timeout(900)
def test_decode_10m_one_head_tree_and_flat(head10m):
    wl, keys, W, desc, oidx, li = head10m
    queries, pos = gen_queries(wl, keys), gen_positions(wl)
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    log("[decode_10m one head] GPU tree select")
    gi, gs, gl = gpu_select(li, queries, pos, prm)
    compare_select(oidx, queries, pos, prm, gi, gs, gl, log=log)
    log("[decode_10m one head] GPU flat select")
    fi, fs, _ = gpu_select(li, queries, pos, prm, flat=True)
    compare_select(oidx, queries, pos, prm, fi, fs, flat=True, log=log)


@pytest.mark.timeout(900)
def test_prefill_10m_one_head_sampled(head10m):
    wl, keys, W, desc, oidx, li = head10m
    wl2 = get_workload("prefill_10m").scaled(n_kv_heads=1)
    queries, pos = gen_queries(wl2, keys), gen_positions(wl2)
    prm = O.SelectParams(wl2.b, wl2.k, wl2.sink, wl2.window)
    log("[prefill_10m one head] GPU tree select, 8192 tokens x 4 heads")
    gi, gs, gl = gpu_select(li, queries, pos, prm)
    rng = np.random.default_rng(9)
    pairs = [(int(t), int(h)) for t, h in zip(rng.integers(0, wl2.n_tokens, 48), rng.integers(0, 4, 48))]
    pairs += [(0, 0), (wl2.n_tokens - 1, 3)]
    compare_select(oidx, queries, pos, prm, gi, gs, gl, pairs=pairs, log=log)
    log("[prefill_10m one head] GPU full scan (row-tiled), 8192 tokens x 4 heads")
    fi, fs, _ = gpu_select(li, queries, pos, prm, flat=True)
    compare_select(oidx, queries, pos, prm, fi, fs, pairs=pairs[:24], flat=True, log=log)


@pytest.mark.timeout(900)
def test_decode_10m_one_head_gpu_build(head10m):
    wl, keys, W, desc, oidx, li = head10m
    log("[10m one head] GPU build")
    lb = gpu_build(desc, keys, W)
    blob = _blob_of(lb)
    gidx = O.index_from_blob(blob, desc)
    check_build(gidx, keys, W, desc, sample=20000, log=log)
    agree = np.mean(gidx.heads[0].assign[0] == oidx.heads[0].assign[0])
    log(f"[10m one head] level-1 agreement with the oracle build {agree:.5f}")
