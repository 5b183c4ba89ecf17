"""GPU parity on the full 10M-key cache: all 8 KV heads (32 query heads),
N = 10,000,000, 64 x 64 x 64 leaf buckets, 10 Lloyd rounds, 10% outlier
keys, built on the GPU.  KV heads 4-7 lie past 2^32 latent elements of the
blob, so these rows exercise the 64-bit section offsets.

The index is the GPU's own build.  Each compared KV head is read back from
the device on its own and checked two ways: its build by the properties its
final state must have (latent within 1 ulp, nearest centroids, stable nested
CSR; a 20,000-key sample), and its select rows against the oracle's select
run on that head's index (descent, key stage, rows)."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from synth import gen_keys, gen_positions, gen_queries, gen_W, get_workload
from tests.gpu_helpers import _dev, _li, gpu_select, one_head_index
from tests.parity import check_build, compare_select, log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def full10m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("decode_10m")
    log("[10m, 8 KV heads] generating 10M keys x 8 heads")
    keys, W = gen_keys(wl), gen_W(wl)
    desc = O.IndexDesc.of(wl)
    log("[10m, 8 KV heads] GPU build")
    li = _li(desc)
    kd = _dev(keys)
    li.build(kd, torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    li.release_build_workspace()
    del kd
    torch.cuda.empty_cache()
    log("[10m, 8 KV heads] index built")
    heads = {}

    def head(h):
        if h not in heads:
            heads.clear()
            log(f"[10m, 8 KV heads] reading back KV head {h}")
            heads[h] = one_head_index(li, desc, h)
        return heads[h]

    return wl, keys, W, desc, li, head


def _one_head_queries(queries, h, g):
    return np.ascontiguousarray(queries[:, h * g:(h + 1) * g])


@pytest.mark.timeout(900)
def test_decode_10m_8_heads_build_and_rows(full10m):
    wl, keys, W, desc, li, head = full10m
    queries, pos = gen_queries(wl, keys), gen_positions(wl)
    prm = O.SelectParams(wl.b, wl.k, wl.sink, wl.window)
    log("[decode_10m, 8 KV heads] GPU tree and flat select, 32 query heads")
    gi, gs, gl = gpu_select(li, queries, pos, prm)
    fi, fs, _ = gpu_select(li, queries, pos, prm, flat=True)
    g = wl.group
    for h in (7, 0):
        oh = head(h)
        log(f"[decode_10m, 8 KV heads] KV head {h}: build properties on 20,000 keys")
        check_build(oh, keys[:, h:h + 1, :], W[h:h + 1], oh.desc, sample=20000, log=log)
        q1 = _one_head_queries(queries, h, g)
        sl = slice(h * g, (h + 1) * g)
        log(f"[decode_10m, 8 KV heads] KV head {h}: tree rows of query heads {h * g}-{h * g + g - 1}")
        compare_select(oh, q1, pos, prm, gi[:, sl], gs[:, sl], gl[:, sl], log=log)
        log(f"[decode_10m, 8 KV heads] KV head {h}: flat rows")
        compare_select(oh, q1, pos, prm, fi[:, sl], fs[:, sl], flat=True, log=log)


@pytest.mark.timeout(900)
def test_prefill_10m_8_heads_sampled_rows(full10m):
    wl, keys, W, desc, li, head = full10m
    wl2 = get_workload("prefill_10m")
    queries, pos = gen_queries(wl2, keys), gen_positions(wl2)
    prm = O.SelectParams(wl2.b, wl2.k, wl2.sink, wl2.window)
    log("[prefill_10m, 8 KV heads] GPU tree select, 8192 tokens x 32 query heads")
    gi, gs, gl = gpu_select(li, queries, pos, prm)
    log("[prefill_10m, 8 KV heads] GPU full scan (row-tiled), 8192 tokens x 32 query heads")
    fi, fs, _ = gpu_select(li, queries, pos, prm, flat=True)
    g, T = wl2.group, wl2.n_tokens
    rng = np.random.default_rng(77)
    total = 0
    for h in (4, 5, 6, 7):
        oh = head(h)
        q1 = _one_head_queries(queries, h, g)
        sl = slice(h * g, (h + 1) * g)
        # every query head of a few tokens (first, last, two at random), and
        # scattered rows
        toks = [0, T - 1] + [int(t) for t in rng.integers(1, T - 1, 2)]
        pairs = [(t, j) for t in toks for j in range(g)]
        pairs += [(int(t), int(j)) for t, j in zip(rng.integers(0, T, 6), rng.integers(0, g, 6))]
        log(f"[prefill_10m, 8 KV heads] KV head {h}: {len(pairs)} tree rows")
        compare_select(oh, q1, pos, prm, gi[:, sl], gs[:, sl], gl[:, sl], pairs=pairs, log=log)
        total += len(pairs)
        fpairs = [(0, 0), (T - 1, g - 1), (int(rng.integers(0, T)), int(rng.integers(0, g)))]
        log(f"[prefill_10m, 8 KV heads] KV head {h}: {len(fpairs)} full-scan rows")
        compare_select(oh, q1, pos, prm, fi[:, sl], fs[:, sl], pairs=fpairs, flat=True, log=log)
    assert total >= 50
