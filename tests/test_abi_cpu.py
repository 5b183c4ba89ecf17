"""The C ABI without a GPU: the library loads, exports every function that
include/lsa.h declares, its structs have the C layout, and invalid arguments
are rejected on the host (nothing is enqueued, so no device is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

from synth import get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")


@pytest.fixture(scope="module")
def A():
    from hierarchical_key_indexer_amd import _abi
    _abi.load()
    return _abi


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function(A):
    names = declared_functions()
    assert len(names) == 23
    lib = A.load()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(A.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} not exported as a text symbol"


def test_struct_layout_matches_c(A, tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(lsa_index_desc), offsetof(lsa_index_desc, fanout),
         offsetof(lsa_index_desc, kmeans_iters), offsetof(lsa_index_desc, seed), sizeof(lsa_select_params),
         offsetof(lsa_select_params, beam));
  return 0;
}}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", str(prog), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    D, S = A.IndexDesc, A.SelectParams
    assert got == [ctypes.sizeof(D), D.fanout.offset, D.kmeans_iters.offset, D.seed.offset, ctypes.sizeof(S),
                   S.beam.offset]


def test_sizes_match_the_blob_layout(A):
    from oracle import lsa_oracle as O
    for name in ("tiny_flat_65k", "decode_1m", "decode_10m"):
        wl = get_workload(name)
        assert A.index_bytes(A.IndexDesc.of(wl)) == O.blob_layout(O.IndexDesc.of(wl))["total"]
    p = A.SelectParams.make(16, 2048, 4, 512)
    assert A.select_out_width(p) == 2564


def _rc(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_validation_rejects_bad_descriptors(A):
    lib = A.load()
    wl = get_workload("decode_1m")
    good = A.IndexDesc.of(wl)
    assert A.index_bytes(good) > 0
    bad_cases = {
        "n_keys": dict(n_keys=0), "n_keys_big": dict(n_keys=1 << 31), "d_latent": dict(d_latent=48),
        "d_head": dict(d_head=100), "fanout": dict(fanout=(64, 1)), "levels": dict(fanout=(2,) * 5),
        "iters": dict(kmeans_iters=-1), "too_many_leaves": dict(fanout=(256, 256, 256)),
    }
    for name, kw in bad_cases.items():
        d = A.IndexDesc.of(wl.scaled(**kw)) if "fanout" not in kw or len(kw["fanout"]) <= 4 else None
        if d is None:
            d = A.IndexDesc.of(wl)
            d.n_levels = 5
        assert lib.lsa_index_bytes(ctypes.byref(d)) == 0, name
        assert A.last_error(), name
    assert lib.lsa_index_bytes(None) == 0


def test_validation_rejects_bad_calls_before_any_device_work(A):
    lib = A.load()
    wl = get_workload("decode_1m")
    d = A.IndexDesc.of(wl)
    p = A.SelectParams.make(16, 2048, 4, 512)
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    # build: NULL pointers, small buffers
    assert lib.lsa_build_index(ctypes.byref(d), None, fake, fake, 1 << 40, fake, 1 << 40, None) == A.LSA_ERR_INVALID_ARG
    assert lib.lsa_build_index(ctypes.byref(d), fake, fake, fake, 10, fake, 1 << 40, None) == A.LSA_ERR_BUFFER_TOO_SMALL
    assert lib.lsa_build_index(ctypes.byref(d), fake, fake, fake, 1 << 40, fake, 10, None) == A.LSA_ERR_BUFFER_TOO_SMALL
    # select: b > fanout, b^L too large, k too large, bad beam, bad head counts, small workspace
    cases = [
        (A.SelectParams.make(65, 2048, 4, 512), 1, 32, A.LSA_ERR_UNSUPPORTED),
        (A.SelectParams.make(16, 5000, 4, 512), 1, 32, A.LSA_ERR_UNSUPPORTED),
        (A.SelectParams.make(16, 0, 4, 512), 1, 32, A.LSA_ERR_UNSUPPORTED),
        (A.SelectParams.make(16, 2048, -1, 512), 1, 32, A.LSA_ERR_INVALID_ARG),
        (A.SelectParams(16, 2048, 4, 512, 7), 1, 32, A.LSA_ERR_INVALID_ARG),
        (p, 1, 30, A.LSA_ERR_INVALID_ARG),
        (p, -1, 32, A.LSA_ERR_INVALID_ARG),
    ]
    for prm, t, hq, code in cases:
        rc = lib.lsa_select(ctypes.byref(d), fake, fake, fake, t, hq, ctypes.byref(prm), fake, None, None, fake,
                            1 << 40, None)
        assert rc == code, (prm.b, prm.k, prm.beam, t, hq, rc, A.last_error())
    rc = lib.lsa_select(ctypes.byref(d), fake, fake, fake, 1, 32, ctypes.byref(p), fake, None, None, fake, 16, None)
    assert rc == A.LSA_ERR_BUFFER_TOO_SMALL
    rc = lib.lsa_select(ctypes.byref(d), None, fake, fake, 1, 32, ctypes.byref(p), fake, None, None, fake, 1 << 40, None)
    assert rc == A.LSA_ERR_INVALID_ARG
    # flat: G = 8 unsupported
    rc = lib.lsa_flat_select(ctypes.byref(d), fake, fake, fake, 1, 64, ctypes.byref(p), fake, None, fake, 1 << 40, None)
    assert rc == A.LSA_ERR_UNSUPPORTED and "query heads per KV head" in A.last_error()
    # global beam limit
    g = A.SelectParams.make(65, 2048, 4, 512, "global")
    assert A.load().lsa_select_workspace_bytes(ctypes.byref(d), ctypes.byref(g), 1, 32) == 0


def test_select_path_follows_the_batch_shape(A):
    """Decode batches take the per-query-head path, large bf16 batches the
    node-major path; fp32 latents, the global beam, wide fanouts and large k
    stay on the per-query-head path."""
    dec, pre = get_workload("decode_1m"), get_workload("prefill_1m")
    d = A.IndexDesc.of(dec)
    p = A.SelectParams.make(dec.b, dec.k, dec.sink, dec.window)
    assert A.select_path(d, p, 1, 32) == A.PATH_PER_QUERY_HEAD
    assert A.select_path(d, p, 4096, 32) == A.PATH_NODE_MAJOR
    assert A.select_path(d, p, 63, 32) == A.PATH_PER_QUERY_HEAD      # 252 query heads per KV head
    assert A.select_path(d, p, 64, 32) == A.PATH_NODE_MAJOR          # 256
    assert A.select_path(d, A.SelectParams.make(16, 2048, 4, 512, "global"), 4096, 32) == A.PATH_PER_QUERY_HEAD
    assert A.select_path(d, A.SelectParams.make(16, 4096, 4, 512), 4096, 32) == A.PATH_PER_QUERY_HEAD
    tiny = get_workload("tiny_flat_65k")
    dt = A.IndexDesc.of(tiny)
    assert A.select_path(dt, A.SelectParams.make(8, 256, 4, 128), 4096, 1) == A.PATH_PER_QUERY_HEAD
    assert A.select_path(A.IndexDesc.of(pre), A.SelectParams.make(16, 2048, 4, 512), 4096, 32) == A.PATH_NODE_MAJOR
    with pytest.raises(A.LsaError):
        A.select_path(d, p, 1, 7)


def test_flat_select_path_follows_the_batch_shape(A):
    """Full scans of large bf16 batches run on the matrix cores (row-tiled);
    decode batches, fp32 latents and k > 2048 keep the per-(token, KV head)
    streaming scan."""
    dec = get_workload("decode_1m")
    d = A.IndexDesc.of(dec)
    p = A.SelectParams.make(dec.b, dec.k, dec.sink, dec.window)
    assert A.flat_select_path(d, p, 1, 32) == A.PATH_PER_QUERY_HEAD
    assert A.flat_select_path(d, p, 63, 32) == A.PATH_PER_QUERY_HEAD     # 252 query heads per KV head
    assert A.flat_select_path(d, p, 64, 32) == A.PATH_ROW_TILED          # 256
    assert A.flat_select_path(d, p, 4096, 32) == A.PATH_ROW_TILED
    assert A.flat_select_path(d, A.SelectParams.make(16, 4096, 4, 512), 4096, 32) == A.PATH_PER_QUERY_HEAD
    tiny = get_workload("tiny_flat_65k")
    assert A.flat_select_path(A.IndexDesc.of(tiny), A.SelectParams.make(8, 256, 4, 128), 4096, 1) == \
        A.PATH_PER_QUERY_HEAD
    with pytest.raises(A.LsaError):
        A.flat_select_path(d, p, 1, 7)


def test_noalloc_select_refuses_batches_beyond_its_scratch(A):
    """A batch whose workspace exceeds the static scratch is refused before
    anything is enqueued (no GPU needed); decode batches of the 1M and 10M
    configurations fit."""
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    for name in ("decode_1m", "decode_10m"):
        wl = get_workload(name)
        d = A.IndexDesc.of(wl)
        p = A.SelectParams.make(wl.b, wl.k, wl.sink, wl.window)
        assert A.select_workspace_bytes(d, p, 1, wl.n_q_heads) <= A.NOALLOC_SCRATCH_BYTES
        need = A.select_workspace_bytes(d, p, 4096, wl.n_q_heads)
        assert need > A.NOALLOC_SCRATCH_BYTES
        rc = A.load().lsa_select_noalloc(ctypes.byref(d), fake, fake, fake, 4096, wl.n_q_heads, ctypes.byref(p),
                                         fake, None, None, None)
        assert rc == A.LSA_ERR_UNSUPPORTED and "static scratch" in A.last_error()
