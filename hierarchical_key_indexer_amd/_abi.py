"""ctypes binding of the LSA indexer's C ABI (include/lsa.h).

Argument marshalling only: every step of the indexer runs in the HIP kernels
of ``liblsa.so``.  PyTorch supplies device memory and streams.  If the shared
library is missing, loading raises at once; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LSA_LIBRARY", os.path.join(HERE, "liblsa.so"))

LSA_OK, LSA_ERR_INVALID_ARG, LSA_ERR_UNSUPPORTED, LSA_ERR_BUFFER_TOO_SMALL, LSA_ERR_BAD_INDEX, LSA_ERR_HIP = range(6)
LSA_F32, LSA_BF16 = 0, 1
LSA_BEAM_PER_PARENT, LSA_BEAM_GLOBAL = 0, 1
DTYPES = {"f32": LSA_F32, "bf16": LSA_BF16}
BEAMS = {"per_parent": LSA_BEAM_PER_PARENT, "global": LSA_BEAM_GLOBAL}

EXPORTS = ("lsa_index_bytes", "lsa_build_workspace_bytes", "lsa_build_index", "lsa_select_out_width",
           "lsa_select_workspace_bytes", "lsa_select_path", "lsa_select", "lsa_flat_workspace_bytes",
           "lsa_flat_select_path", "lsa_flat_select", "lsa_last_error", "lsa_abi_version",
           "lsa_set_profile_events", "lsa_pca_workspace_bytes", "lsa_pca_covariance", "lsa_pca_map",
           "lsa_sparse_attention_workspace_bytes", "lsa_sparse_attention", "lsa_select_noalloc",
           "lsa_append_pool_bytes", "lsa_append_keys", "lsa_select_appended_workspace_bytes",
           "lsa_select_appended")
NOALLOC_SCRATCH_BYTES = 32 << 20
STAGE_PROJECT, STAGE_DESCEND, STAGE_GATHER, STAGE_MERGE, STAGE_FLAT, STAGE_SAMPLE = 1, 2, 3, 4, 5, 6
PATH_PER_QUERY_HEAD, PATH_NODE_MAJOR, PATH_ROW_TILED = 0, 1, 2


class IndexDesc(ctypes.Structure):
    _fields_ = [("n_keys", ctypes.c_int64), ("n_kv_heads", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("key_dtype", ctypes.c_int32), ("latent_dtype", ctypes.c_int32),
                ("n_levels", ctypes.c_int32), ("fanout", ctypes.c_int32 * 4), ("kmeans_iters", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]

    @staticmethod
    def make(n_keys, n_kv_heads, d_head, d_latent, key_dtype, latent_dtype, fanout, kmeans_iters, seed):
        f = list(fanout) + [0] * (4 - len(fanout))
        return IndexDesc(n_keys, n_kv_heads, d_head, d_latent, DTYPES.get(key_dtype, key_dtype),
                         DTYPES.get(latent_dtype, latent_dtype), len(fanout), (ctypes.c_int32 * 4)(*f),
                         kmeans_iters, seed)

    @staticmethod
    def of(wl) -> "IndexDesc":
        return IndexDesc.make(wl.n_keys, wl.n_kv_heads, wl.d_head, wl.d_latent, wl.key_dtype, wl.latent_dtype,
                              wl.fanout, wl.kmeans_iters, wl.seed)


class SelectParams(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("k", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("beam", ctypes.c_int32)]

    @staticmethod
    def make(b, k, sink, window, beam="per_parent"):
        return SelectParams(b, k, sink, window, BEAMS.get(beam, beam))


class LsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lsa error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblsa.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with hierarchical_key_indexer_amd.build_lib.build()")
    lib = ctypes.CDLL(path)
    P, SZ, I32, VP = ctypes.POINTER, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
    D, S = P(IndexDesc), P(SelectParams)
    lib.lsa_index_bytes.argtypes, lib.lsa_index_bytes.restype = [D], SZ
    lib.lsa_build_workspace_bytes.argtypes, lib.lsa_build_workspace_bytes.restype = [D], SZ
    lib.lsa_build_index.argtypes = [D, VP, VP, VP, SZ, VP, SZ, VP]
    lib.lsa_build_index.restype = ctypes.c_int
    lib.lsa_select_out_width.argtypes, lib.lsa_select_out_width.restype = [S], I32
    lib.lsa_select_workspace_bytes.argtypes, lib.lsa_select_workspace_bytes.restype = [D, S, I32, I32], SZ
    lib.lsa_flat_workspace_bytes.argtypes, lib.lsa_flat_workspace_bytes.restype = [D, S, I32, I32], SZ
    lib.lsa_select_path.argtypes, lib.lsa_select_path.restype = [D, S, I32, I32], I32
    lib.lsa_flat_select_path.argtypes, lib.lsa_flat_select_path.restype = [D, S, I32, I32], I32
    lib.lsa_select.argtypes = [D, VP, VP, VP, I32, I32, S, VP, VP, VP, VP, SZ, VP]
    lib.lsa_select.restype = ctypes.c_int
    lib.lsa_append_pool_bytes.argtypes, lib.lsa_append_pool_bytes.restype = [D, I32], SZ
    lib.lsa_append_keys.argtypes, lib.lsa_append_keys.restype = [D, VP, VP, I32, I32, VP, I32, VP], ctypes.c_int
    lib.lsa_select_appended_workspace_bytes.argtypes = [D, S, I32, I32]
    lib.lsa_select_appended_workspace_bytes.restype = SZ
    lib.lsa_select_appended.argtypes = [D, VP, VP, I32, I32, VP, VP, I32, I32, S, VP, VP, VP, VP, SZ, VP]
    lib.lsa_select_appended.restype = ctypes.c_int
    lib.lsa_select_noalloc.argtypes = [D, VP, VP, VP, I32, I32, S, VP, VP, VP, VP]
    lib.lsa_select_noalloc.restype = ctypes.c_int
    lib.lsa_flat_select.argtypes = [D, VP, VP, VP, I32, I32, S, VP, VP, VP, SZ, VP]
    lib.lsa_flat_select.restype = ctypes.c_int
    lib.lsa_last_error.argtypes, lib.lsa_last_error.restype = [], ctypes.c_char_p
    lib.lsa_abi_version.argtypes, lib.lsa_abi_version.restype = [], I32
    lib.lsa_set_profile_events.argtypes, lib.lsa_set_profile_events.restype = [I32, VP, VP], ctypes.c_int
    lib.lsa_pca_workspace_bytes.argtypes, lib.lsa_pca_workspace_bytes.restype = [D], SZ
    lib.lsa_pca_covariance.argtypes = [D, VP, VP, VP, SZ, VP]
    lib.lsa_pca_covariance.restype = ctypes.c_int
    lib.lsa_pca_map.argtypes = [D, VP, VP, VP]
    lib.lsa_pca_map.restype = ctypes.c_int
    lib.lsa_sparse_attention_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.lsa_sparse_attention_workspace_bytes.restype = SZ
    lib.lsa_sparse_attention.argtypes = [D, VP, VP, VP, VP, I32, I32, I32, ctypes.c_float, VP, VP, SZ, VP]
    lib.lsa_sparse_attention.restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().lsa_last_error().decode()


def _check(rc: int) -> None:
    if rc != LSA_OK:
        raise LsaError(rc, last_error())


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None stays NULL)."""
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ---- size queries ------------------------------------------------------------

def index_bytes(desc: IndexDesc) -> int:
    n = load().lsa_index_bytes(ctypes.byref(desc))
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def build_workspace_bytes(desc: IndexDesc) -> int:
    n = load().lsa_build_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def select_out_width(params: SelectParams) -> int:
    return load().lsa_select_out_width(ctypes.byref(params))


def select_workspace_bytes(desc, params, n_tokens, n_q_heads) -> int:
    n = load().lsa_select_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), n_tokens, n_q_heads)
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def flat_select_path(desc, params, n_tokens, n_q_heads) -> int:
    """PATH_PER_QUERY_HEAD or PATH_ROW_TILED: how lsa_flat_select computes a
    batch of this shape."""
    r = load().lsa_flat_select_path(ctypes.byref(desc), ctypes.byref(params), n_tokens, n_q_heads)
    if r < 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return r


def select_path(desc, params, n_tokens, n_q_heads) -> int:
    """PATH_PER_QUERY_HEAD or PATH_NODE_MAJOR: how lsa_select computes a
    batch of this shape."""
    r = load().lsa_select_path(ctypes.byref(desc), ctypes.byref(params), n_tokens, n_q_heads)
    if r < 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return r


def flat_workspace_bytes(desc, params, n_tokens, n_q_heads) -> int:
    n = load().lsa_flat_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), n_tokens, n_q_heads)
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


# ---- entry points (raw pointers) --------------------------------------------

def lsa_build_index(desc, keys, W, index, workspace, stream=None) -> None:
    """keys [N, Hkv, d] (fp32 or bf16), W [Hkv, d, dl] fp32, index/workspace
    uint8 tensors on the GPU."""
    _check(load().lsa_build_index(ctypes.byref(desc), _ptr(keys), _ptr(W), _ptr(index), index.numel(),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))


def lsa_select(desc, index, queries, q_pos, params, out_idx, out_scores=None, out_leaves=None, workspace=None,
               stream=None) -> None:
    t, hq = queries.shape[0], queries.shape[1]
    _check(load().lsa_select(ctypes.byref(desc), _ptr(index), _ptr(queries), _ptr(q_pos), t, hq,
                             ctypes.byref(params), _ptr(out_idx), _ptr(out_scores), _ptr(out_leaves),
                             _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream)))


def append_pool_bytes(desc, capacity) -> int:
    n = load().lsa_append_pool_bytes(ctypes.byref(desc), capacity)
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def select_appended_workspace_bytes(desc, params, n_tokens, n_q_heads) -> int:
    n = load().lsa_select_appended_workspace_bytes(ctypes.byref(desc), ctypes.byref(params), n_tokens, n_q_heads)
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def lsa_append_keys(desc, index, keys, first, pool, capacity, stream=None) -> None:
    """keys [n_new, Hkv, d] on the GPU into pool slots [first, first + n_new)."""
    _check(load().lsa_append_keys(ctypes.byref(desc), _ptr(index), _ptr(keys), keys.shape[0], first, _ptr(pool),
                                  capacity, _stream(stream)))


def lsa_select_appended(desc, index, pool, capacity, n_appended, queries, q_pos, params, out_idx, out_scores=None,
                        out_leaves=None, workspace=None, stream=None) -> None:
    t, hq = queries.shape[0], queries.shape[1]
    _check(load().lsa_select_appended(ctypes.byref(desc), _ptr(index), _ptr(pool), capacity, n_appended,
                                      _ptr(queries), _ptr(q_pos), t, hq, ctypes.byref(params), _ptr(out_idx),
                                      _ptr(out_scores), _ptr(out_leaves), _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _stream(stream)))


def lsa_select_noalloc(desc, index, queries, q_pos, params, out_idx, out_scores=None, out_leaves=None,
                       stream=None) -> None:
    """lsa_select on the library's static device scratch (no workspace)."""
    t, hq = queries.shape[0], queries.shape[1]
    _check(load().lsa_select_noalloc(ctypes.byref(desc), _ptr(index), _ptr(queries), _ptr(q_pos), t, hq,
                                     ctypes.byref(params), _ptr(out_idx), _ptr(out_scores), _ptr(out_leaves),
                                     _stream(stream)))


def lsa_flat_select(desc, index, queries, q_pos, params, out_idx, out_scores=None, workspace=None,
                    stream=None) -> None:
    t, hq = queries.shape[0], queries.shape[1]
    _check(load().lsa_flat_select(ctypes.byref(desc), _ptr(index), _ptr(queries), _ptr(q_pos), t, hq,
                                  ctypes.byref(params), _ptr(out_idx), _ptr(out_scores), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(stream)))


# ---- training-free latent map ----------------------------------------------------

def pca_workspace_bytes(desc: IndexDesc) -> int:
    n = load().lsa_pca_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise LsaError(LSA_ERR_INVALID_ARG, last_error())
    return n


def lsa_pca_covariance(desc, keys, cov, workspace, stream=None) -> None:
    """keys [N, Hkv, d] (fp32 or bf16) and cov [Hkv, d, d] float64 on the GPU;
    workspace a uint8 GPU tensor of pca_workspace_bytes(desc) bytes."""
    _check(load().lsa_pca_covariance(ctypes.byref(desc), _ptr(keys), _ptr(cov), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))


def lsa_pca_map(desc, cov):
    """Host: cov [Hkv, d, d] float64 (numpy) -> (W [Hkv, d, d_latent] float32,
    eigenvalues [Hkv, d_latent] float64)."""
    import numpy as np
    cov = np.ascontiguousarray(cov, dtype=np.float64)
    hk, d, dl = desc.n_kv_heads, desc.d_head, desc.d_latent
    assert cov.shape == (hk, d, d), cov.shape
    W = np.empty((hk, d, dl), dtype=np.float32)
    lam = np.empty((hk, dl), dtype=np.float64)
    _check(load().lsa_pca_map(ctypes.byref(desc), cov.ctypes.data, W.ctypes.data, lam.ctypes.data))
    return W, lam


# ---- exact sparse attention ----------------------------------------------------------

def sparse_attention_workspace_bytes(desc, width, n_tokens, n_q_heads) -> int:
    return load().lsa_sparse_attention_workspace_bytes(ctypes.byref(desc), width, n_tokens, n_q_heads)


def lsa_sparse_attention(desc, queries, keys, values, idx, scale, out, workspace=None, stream=None) -> None:
    """queries [T, Hq, d], keys / values [N, Hkv, d] (key dtype), idx [T, Hq,
    width] int32, out [T, Hq, d] float32, all on the GPU; workspace a uint8 GPU
    tensor of sparse_attention_workspace_bytes bytes (allocated here if None)."""
    t, hq, width = idx.shape
    if workspace is None:
        import torch
        n = sparse_attention_workspace_bytes(desc, width, t, hq)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=out.device)
    _check(load().lsa_sparse_attention(ctypes.byref(desc), _ptr(queries), _ptr(keys), _ptr(values), _ptr(idx),
                                       width, t, hq, float(scale), _ptr(out), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))


def device_status(workspace) -> int:
    """The device status a finished select call left in its workspace (bytes
    [0, 4)): LSA_OK or LSA_ERR_BAD_INDEX.  Synchronises with the device."""
    return int(workspace[:4].view(__import__("torch").int32).item())


def set_profile_events(stage: int, start, stop) -> None:
    """Record raw hipEvent_t handles around one stage of later select calls
    (None, None switches it off)."""
    _check(load().lsa_set_profile_events(stage, start, stop))
