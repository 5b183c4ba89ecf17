"""The library's host eigensolver (lsa_pca_map) against the oracle's map.

lsa_pca_map touches no device, so these run on the CPU: the covariance comes
from the oracle (float64), the library returns W and the eigenvalues, and the
oracle's eigendecomposition of the same matrix is the reference.  The spectra
used here are well separated, so eigenvectors are compared entry by entry
(W is stored as fp32: tolerance 1e-6)."""
import numpy as np
import pytest

from oracle import lsa_oracle as O
from hierarchical_key_indexer_amd import _abi as A


@pytest.fixture(scope="module", autouse=True)
def _lib():
    A.load()


def _desc(n, hk, d, dl, dtype="f32"):
    return A.IndexDesc.make(n, hk, d, dl, dtype, dtype, (4,), 1, 0)


def _spread_keys(rng, n, hk, d):
    # per head, scales falling geometrically: distinct, well separated eigenvalues
    scale = 2.0 ** (-np.arange(d) / 8.0)
    x = rng.standard_normal((n, hk, d)) * scale
    q = [np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(hk)]
    return np.stack([x[:, h] @ q[h].T for h in range(hk)], axis=1).astype(np.float32)


@pytest.mark.parametrize("d,dl", [(64, 32), (128, 64), (256, 64)])
def test_host_map_matches_oracle(d, dl):
    rng = np.random.default_rng(d)
    keys = _spread_keys(rng, 4 * d, 2, d)
    cov = O.key_covariance(keys, "f32")
    Wo, lo = O.pca_from_covariance(cov, dl)
    W, lam = A.lsa_pca_map(_desc(keys.shape[0], 2, d, dl), cov)
    assert np.allclose(lam, lo, rtol=1e-9, atol=1e-14)
    assert np.abs(W - Wo).max() < 1e-6


def test_host_map_exact_basis():
    # a diagonal covariance with a signed permutation basis: W is that permutation
    d, dl = 64, 32
    rng = np.random.default_rng(1)
    perm = rng.permutation(d)
    diag = np.zeros((1, d, d))
    for i in range(d):
        diag[0, perm[i], perm[i]] = float(d - i)
    W, lam = A.lsa_pca_map(_desc(10, 1, d, dl), diag)
    assert np.array_equal(lam[0], np.arange(d, d - dl, -1, dtype=np.float64))
    want = np.zeros((d, dl), dtype=np.float32)
    for c in range(dl):
        want[perm[c], c] = 1.0
    assert np.array_equal(W[0], want)


def test_host_map_errors():
    lib = A.load()
    d = _desc(100, 1, 64, 32)
    assert lib.lsa_pca_map(d, None, None, None) == A.LSA_ERR_INVALID_ARG
    bad = _desc(100, 1, 48, 32)                     # d_head not supported
    cov = np.zeros((1, 48, 48))
    W = np.zeros((1, 48, 32), dtype=np.float32)
    assert lib.lsa_pca_map(bad, cov.ctypes.data, W.ctypes.data, None) == A.LSA_ERR_UNSUPPORTED
    assert "d_head" in A.last_error()
    assert lib.lsa_pca_workspace_bytes(bad) == 0
    assert A.pca_workspace_bytes(d) > 0
