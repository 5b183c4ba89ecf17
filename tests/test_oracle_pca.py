"""Pins of the oracle's training-free latent map (PCA of each KV head's keys).

[WPN] "How does LSA work?" names a training-free option built on a PCA map;
the reading (leading eigenvectors of the mean-centred key covariance, sorted by
eigenvalue, signed so the largest-magnitude entry is positive) is checked here
against closed forms and invariants, none of which re-types the oracle."""
import numpy as np
import pytest

from oracle import lsa_oracle as O


def _keys(rows):
    """[N, d] values -> keys [N, 1, d] stored as fp32."""
    return np.asarray(rows, dtype=np.float32)[:, None, :]


def test_two_dimensional_closed_form():
    # points (1,1), (-1,-1), (s,-s), (-s,s): covariance 1/2 [[1+s^2, 1-s^2], [1-s^2, 1+s^2]],
    # eigenpairs 1 along (1,1)/sqrt2 and s^2 along (1,-1)/sqrt2
    s = 0.5
    W, lam = O.pca_map(_keys([[1, 1], [-1, -1], [s, -s], [-s, s]]), "f32", 2)
    assert np.allclose(lam[0], [1.0, s * s], rtol=0, atol=1e-15)
    r = 1 / np.sqrt(2)
    # equal magnitudes: the lower row is the positive one
    assert np.allclose(W[0], [[r, r], [r, -r]], rtol=0, atol=1e-15)


def test_signed_permutation_basis_is_recovered_exactly():
    # keys +-a_i e_pi(i): the covariance is diagonal with entries 2 a_i^2 / N
    d, dl = 8, 5
    perm = [3, 0, 6, 1, 7, 2, 5, 4]
    a = [8.0, 7.0, 6.0, 5.0, 4.0, 3.0, 2.0, 1.0]
    rows = []
    for i in range(d):
        e = np.zeros(d)
        e[perm[i]] = a[i]
        rows += [e, -e]
    W, lam = O.pca_map(_keys(rows), "f32", dl)
    n = 2 * d
    assert np.array_equal(lam[0], [2 * a[i] ** 2 / n for i in range(dl)])
    want = np.zeros((d, dl))
    for c in range(dl):
        want[perm[c], c] = 1.0
    assert np.array_equal(W[0], want)


def test_a_constant_offset_changes_nothing():
    # the covariance is mean-centred: shifting every key leaves the map alone
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(64, 2, 6)).astype(np.float32)
    off = rng.integers(-100, 101, size=(1, 2, 6)).astype(np.float32)
    W0, l0 = O.pca_map(x, "f32", 3)
    W1, l1 = O.pca_map(x + off, "f32", 3)
    assert np.allclose(l0, l1, rtol=1e-12, atol=0)
    assert np.allclose(W0, W1, rtol=0, atol=1e-9)


def test_heads_are_independent_and_the_layout_is_head_dim_latent():
    # head 1 holds head 0's keys with two coordinates swapped: its map is head
    # 0's with the same two rows swapped
    rng = np.random.default_rng(4)
    x0 = rng.standard_normal((200, 5)).astype(np.float32)
    x1 = x0[:, [1, 0, 2, 3, 4]]
    W, lam = O.pca_map(np.stack([x0, x1], axis=1), "f32", 3)
    assert W.shape == (2, 5, 3) and lam.shape == (2, 3)
    assert np.allclose(lam[0], lam[1], rtol=1e-12)
    assert np.allclose(W[1], W[0][[1, 0, 2, 3, 4]], atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_properties_on_random_keys(dtype):
    rng = np.random.default_rng(5)
    d, dl = 32, 8
    x = (rng.standard_normal((500, 2, d)) * np.linspace(3, 0.1, d)).astype(np.float32)
    keys = O.f64_to_bf16_bits(O.round_bf16(x.astype(np.float64))) if dtype == "bf16" else x
    W, lam = O.pca_map(keys, dtype, dl)
    xv = O.stored_to_f64(keys, dtype)
    for h in range(2):
        xc = xv[:, h, :] - xv[:, h, :].mean(0)
        C = xc.T @ xc / xc.shape[0]
        # orthonormal columns; each is an eigenvector with its eigenvalue
        assert np.allclose(W[h].T @ W[h], np.eye(dl), atol=1e-12)
        assert np.allclose(C @ W[h], W[h] * lam[h], atol=1e-10)
        # descending, and the leading ones: no eigenvalue of C exceeds the last kept one
        # unless it is kept
        assert np.all(np.diff(lam[h]) <= 0)
        allw = np.linalg.eigvalsh(C)[::-1]
        assert np.allclose(lam[h], allw[:dl], rtol=1e-12)
        # the variance of the projected keys is the sum of the kept eigenvalues
        assert np.isclose(((xc @ W[h]) ** 2).mean(0).sum(), lam[h].sum(), rtol=1e-12)
        # sign convention
        for c in range(dl):
            r = int(np.argmax(np.abs(W[h][:, c])))
            assert W[h][r, c] > 0
