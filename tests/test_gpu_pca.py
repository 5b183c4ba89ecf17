"""lsa_pca_covariance on the GPU against the oracle's covariance, and the
whole training-free map (device covariance, host eigenvectors) against the
oracle's map.

Tolerance of the covariance, from the arithmetic: the kernel sums, per chunk
of m keys, products of fp32 keys shifted by the head's first key (one rounding
each) in fp32, and adds chunks in fp64.  By the standard bound for recursive
summation, entry (i, j) is off by at most (m + 2) u sum_k |x~_ki x~_kj| / N
(u = 2^-24, x~ the shifted keys), and the centring term by at most
(m + 2) u (|m_i| a_j + |m_j| a_i) with a = sum_k |x~_k| / N.  The test uses
that bound, entry by entry, doubled."""
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


def _keys(rng, n, hk, d, dtype, offset=0.0, scale=None):
    scale = 2.0 ** (-np.arange(d) / 8.0) if scale is None else scale
    x = rng.standard_normal((n, hk, d)) * scale + offset
    q = [np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(hk)]
    x = np.stack([x[:, h] @ q[h].T for h in range(hk)], axis=1)
    if dtype == "bf16":
        return O.f64_to_bf16_bits(O.round_bf16(x))
    return x.astype(np.float32)


def _gpu_cov(A, desc, keys):
    dev = torch.from_numpy(keys.view(np.int16) if keys.dtype == np.uint16 else keys).cuda()
    cov = torch.empty((desc.n_kv_heads, desc.d_head, desc.d_head), dtype=torch.float64, device="cuda")
    ws = torch.empty(A.pca_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    A.lsa_pca_covariance(desc, dev, cov, ws)
    torch.cuda.synchronize()
    return cov.cpu().numpy()


def _bound(x, m):
    """Entry-wise error bound of the kernel's covariance (see the module doc)."""
    u = 2.0 ** -24
    n, hk, d = x.shape
    out = np.empty((hk, d, d))
    for h in range(hk):
        xs = np.abs(x[:, h, :] - x[0, h, :])
        mean = np.abs((x[:, h, :] - x[0, h, :]).mean(0))
        a = xs.mean(0)
        out[h] = (m + 2) * u * (xs.T @ xs / n + np.outer(mean, a) + np.outer(a, mean))
    return out


CASES = [  # n, hk, d, dtype, offset
    (50_000, 2, 128, "bf16", 0.0),
    (4_097, 2, 128, "bf16", 3.0),        # two chunks, ragged; a large mean
    (33, 3, 64, "f32", 0.0),             # one partial tile
    (1, 1, 64, "f32", 0.0),              # a single key: zero covariance
    (10_000, 1, 256, "f32", -1.0),       # four passes over the output blocks
    (1_100_000, 1, 128, "bf16", 0.5),    # the full chunk count (256 chunks)
]


@pytest.mark.parametrize("n,hk,d,dtype,offset", CASES)
def test_covariance_matches_oracle(n, hk, d, dtype, offset):
    from hierarchical_key_indexer_amd import _abi as A
    log(f"[pca] covariance n={n} hk={hk} d={d} {dtype}")
    rng = np.random.default_rng(n + d)
    keys = _keys(rng, n, hk, d, dtype, offset)
    desc = A.IndexDesc.make(n, hk, d, 32, dtype, dtype, (4,), 1, 0)
    got = _gpu_cov(A, desc, keys)
    want = O.key_covariance(keys, dtype)
    x = O.stored_to_f64(keys, dtype)
    nch = min(256, max(1, -(-n // 4096)))
    m = -(-n // nch)
    err = np.abs(got - want)
    bound = 2.0 * _bound(x, m) + 1e-300
    assert np.all(err <= bound), f"worst ratio {np.max(err / bound):.3g}"
    assert np.array_equal(got, np.swapaxes(got, 1, 2)) or np.allclose(got, np.swapaxes(got, 1, 2), rtol=0,
                                                                       atol=float(bound.max()))


@pytest.mark.parametrize("d,dl", [(128, 64), (64, 32)])
def test_map_matches_oracle(d, dl):
    # The device covariance differs from the oracle's by E; the library's
    # eigenpairs of it must lie within the perturbation bounds of the oracle's:
    # each eigenvalue within ||E||_2 (Weyl), each eigenvector within
    # sqrt(2) ||E||_2 / (gap - ||E||_2) of the oracle's (Davis-Kahan sin-theta,
    # up to the sign), plus the fp32 rounding of W.
    from hierarchical_key_indexer_amd import _abi as A
    log(f"[pca] map d={d} dl={dl}")
    rng = np.random.default_rng(7 * d)
    n = 20_000
    # the kept directions have scales 3 .. 1 (eigenvalue gaps ~0.1), the rest 0.3
    scale = np.concatenate([np.linspace(3.0, 1.0, dl), np.full(d - dl, 0.3)])
    keys = _keys(rng, n, 2, d, "bf16", scale=scale)
    desc = A.IndexDesc.make(n, 2, d, dl, "bf16", "bf16", (4,), 1, 0)
    cov_g = _gpu_cov(A, desc, keys)
    W, lam = A.lsa_pca_map(desc, cov_g)
    cov_o = O.key_covariance(keys, "bf16")
    Wo, lo = O.pca_from_covariance(cov_o, dl)
    for h in range(2):
        e = np.linalg.norm(cov_g[h] - cov_o[h], 2)
        full = np.linalg.eigvalsh(cov_o[h])[::-1]
        assert np.all(np.abs(lam[h] - lo[h]) <= e + 1e-12 * full[0])
        for c in range(dl):
            gap = min(full[c - 1] - full[c] if c > 0 else np.inf, full[c] - full[c + 1])
            assert gap > 2 * e, "the spectrum of this input is not separated enough for the check"
            dist = min(np.linalg.norm(W[h][:, c] - Wo[h][:, c]), np.linalg.norm(W[h][:, c] + Wo[h][:, c]))
            assert dist <= np.sqrt(2) * e / (gap - e) + 1e-6, (h, c, dist, e, gap)
            r = int(np.argmax(np.abs(W[h][:, c])))
            assert W[h][r, c] > 0
        # orthonormal columns in fp32
        assert np.allclose(W[h].T.astype(np.float64) @ W[h], np.eye(dl), atol=1e-6)


def test_covariance_validation():
    from hierarchical_key_indexer_amd import _abi as A
    desc = A.IndexDesc.make(100, 1, 64, 32, "f32", "f32", (4,), 1, 0)
    lib = A.load()
    ws = torch.empty(A.pca_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    assert lib.lsa_pca_covariance(desc, None, None, ws.data_ptr(), ws.numel(), None) == A.LSA_ERR_INVALID_ARG
    keys = torch.zeros((100, 1, 64), dtype=torch.float32, device="cuda")
    cov = torch.zeros((1, 64, 64), dtype=torch.float64, device="cuda")
    assert lib.lsa_pca_covariance(desc, keys.data_ptr(), cov.data_ptr(), ws.data_ptr(), 16, None) == \
        A.LSA_ERR_BUFFER_TOO_SMALL
