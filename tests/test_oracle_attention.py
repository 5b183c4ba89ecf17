"""Pins of the oracle's exact sparse attention over a row of selected keys
([WPN] "How does LSA work?", step 3: plain softmax attention restricted to
the listed keys).  Closed forms, none of which re-types the oracle."""
import numpy as np

from oracle import lsa_oracle as O


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def test_single_key_returns_its_value():
    k = _f32([[[1.0, 2.0]], [[3.0, -1.0]]])          # N=2, Hkv=1, d=2
    v = _f32([[[5.0, 6.0]], [[-7.0, 8.0]]])
    q = _f32([[[0.5, 0.25]]])
    out = O.sparse_attention(q, k, v, np.array([[[1, -1, -1]]]), "f32", 1.0)
    assert np.array_equal(out[0, 0], [-7.0, 8.0])


def test_two_keys_closed_form_weights():
    # scores a and b: weights 1 / (1 + e^(b - a)) and its complement
    k = _f32([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = _f32([[[1.0, 0.0]], [[0.0, 1.0]]])
    q = _f32([[[2.0, 0.5]]])
    scale = 0.75
    a, b = scale * 2.0, scale * 0.5
    wa = 1.0 / (1.0 + np.exp(b - a))
    out = O.sparse_attention(q, k, v, np.array([[[0, 1]]]), "f32", scale)
    assert np.allclose(out[0, 0], [wa, 1.0 - wa], rtol=0, atol=1e-15)


def test_zero_scale_is_the_mean_and_padding_is_ignored():
    rng = np.random.default_rng(0)
    k = _f32(rng.standard_normal((10, 1, 4)))
    v = _f32(rng.standard_normal((10, 1, 4)))
    q = _f32(rng.standard_normal((1, 1, 4)))
    sel = [7, 2, 9]
    out = O.sparse_attention(q, k, v, np.array([[[7, -1, 2, -1, 9]]]), "f32", 0.0)
    assert np.allclose(out[0, 0], v[sel, 0, :].astype(np.float64).mean(0), atol=1e-15)


def test_entries_outside_the_cache_are_padding():
    k = _f32([[[1.0]], [[2.0]]])
    v = _f32([[[3.0]], [[4.0]]])
    q = _f32([[[0.0]]])
    out = O.sparse_attention(q, k, v, np.array([[[1, 2, 7, -5]]]), "f32", 1.0)
    assert np.array_equal(out[0, 0], [4.0])


def test_empty_row_gives_zeros_and_gqa_reads_its_kv_head():
    # two KV heads, G = 2: query heads 2 and 3 read KV head 1
    k = _f32(np.zeros((3, 2, 2)))
    v = _f32([[[1, 1], [10, 10]], [[2, 2], [20, 20]], [[3, 3], [30, 30]]])
    q = _f32(np.ones((1, 4, 2)))
    idx = np.array([[[0, 1], [-1, -1], [2, -1], [0, 2]]])
    out = O.sparse_attention(q, k, v, idx, "f32", 1.0)
    assert np.array_equal(out[0, 0], [1.5, 1.5])      # equal scores: mean over KV head 0
    assert np.array_equal(out[0, 1], [0.0, 0.0])      # empty row
    assert np.array_equal(out[0, 2], [30.0, 30.0])    # KV head 1
    assert np.array_equal(out[0, 3], [20.0, 20.0])


def test_shift_invariance_and_bf16_storage():
    # adding the same vector c to every key adds scale * q.c to every score:
    # the output does not change (small integers: every value is exact)
    rng = np.random.default_rng(1)
    k = rng.integers(-4, 5, size=(50, 1, 8)).astype(np.float64)
    c = rng.integers(-4, 5, size=(1, 1, 8)).astype(np.float64)
    v = rng.integers(-4, 5, size=(50, 1, 8)).astype(np.float64)
    q = rng.integers(-2, 3, size=(1, 1, 8)).astype(np.float64) / 4
    idx = rng.permutation(50)[None, None, :20]
    bf = lambda x: O.f64_to_bf16_bits(x)
    a = O.sparse_attention(bf(q), bf(k), bf(v), idx, "bf16", 0.3)
    b = O.sparse_attention(bf(q), bf(k + c), bf(v), idx, "bf16", 0.3)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    # bf16 storage is decoded: the same values stored as fp32 give the same result
    c32 = O.sparse_attention(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), idx, "f32", 0.3)
    assert np.array_equal(a, c32)
