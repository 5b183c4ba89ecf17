"""Seeded, chunk-regenerable synthetic workloads for the LSA indexer.

The five workloads follow the sizes and distributions of the long-context
setting the Latent Sparse Attention pages describe (1M-10M cached tokens,
128-dim heads, grouped query heads): keys are drawn around seeded Gaussian
centers, queries are noisy copies of random cached keys, the latent map W is
Gaussian.  Nothing here performs a step of the indexer.

Random streams
--------------
Every array is drawn from ``numpy.random.Generator(PCG64(SeedSequence(
entropy, spawn_key=(stream, head, chunk))))``.  ``entropy`` is
``20261030 + cache_id`` for key-cache streams and ``20261030 + query_id`` for
query streams, so the 1M decode and 1M prefill workloads share one cache (and
likewise at 10M) while drawing their own queries.  Keys come in chunks of
``2**20`` rows so any chunk can be regenerated on its own.

stream 0  centers ~ N(0, I_d), one set per KV head
stream 1  key -> center id, uniform
stream 2  key noise ~ N(0, I_d)
stream 3  outlier mask, uniform < outlier_frac
stream 4  latent map W ~ N(0, 1/d_head), one [d_head, d_latent] per KV head
stream 5  query source key r ~ U[0, N)
stream 6  query noise ~ N(0, I_d)

A key is ``center + sigma * noise``; an outlier key is ``noise`` itself (an
independent N(0, I) draw).  A query is ``key_r + 0.3 * noise`` rounded to the
key dtype.  bf16 storage uses round-to-nearest-even of the fp32 draw.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

ENTROPY_BASE = 20261030
CHUNK = 1 << 20

S_CENTERS, S_ASSIGN, S_NOISE, S_OUTLIER, S_W, S_QKEY, S_QNOISE = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cache_id: int
    query_id: int
    n_keys: int
    n_kv_heads: int
    group: int            # query heads per KV head
    d_head: int
    d_latent: int
    key_dtype: str        # "f32" | "bf16"
    latent_dtype: str     # "f32" | "bf16"
    fanout: tuple
    kmeans_iters: int
    n_centers: int
    sigma: float
    outlier_frac: float
    n_tokens: int
    b: int
    k: int
    sink: int
    window: int
    query_noise: float = 0.3
    seed: int = 0x5EED

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def n_levels(self) -> int:
        return len(self.fanout)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1-level index of 256 buckets over 65,536 fp32 keys, one head.
    "tiny_flat_65k": Workload(
        name="tiny_flat_65k", cache_id=0, query_id=0, n_keys=65536,
        n_kv_heads=1, group=1, d_head=128, d_latent=32, key_dtype="f32",
        latent_dtype="f32", fanout=(256,), kmeans_iters=10, n_centers=256,
        sigma=0.5, outlier_frac=0.0, n_tokens=64, b=8, k=256, sink=4,
        window=128, seed=0x5EED0),
    # 2-level tree (64 x 64) over 1M bf16 keys, 8 KV heads x 4 query heads, one token.
    "decode_1m": Workload(
        name="decode_1m", cache_id=1, query_id=1, n_keys=1 << 20,
        n_kv_heads=8, group=4, d_head=128, d_latent=64, key_dtype="bf16",
        latent_dtype="bf16", fanout=(64, 64), kmeans_iters=10, n_centers=4096,
        sigma=0.5, outlier_frac=0.0, n_tokens=1, b=16, k=2048, sink=4,
        window=512, seed=0x5EED1),
    # same cache and index, a causal chunk of 4096 tokens at the tail.
    "prefill_1m": Workload(
        name="prefill_1m", cache_id=1, query_id=2, n_keys=1 << 20,
        n_kv_heads=8, group=4, d_head=128, d_latent=64, key_dtype="bf16",
        latent_dtype="bf16", fanout=(64, 64), kmeans_iters=10, n_centers=4096,
        sigma=0.5, outlier_frac=0.0, n_tokens=4096, b=16, k=2048, sink=4,
        window=512, seed=0x5EED1),
    # 3-level tree (64^3) over 10M bf16 keys with 10% outliers, one token.
    "decode_10m": Workload(
        name="decode_10m", cache_id=3, query_id=3, n_keys=10_000_000,
        n_kv_heads=8, group=4, d_head=128, d_latent=64, key_dtype="bf16",
        latent_dtype="bf16", fanout=(64, 64, 64), kmeans_iters=10,
        n_centers=65536, sigma=0.5, outlier_frac=0.1, n_tokens=1, b=8,
        k=2048, sink=4, window=1024, seed=0x5EED3),
    # same cache and index, a causal chunk of 8192 tokens at the tail.
    "prefill_10m": Workload(
        name="prefill_10m", cache_id=3, query_id=4, n_keys=10_000_000,
        n_kv_heads=8, group=4, d_head=128, d_latent=64, key_dtype="bf16",
        latent_dtype="bf16", fanout=(64, 64, 64), kmeans_iters=10,
        n_centers=65536, sigma=0.5, outlier_frac=0.1, n_tokens=8192, b=8,
        k=2048, sink=4, window=1024, seed=0x5EED3),
}


def get_workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.scaled(**overrides) if overrides else wl


def _gen(entropy: int, stream: int, head: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy, spawn_key=(stream, head, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 storage bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _centers(wl: Workload, h: int) -> np.ndarray:
    e = ENTROPY_BASE + wl.cache_id
    return _gen(e, S_CENTERS, h, 0).standard_normal((wl.n_centers, wl.d_head), dtype=np.float32)


def _key_chunk_f32(wl: Workload, h: int, c: int, centers: np.ndarray) -> np.ndarray:
    e = ENTROPY_BASE + wl.cache_id
    lo = c * CHUNK
    n = min(wl.n_keys, lo + CHUNK) - lo
    ids = _gen(e, S_ASSIGN, h, c).integers(0, wl.n_centers, size=n)
    noise = np.empty((n, wl.d_head), dtype=np.float32)
    _gen(e, S_NOISE, h, c).standard_normal(dtype=np.float32, out=noise)
    keys = centers[ids]
    keys += np.float32(wl.sigma) * noise
    if wl.outlier_frac > 0.0:
        out = _gen(e, S_OUTLIER, h, c).random(n) < wl.outlier_frac
        keys[out] = noise[out]
    return keys


def gen_keys_head_f32(wl: Workload, h: int, lo: int = 0, hi: int | None = None) -> np.ndarray:
    """fp32 draws of keys [lo, hi) of KV head h (before storage rounding)."""
    hi = wl.n_keys if hi is None else hi
    centers = _centers(wl, h)
    parts = []
    for c in range(lo // CHUNK, (hi - 1) // CHUNK + 1):
        blk = _key_chunk_f32(wl, h, c, centers)
        base = c * CHUNK
        parts.append(blk[max(lo, base) - base: min(hi, base + len(blk)) - base])
    return np.concatenate(parts, axis=0)


def gen_keys(wl: Workload) -> np.ndarray:
    """The key cache [N, Hkv, d_head]: float32 (key_dtype f32) or uint16 bf16 bits."""
    n, hk, d = wl.n_keys, wl.n_kv_heads, wl.d_head
    out_dt = np.float32 if wl.key_dtype == "f32" else np.uint16
    out = np.empty((n, hk, d), dtype=out_dt)
    nchunks = (n + CHUNK - 1) // CHUNK
    centers = [_centers(wl, h) for h in range(hk)]

    def work(job):
        h, c = job
        blk = _key_chunk_f32(wl, h, c, centers[h])
        lo = c * CHUNK
        out[lo:lo + len(blk), h, :] = blk if wl.key_dtype == "f32" else f32_to_bf16_bits(blk)

    jobs = [(h, c) for h in range(hk) for c in range(nchunks)]
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return out


def gen_keys_range(wl: Workload, lo: int, hi: int) -> np.ndarray:
    """Keys [lo, hi) of every KV head, [hi - lo, Hkv, d_head] in the key
    storage dtype, drawn as a cache of max(hi, N) keys would hold them: the
    streams are sequential within a chunk, so positions at or past N are the
    keys that arrive after a cache of N keys, and positions below N equal
    gen_keys(wl)."""
    big = wl.scaled(n_keys=max(hi, wl.n_keys))
    out = np.stack([gen_keys_head_f32(big, h, lo, hi) for h in range(wl.n_kv_heads)], axis=1)
    return out if wl.key_dtype == "f32" else f32_to_bf16_bits(out)


def gen_W(wl: Workload) -> np.ndarray:
    """Latent maps [Hkv, d_head, d_latent] fp32, entries ~ N(0, 1/d_head)."""
    e = ENTROPY_BASE + wl.cache_id
    scale = np.float32(1.0 / np.sqrt(wl.d_head))
    return np.stack([
        _gen(e, S_W, h, 0).standard_normal((wl.d_head, wl.d_latent), dtype=np.float32) * scale
        for h in range(wl.n_kv_heads)])


def gen_positions(wl: Workload) -> np.ndarray:
    """Query positions: the last n_tokens positions of the cache."""
    return np.arange(wl.n_keys - wl.n_tokens, wl.n_keys, dtype=np.int32)


def gen_queries(wl: Workload, keys: np.ndarray) -> np.ndarray:
    """Queries [T, Hq, d_head] in the key storage dtype: key_r + 0.3 * noise."""
    e = ENTROPY_BASE + wl.query_id
    t, hq, d = wl.n_tokens, wl.n_q_heads, wl.d_head
    q = np.empty((t, hq, d), dtype=np.float32)
    for qh in range(hq):
        h = qh // wl.group
        r = _gen(e, S_QKEY, qh, 0).integers(0, wl.n_keys, size=t)
        noise = _gen(e, S_QNOISE, qh, 0).standard_normal((t, d), dtype=np.float32)
        src = keys[r, h, :]
        src = src if wl.key_dtype == "f32" else bf16_bits_to_f32(src)
        q[:, qh, :] = src + np.float32(wl.query_noise) * noise
    return q if wl.key_dtype == "f32" else f32_to_bf16_bits(q)
