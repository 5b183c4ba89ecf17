"""CPU oracle for the Latent Sparse Attention (LSA) indexer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and does not import it.

What it computes, and where the pages say so
--------------------------------------------
The method (page "Latent Sparse Attention (LSA): The 72.4x and 22.7x Speedups,
and What They Compare Against", wpnews.pro, section "How does LSA work?"):

1. keys are clustered into buckets in a latent space, organised as a hierarchy
   (step 1) -> ``latent_keys`` + ``build_index`` (Lloyd k-means per node);
2. selection works on clusters before keys: the query is compared with the
   bucket centroids, and only the buckets that win are opened and their keys
   scored (step 2) -> ``descend`` + the key stage of ``select_one``;
3. what the query finally reads is those winning far keys, together with the
   first (sink) positions and the positions just before it (step 3) ->
   ``segments`` and the output row of ``select``.

The same descent is drawn on "Latent Sparse Attention: tree search over keys
for 10M-token context" (bayesiansapien wiki), TL;DR and flowchart: the query
compares the query with cluster centroids and walks down into a handful of the
highest-scoring buckets, in place of scoring every key; scoring every key is
``flat_select``.

Readings taken where the pages are silent:
per-parent beam (every kept node keeps its top-b children), inner-product
scores, top-down Lloyd k-means with seeded Forgy init (splitmix64), empty
clusters keep their centroid and score -inf, ties to the lowest id/index,
sink = positions [0, sink), window = the last ``window`` positions up to p,
long-range candidates C(p) = [sink, p - window], top-k reported in ascending
index order, -1 padding.

Arithmetic: every value is widened from its stored format (bf16 / fp32) to
float64 and all sums are float64.  Latent keys, latent queries and the scoring
copy of centroids are rounded once (round-to-nearest-even) to the latent dtype;
centroids are kept as fp32 values, exactly as stored.  Squared distances are
evaluated as |x|^2 - 2 x.mu + |mu|^2 in float64; their rounding (< 1e-15
relative to |x|^2 + |mu|^2) is far below the 1e-4 assignment tolerance, and
exact ties are decided on these float64 values (lowest cluster id wins).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import scipy.sparse

# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 storage bits (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), once.

    bf16 keeps 8 significant bits: for |x| in [2^e, 2^(e+1)) the spacing is
    2^(e-7); below 2^-126 the spacing is the subnormal step 2^-133.  Scaling by
    a power of two and ``rint`` (ties to even) are exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -ulp_exp)), ulp_exp)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(x == 0, x, r)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp32 value (IEEE conversion, RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_latent(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Storage bits of float64 values that are already bf16 values."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    assert np.all((u & np.uint32(0xFFFF)) == 0), "value is not a bf16 value"
    return (u >> np.uint32(16)).astype(np.uint16)


def stored_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen keys/queries held in their storage format to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014; public-domain constants of Vigna's splitmix64.c)
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def _mix64(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


class SplitMix64:
    """The splitmix64 generator: state += gamma, output = mix(state)."""

    def __init__(self, seed: int):
        self.state = seed & _M64

    def next(self) -> int:
        self.state = (self.state + _GAMMA) & _M64
        return _mix64(self.state)


def node_stream(seed: int, head: int, level: int, node: int) -> SplitMix64:
    """Generator that seeds the k-means of one tree node.

    tag = (head * 16 + level) * 2^32 + node; the stream is a splitmix64
    generator started at ``seed XOR first_output(splitmix64(tag))``.
    """
    tag = (((head * 16 + level) << 32) + node) & _M64
    return SplitMix64((seed & _M64) ^ SplitMix64(tag).next())


def kmeans_init_positions(seed: int, head: int, level: int, node: int, m: int, f: int) -> list:
    """Seeded Forgy init: ordinals (into the node's ascending-index member list)
    of the members that become the initial centroids of children 0, 1, ...

    With m <= f members, child c starts at member c (c < m) and the remaining
    children stay void.  Otherwise draw u = next() mod m, skipping repeats,
    until f distinct ordinals are chosen; child c takes the c-th distinct draw.
    """
    if m <= f:
        return list(range(m))
    g = node_stream(seed, head, level, node)
    chosen, seen = [], set()
    while len(chosen) < f:
        u = g.next() % m
        if u not in seen:
            seen.add(u)
            chosen.append(u)
    return chosen


# ----------------------------------------------------------------------------
# Lloyd k-means (the clustering that forms the buckets: step 1 of "How does
# LSA work?" groups keys into a hierarchy of buckets in latent space but names
# no algorithm; Lloyd's two-step iteration is the reading)
# ----------------------------------------------------------------------------


def sq_dists(x: np.ndarray, c: np.ndarray, xx: np.ndarray | None = None) -> np.ndarray:
    """Squared Euclidean distances [m, F] in float64: |x|^2 - 2 x.c + |c|^2."""
    if xx is None:
        xx = np.einsum("ij,ij->i", x, x)
    d = x @ c.T
    d *= -2.0
    d += np.einsum("ij,ij->i", c, c)[None, :]
    d += xx[:, None]
    return d


def assign_nearest(x: np.ndarray, c: np.ndarray, xx: np.ndarray | None = None, chunk: int = 1 << 16) -> np.ndarray:
    """Index of the nearest centroid for every row; ties -> lowest index."""
    if xx is None:
        xx = np.einsum("ij,ij->i", x, x)
    out = np.empty(len(x), dtype=np.int64)
    for lo in range(0, len(x), chunk):
        out[lo:lo + chunk] = np.argmin(sq_dists(x[lo:lo + chunk], c, xx[lo:lo + chunk]), axis=1)
    return out


def member_means(x: np.ndarray, a: np.ndarray, n: int):
    """(counts [n], sums [n, d]) of the rows of x grouped by label a, as the
    product of the n x m membership (one-hot) matrix with x, in float64."""
    cnt = np.bincount(a, minlength=n)
    member = scipy.sparse.csr_matrix((np.ones(len(a)), (a, np.arange(len(a)))), shape=(n, len(a)))
    return cnt, np.asarray(member @ x)


def lloyd(x: np.ndarray, f: int, iters: int, init_pos: list):
    """Lloyd k-means of one node's members ``x`` (ascending key order).

    Returns (centroids [f, d] fp32 values as float64, assignment [m],
    n_initialised).  Void children (index >= n_initialised) have zero
    centroids and take no members.  An initialised child that loses all its
    members keeps its centroid.  After ``iters`` (assign, update) rounds a
    final assign is made against the last centroids, which are the stored
    ones.
    """
    nv = len(init_pos)
    cent = np.zeros((f, x.shape[1]))
    if nv == 0:
        return cent, np.zeros(0, dtype=np.int64), 0
    cent[:nv] = round_f32(x[np.asarray(init_pos)])
    xx = np.einsum("ij,ij->i", x, x)
    for _ in range(iters):
        a = assign_nearest(x, cent[:nv], xx)
        cnt, sums = member_means(x, a, nv)
        nz = cnt > 0
        cent[:nv][nz] = round_f32(sums[nz] / cnt[nz, None])
    return cent, assign_nearest(x, cent[:nv], xx), nv


def lloyd_objective(x: np.ndarray, cent: np.ndarray, a: np.ndarray) -> float:
    d = x - cent[a]
    return float(np.einsum("ij,ij->", d, d))


# ----------------------------------------------------------------------------
# training-free latent map (PCA)
# ----------------------------------------------------------------------------
# [WPN] "How does LSA work?" lists, next to the distilled map, a training-free
# option that builds the latent map from a PCA.  The page gives no detail; the
# plainest reading: per KV head, the d_l leading eigenvectors of the keys'
# (mean-centred) covariance are the columns of W_h.  Centring does not change
# a ranking by q~ . k~ (it shifts every key's score of one query by the same
# amount).  Eigenvalues are reported in descending order; each eigenvector is
# signed so that its entry of largest magnitude (lowest index on a tie) is
# positive.


def key_covariance(keys: np.ndarray, key_dtype: str) -> np.ndarray:
    """Per KV head the covariance (1/N) sum_j (k_j - mean)(k_j - mean)^T of the
    keys [N, Hkv, d_head], in float64: [Hkv, d_head, d_head]."""
    x = stored_to_f64(keys, key_dtype)
    n, hk, d = x.shape
    out = np.empty((hk, d, d))
    for h in range(hk):
        xc = x[:, h, :] - x[:, h, :].mean(axis=0)
        out[h] = xc.T @ xc / n
    return out


def sign_fix(v: np.ndarray) -> np.ndarray:
    """Columns of v signed so the entry of largest magnitude (lowest row on a
    tie) is positive."""
    v = v.copy()
    for c in range(v.shape[1]):
        r = int(np.argmax(np.abs(v[:, c])))
        if v[r, c] < 0:
            v[:, c] = -v[:, c]
    return v


def pca_from_covariance(cov: np.ndarray, d_latent: int):
    """W [Hkv, d_head, d_latent] float64 (leading eigenvectors as columns) and
    their eigenvalues [Hkv, d_latent], descending."""
    hk, d, _ = cov.shape
    W = np.empty((hk, d, d_latent))
    lam = np.empty((hk, d_latent))
    for h in range(hk):
        w, v = np.linalg.eigh(cov[h])           # ascending
        order = np.argsort(-w, kind="stable")[:d_latent]
        lam[h] = w[order]
        W[h] = sign_fix(v[:, order])
    return W, lam


def pca_map(keys: np.ndarray, key_dtype: str, d_latent: int):
    """The training-free latent map of the keys: (W, eigenvalues)."""
    return pca_from_covariance(key_covariance(keys, key_dtype), d_latent)


# ----------------------------------------------------------------------------
# the index
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class IndexDesc:
    n_keys: int
    n_kv_heads: int
    d_head: int
    d_latent: int
    key_dtype: str
    latent_dtype: str
    fanout: tuple
    kmeans_iters: int
    seed: int

    @property
    def n_levels(self) -> int:
        return len(self.fanout)

    def nodes(self, level: int) -> int:
        """Nodes at ``level`` (1-based), the product of the first fanouts."""
        return int(np.prod(self.fanout[:level], dtype=np.int64))

    @staticmethod
    def of(wl) -> "IndexDesc":
        return IndexDesc(wl.n_keys, wl.n_kv_heads, wl.d_head, wl.d_latent, wl.key_dtype,
                         wl.latent_dtype, tuple(wl.fanout), wl.kmeans_iters, wl.seed)


@dataclasses.dataclass
class HeadIndex:
    W: np.ndarray            # [d_head, d_latent] fp32 values (float64)
    centroids: list          # per level [P_l, d_latent] fp32 values
    cscore: list             # per level [P_l, d_latent] latent-dtype values (scoring copy)
    offsets: list            # per level [P_l + 1] int64, CSR row ranges
    valid: list              # per level [P_l] bool, child was initialised
    perm: np.ndarray         # [N] key index of each CSR row
    csr_latent: np.ndarray   # [N, d_latent] latent of key perm[r] at row r
    assign: list             # per level [N] node id of each key (by key index)


@dataclasses.dataclass
class OracleIndex:
    desc: IndexDesc
    heads: list


def latent_keys(keys_h: np.ndarray, w_h: np.ndarray, key_dtype: str, latent_dtype: str) -> np.ndarray:
    """k~ = round_latent(k . W_h) for every key of one KV head (step 1 of
    "How does LSA work?": keys live in a latent space).  ``keys_h`` is [N, d]
    in storage format, ``w_h`` [d, d_latent] fp32."""
    k64 = stored_to_f64(keys_h, key_dtype)
    return round_latent(k64 @ w_h.astype(np.float64), latent_dtype)


def build_head(lat: np.ndarray, w_h: np.ndarray, desc: IndexDesc, h: int) -> HeadIndex:
    """Top-down hierarchy for one KV head.

    The root owns every key.  Level l splits every node of level l-1 into
    F_l children by Lloyd k-means on the node's own members; child id =
    parent_id * F_l + c.  The nodes of one level are independent, so their
    iterations run side by side here.
    """
    n, d = lat.shape
    members = [np.arange(n, dtype=np.int64)]          # node -> ascending key indices
    cents, cscores, offs, valids, assigns = [], [], [], [], []
    for lev, f in enumerate(desc.fanout, start=1):
        p_count = len(members)
        cent = np.zeros((p_count * f, d))
        valid = np.zeros(p_count * f, dtype=bool)
        node_of = np.zeros(n, dtype=np.int64)
        child_members = []
        for p, mem in enumerate(members):
            init = kmeans_init_positions(desc.seed, h, lev, p, len(mem), f)
            c_p, a_p, nv = lloyd(lat[mem], f, desc.kmeans_iters, init)
            cent[p * f:(p + 1) * f] = c_p
            valid[p * f:p * f + nv] = True
            for c in range(f):
                child_members.append(mem[a_p == c])
            node_of[mem] = p * f + a_p
        counts = np.array([len(m) for m in child_members], dtype=np.int64)
        offs.append(np.concatenate([[0], np.cumsum(counts)]))
        cents.append(cent)
        cscores.append(round_latent(cent, desc.latent_dtype))
        valids.append(valid)
        assigns.append(node_of)
        members = child_members
    perm = np.concatenate(members) if members else np.zeros(0, dtype=np.int64)
    return HeadIndex(W=w_h.astype(np.float64), centroids=cents, cscore=cscores, offsets=offs,
                     valid=valids, perm=perm, csr_latent=lat[perm], assign=assigns)


def build_index(keys: np.ndarray, W: np.ndarray, desc: IndexDesc, heads=None, progress=None,
                workers: int = 1) -> OracleIndex:
    """Index of every KV head.  ``keys`` [N, Hkv, d] storage format,
    ``W`` [Hkv, d, d_latent] fp32.  ``heads`` restricts the build to some
    heads (the others are left as None); ``workers`` builds heads in threads
    (the heads are independent)."""
    out = [None] * desc.n_kv_heads
    todo = list(range(desc.n_kv_heads) if heads is None else heads)

    def one(h):
        lat = latent_keys(keys[:, h, :], W[h], desc.key_dtype, desc.latent_dtype)
        out[h] = build_head(lat, W[h], desc, h)
        if progress:
            progress(f"oracle index head {h} built")

    if workers > 1 and len(todo) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(min(workers, len(todo))) as ex:
            list(ex.map(one, todo))
    else:
        for h in todo:
            one(h)
    return OracleIndex(desc=desc, heads=out)


# ----------------------------------------------------------------------------
# selection
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class SelectParams:
    b: int
    k: int
    sink: int
    window: int
    beam: str = "per_parent"     # or "global"

    @property
    def width(self) -> int:
        return self.sink + self.k + self.window


def segments(p: int, sink: int, window: int):
    """(sink positions, window positions, (lo, hi) of long-range candidates).

    Step 3 of "How does LSA work?": a query attends to the selected long-range
    keys plus the attention sink and a local window.  Sink = [0, min(sink, p+1));
    window = [max(sink, p-window+1), p]; candidates C(p) = [sink, p-window]
    (inclusive, empty when hi < lo), so the three parts never overlap and no
    index exceeds p.
    """
    s = list(range(0, min(sink, p + 1)))
    w = list(range(max(sink, p - window + 1), p + 1))
    return s, w, (sink, p - window)


def query_latent(q_row: np.ndarray, hidx: HeadIndex, key_dtype: str, latent_dtype: str) -> np.ndarray:
    """q~ = round_latent(q . W_h): the query enters the keys' latent space."""
    return round_latent(stored_to_f64(q_row, key_dtype) @ hidx.W, latent_dtype)


def _top_by_score(ids: np.ndarray, scores: np.ndarray, n: int) -> np.ndarray:
    """The first n of ``ids`` ordered by (score descending, id ascending)."""
    order = np.lexsort((ids, -scores))
    return ids[order[:n]]


def descend(hidx: HeadIndex, fanout: tuple, qlat: np.ndarray, b: int, beam: str) -> np.ndarray:
    """Centroid scoring and descent (step 2 of "How does LSA work?"; the
    bayesiansapien TL;DR's tree search over a few buckets).

    Level by level, the children of every kept node are scored by the inner
    product q~ . mu^ with the scoring copy of their centroid; empty children
    score -inf and are never kept.  Per-parent beam: each kept node keeps its
    top-min(b, F) children.  Global beam: the level keeps the top-b children
    over the whole frontier.  Returns the leaf ids in frontier order.
    """
    frontier = np.zeros(1, dtype=np.int64)
    for lev, f in enumerate(fanout):
        cnt = np.diff(hidx.offsets[lev])
        kids = (frontier[:, None] * f + np.arange(f)[None, :])        # [|frontier|, F]
        sc = hidx.cscore[lev][kids] @ qlat                             # [|frontier|, F]
        nonempty = cnt[kids] > 0
        if beam == "per_parent":
            new = []
            for i in range(len(frontier)):
                ids = kids[i][nonempty[i]]
                new.append(_top_by_score(ids, sc[i][nonempty[i]], min(b, f)))
            frontier = np.concatenate(new) if new else np.zeros(0, dtype=np.int64)
        elif beam == "global":
            frontier = _top_by_score(kids[nonempty], sc[nonempty], b)
        else:
            raise ValueError(beam)
    return frontier


def select_one(idx: OracleIndex, h: int, qlat: np.ndarray, p: int, prm: SelectParams, flat: bool = False,
               leaves=None, appended=None) -> dict:
    """The whole selection of one query head at position p.

    Candidates are the members of the selected leaves (all keys when ``flat``)
    that fall in C(p); each is scored s_j = q~ . k~_j; the top-k by (s desc,
    j asc) are kept (Wink Pings: after the clusters are scored, only the keys
    inside the chosen clusters are scored).  Fewer than k candidates: all of them.  ``leaves`` replaces the
    descent by a given leaf set (the key stage alone).  ``appended`` (the
    head's ``Appended`` keys) adds the keys that joined the selected leaves
    after the build, at positions N, N + 1, ...
    """
    hidx = idx.heads[h]
    _, _, (lo, hi) = segments(p, prm.sink, prm.window)
    if flat:
        leaves = None
        rows = np.arange(len(hidx.perm), dtype=np.int64)
    else:
        if leaves is None:
            leaves = descend(hidx, idx.desc.fanout, qlat, prm.b, prm.beam)
        leaves = np.asarray(leaves, dtype=np.int64)
        off = hidx.offsets[-1]
        rows = (np.concatenate([np.arange(off[c], off[c + 1]) for c in leaves])
                if len(leaves) else np.zeros(0, dtype=np.int64))
    j = hidx.perm[rows]
    keep = (j >= lo) & (j <= hi)
    rows, j = rows[keep], j[keep]
    lat = hidx.csr_latent[rows]
    if appended is not None and len(appended.leaf):
        aj = len(hidx.perm) + np.arange(len(appended.leaf), dtype=np.int64)
        mine = np.ones(len(aj), dtype=bool) if flat else np.isin(appended.leaf, leaves)
        mine &= (aj >= lo) & (aj <= hi)
        j = np.concatenate([j, aj[mine]])
        lat = np.concatenate([lat, appended.latent[mine]])
    s = lat @ qlat
    order = np.lexsort((j, -s))[:prm.k]
    top_j, top_s = j[order], s[order]
    asc = np.argsort(top_j, kind="stable")
    return dict(leaves=leaves, cand_idx=j, cand_scores=s, cand_scale=dot_scale(qlat, lat),
                top_idx=top_j[asc], top_scores=top_s[asc],
                kth=top_s[-1] if len(j) > prm.k else -np.inf)


def _row(res: dict, p: int, prm: SelectParams):
    s, w, _ = segments(p, prm.sink, prm.window)
    row = np.full(prm.width, -1, dtype=np.int32)
    row[:len(s)] = s
    row[prm.sink:prm.sink + len(res["top_idx"])] = res["top_idx"]
    row[prm.sink + prm.k:prm.sink + prm.k + len(w)] = w
    sc = np.full(prm.k, -np.inf)
    sc[:len(res["top_scores"])] = res["top_scores"]
    return row, sc


def select(idx: OracleIndex, queries: np.ndarray, q_pos: np.ndarray, prm: SelectParams,
           flat: bool = False, pairs=None, appended=None):
    """Output rows [sink | top-k (ascending index) | window], -1 padded, for
    every (token, query head), or only for the listed ``pairs``.

    Query head hq uses KV head hq // G.  ``appended`` (one ``Appended`` per KV
    head) adds keys that joined the index after its build.  Returns (rows,
    scores, leaves, results) where ``results[(t, hq)]`` keeps the per-query
    detail.
    """
    desc = idx.desc
    t_n, hq_n = queries.shape[0], queries.shape[1]
    g = hq_n // desc.n_kv_heads
    todo = pairs if pairs is not None else [(t, hq) for t in range(t_n) for hq in range(hq_n)]
    rows, scores, leaves, results = {}, {}, {}, {}
    for (t, hq) in todo:
        h = hq // g
        p = int(q_pos[t])
        qlat = query_latent(queries[t, hq], idx.heads[h], desc.key_dtype, desc.latent_dtype)
        res = select_one(idx, h, qlat, p, prm, flat=flat, appended=None if appended is None else appended[h])
        res["qlat"] = qlat
        rows[(t, hq)], scores[(t, hq)] = _row(res, p, prm)
        leaves[(t, hq)] = res["leaves"]
        results[(t, hq)] = res
    return rows, scores, leaves, results


def flat_select(idx: OracleIndex, queries, q_pos, prm: SelectParams, pairs=None, appended=None):
    """Full-scan indexer: every key of C(p) is a candidate (the quadratic path
    that scores every key, drawn dashed in the bayesiansapien flowchart)."""
    return select(idx, queries, q_pos, prm, flat=True, pairs=pairs, appended=appended)


# ----------------------------------------------------------------------------
# incremental upkeep: keys that arrive after the build
# ----------------------------------------------------------------------------
# Every decode step adds a key to the cache; the pages say the cache stays
# full length ("Gaps" on the bayesiansapien wiki) and that decode runs inside
# a captured loop ("Can I run LSA?" on wpnews), but nothing about how new
# keys enter the index.  Reading: a new key joins the tree without changing
# it.  Its latent is computed as the build computes every key's; it then
# descends from the root, at every level to the child of the current node
# whose stored (fp32) centroid is nearest in squared Euclidean distance among
# the children that hold keys, ties to the lowest child id (the build's own
# assignment rule, applied once with the centroids held fixed).  The leaf it
# reaches holds it from then on, so a query that keeps that leaf scores it.
# Centroids and earlier members do not move; re-clustering is a new build.
# The i-th key appended to a KV head sits at position N + i.


@dataclasses.dataclass
class Appended:
    latent: np.ndarray       # [A, d_latent] latent-dtype values, in arrival order
    leaf: np.ndarray         # [A] leaf id each key joined


def route_key(hidx: HeadIndex, fanout: tuple, x: np.ndarray) -> int:
    """The leaf a latent key x reaches: at every level the nearest non-empty
    child of the current node (float64 distances, ties to the lowest id)."""
    node = 0
    for lev, f in enumerate(fanout):
        kids = node * f + np.arange(f)
        nonempty = np.diff(hidx.offsets[lev])[kids] > 0
        mu = hidx.centroids[lev][kids]
        d = sq_dists(x[None, :], mu)[0]
        d[~nonempty] = np.inf
        node = int(kids[int(np.argmin(d))])
    return node


def append_keys(idx: OracleIndex, keys_new: np.ndarray, prev=None) -> list:
    """Append keys ``keys_new`` [A, Hkv, d_head] (storage format) to every KV
    head; ``prev`` holds the keys appended before (None: none).  Returns one
    ``Appended`` per head, the earlier keys first."""
    desc = idx.desc
    out = []
    for h, hidx in enumerate(idx.heads):
        lat = latent_keys(keys_new[:, h, :], hidx.W, desc.key_dtype, desc.latent_dtype)
        leaf = np.array([route_key(hidx, desc.fanout, x) for x in lat], dtype=np.int64)
        if prev is not None:
            lat = np.concatenate([prev[h].latent, lat])
            leaf = np.concatenate([prev[h].leaf, leaf])
        out.append(Appended(latent=lat, leaf=leaf))
    return out


def index_with_appended(idx: OracleIndex, appended: list) -> OracleIndex:
    """The index the appended keys define: every appended key placed in its
    leaf (after the leaf's earlier members, its position being larger), every
    level's ranges grown to match, centroids unchanged.  Selecting on it is
    what selecting with ``appended`` must give."""
    desc = idx.desc
    n0 = desc.n_keys
    heads = []
    for hidx, app in zip(idx.heads, appended):
        a = len(app.leaf)
        n_leaves = desc.nodes(desc.n_levels)
        leaf_all = np.empty(n0 + a, dtype=np.int64)
        leaf_all[hidx.perm] = np.repeat(np.arange(n_leaves), np.diff(hidx.offsets[-1]))
        leaf_all[n0:] = app.leaf
        lat_all = np.empty((n0 + a, hidx.csr_latent.shape[1]))
        lat_all[hidx.perm] = hidx.csr_latent
        lat_all[n0:] = app.latent
        perm = np.argsort(leaf_all, kind="stable")
        offs, assign = [], []
        for lev in range(1, desc.n_levels + 1):
            node_of = leaf_all // (n_leaves // desc.nodes(lev))
            offs.append(np.concatenate([[0], np.cumsum(np.bincount(node_of, minlength=desc.nodes(lev)))]))
            assign.append(node_of)
        heads.append(HeadIndex(W=hidx.W, centroids=hidx.centroids, cscore=hidx.cscore, offsets=offs,
                               valid=hidx.valid, perm=perm, csr_latent=lat_all[perm], assign=assign))
    return OracleIndex(desc=dataclasses.replace(desc, n_keys=n0 + max(len(x.leaf) for x in appended)),
                       heads=heads)


# ----------------------------------------------------------------------------
# index blob (the byte layout include/lsa.h specifies), written from the spec
# ----------------------------------------------------------------------------

DTYPE_CODE = {"f32": 0, "bf16": 1}
HEADER_BYTES = 256
BLOB_VERSION = 1


def _align256(x: int) -> int:
    return (x + 255) // 256 * 256


def blob_layout(desc: IndexDesc) -> dict:
    """Section offsets, in the order W, centroids[l], cscore[l], offsets[l],
    perm, latent; each section starts on a 256-byte boundary."""
    hk, n, dl, dh = desc.n_kv_heads, desc.n_keys, desc.d_latent, desc.d_head
    ls = 2 if desc.latent_dtype == "bf16" else 4
    cur = HEADER_BYTES
    lay = {}

    def put(name, size):
        nonlocal cur
        lay[name] = cur
        cur = _align256(cur + size)

    put("W", hk * dh * dl * 4)
    for lev in range(1, desc.n_levels + 1):
        put(f"cent{lev}", hk * desc.nodes(lev) * dl * 4)
    for lev in range(1, desc.n_levels + 1):
        put(f"cscore{lev}", hk * desc.nodes(lev) * dl * ls)
    for lev in range(1, desc.n_levels + 1):
        put(f"off{lev}", hk * (desc.nodes(lev) + 1) * 4)
    put("perm", hk * n * 4)
    put("latent", hk * n * dl * ls)
    lay["total"] = cur
    return lay


def index_blob(idx: OracleIndex) -> np.ndarray:
    """Serialise an oracle index to the blob format (uint8 array)."""
    desc = idx.desc
    lay = blob_layout(desc)
    blob = np.zeros(lay["total"], dtype=np.uint8)

    def put_bytes(off, arr):
        raw = np.ascontiguousarray(arr).view(np.uint8).ravel()
        blob[off:off + raw.size] = raw

    def lat_store(x):
        return f64_to_bf16_bits(x) if desc.latent_dtype == "bf16" else x.astype(np.float32)

    hdr = np.zeros(HEADER_BYTES, dtype=np.uint8)
    hdr[0:4] = np.frombuffer(b"LSA1", dtype=np.uint8)
    hdr[4:8] = np.array([BLOB_VERSION], dtype="<u4").view(np.uint8)
    hdr[8:16] = np.array([desc.n_keys], dtype="<i8").view(np.uint8)
    fan = list(desc.fanout) + [0] * (4 - desc.n_levels)
    i32 = [desc.n_kv_heads, desc.d_head, desc.d_latent, DTYPE_CODE[desc.key_dtype],
           DTYPE_CODE[desc.latent_dtype], desc.n_levels] + fan + [desc.kmeans_iters, 0]
    hdr[16:64] = np.array(i32, dtype="<i4").view(np.uint8)
    u64 = [desc.seed, lay["total"], lay["W"], lay["perm"], lay["latent"]]
    u64 += [lay.get(f"cent{l_}", 0) for l_ in range(1, 5)]
    u64 += [lay.get(f"cscore{l_}", 0) for l_ in range(1, 5)]
    u64 += [lay.get(f"off{l_}", 0) for l_ in range(1, 5)]
    hdr[64:64 + 8 * len(u64)] = np.array(u64, dtype="<u8").view(np.uint8)
    blob[:HEADER_BYTES] = hdr

    heads = idx.heads
    put_bytes(lay["W"], np.stack([hh.W for hh in heads]).astype(np.float32))
    for lev in range(1, desc.n_levels + 1):
        put_bytes(lay[f"cent{lev}"], np.stack([hh.centroids[lev - 1] for hh in heads]).astype(np.float32))
        put_bytes(lay[f"cscore{lev}"], lat_store(np.stack([hh.cscore[lev - 1] for hh in heads])))
        put_bytes(lay[f"off{lev}"], np.stack([hh.offsets[lev - 1] for hh in heads]).astype(np.int32))
    put_bytes(lay["perm"], np.stack([hh.perm for hh in heads]).astype(np.int32))
    put_bytes(lay["latent"], lat_store(np.stack([hh.csr_latent for hh in heads])))
    return blob


def index_from_blob(blob: np.ndarray, desc: IndexDesc) -> OracleIndex:
    """Read a blob back into oracle form (levels, perm, CSR latent).  Used to
    inspect an index's arrays; ``assign`` is derived from perm and offsets."""
    lay = blob_layout(desc)
    hk, n, dl, dh = desc.n_kv_heads, desc.n_keys, desc.d_latent, desc.d_head
    blob = np.asarray(blob, dtype=np.uint8)

    def take(name, dt, count):
        off = lay[name]
        return blob[off:off + count * np.dtype(dt).itemsize].view(dt)

    def lat_load(name, count):
        if desc.latent_dtype == "bf16":
            return bf16_bits_to_f64(take(name, np.uint16, count))
        return take(name, np.float32, count).astype(np.float64)

    W = take("W", np.float32, hk * dh * dl).reshape(hk, dh, dl)
    perm = take("perm", np.int32, hk * n).reshape(hk, n).astype(np.int64)
    lat = lat_load("latent", hk * n * dl).reshape(hk, n, dl)
    heads = []
    for h in range(hk):
        cents, cs, offs, asg = [], [], [], []
        for lev in range(1, desc.n_levels + 1):
            pn = desc.nodes(lev)
            cents.append(take(f"cent{lev}", np.float32, hk * pn * dl).reshape(hk, pn, dl)[h].astype(np.float64))
            cs.append(lat_load(f"cscore{lev}", hk * pn * dl).reshape(hk, pn, dl)[h])
            o = take(f"off{lev}", np.int32, hk * (pn + 1)).reshape(hk, pn + 1)[h].astype(np.int64)
            offs.append(o)
            node_of = np.empty(n, dtype=np.int64)
            node_of[perm[h]] = np.repeat(np.arange(pn), np.diff(o))
            asg.append(node_of)
        heads.append(HeadIndex(W=W[h].astype(np.float64), centroids=cents, cscore=cs, offsets=offs,
                               valid=[None] * desc.n_levels, perm=perm[h], csr_latent=lat[h], assign=asg))
    return OracleIndex(desc=desc, heads=heads)


def dot_scale(qlat: np.ndarray, klat: np.ndarray) -> np.ndarray:
    """sum_i |q_i k_i|: the conditioning scale of a dot product, used to state
    score tolerances relative to it."""
    return np.abs(klat) @ np.abs(qlat)

# ----------------------------------------------------------------------------
# exact sparse attention over the selected keys
# ----------------------------------------------------------------------------
# [WPN] "How does LSA work?", step 3: the query attends to the selected
# far keys the indexer chose, the sink positions and the recent window, and the
# attention kernel itself is unchanged.  So the step after the indexer is
# ordinary softmax attention restricted to the row's listed keys:
#   out = sum_j softmax_j(scale * q . k_j) v_j  over the entries j of the row
# that name a key, i.e. lie in [0, N) (anything else is padding; an entry
# listed twice counts twice; a row with no key gives zeros).


def sparse_attention(queries: np.ndarray, keys: np.ndarray, values: np.ndarray, idx: np.ndarray,
                     key_dtype: str, scale: float) -> np.ndarray:
    """queries [T, Hq, d], keys / values [N, Hkv, d] (stored, key_dtype), idx
    [T, Hq, width] int -> out [T, Hq, d] float64."""
    q = stored_to_f64(queries, key_dtype)
    k = stored_to_f64(keys, key_dtype)
    v = stored_to_f64(values, key_dtype)
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((T, Hq, d))
    for t in range(T):
        for hq in range(Hq):
            h = hq // G
            r = idx[t, hq]
            sel = r[(r >= 0) & (r < k.shape[0])]
            if sel.size == 0:
                continue
            s = scale * (k[sel, h, :] @ q[t, hq])
            w = np.exp(s - s.max())
            out[t, hq] = (w / w.sum()) @ v[sel, h, :]
    return out
