// Selection for gfx950: centroid descent, gather-and-score, top-k, assembly,
// and the full-scan baseline.
//
// Steps 2 and 3 of "How does LSA work?" (page "Latent Sparse Attention (LSA):
// The 72.4x and 22.7x Speedups, and What They Compare Against"): the query is
// compared with bucket centroids, only the winning buckets' keys are scored,
// and its row lists those keys with the sink positions and the recent window.
// The full scan is the dashed, quadratic path of the flowchart on "Latent
// Sparse Attention: tree search over keys for 10M-token context".
//
//   descend_split_kernel  decode shapes (per-parent beam, fanouts <= 64, at
//                    most 16 kept level-1 nodes): one workgroup per (kept
//                    level-1 node, query head) descends that subtree, writes
//                    its leaves into fixed slots and scores 64 samples
//   gather_split_kernel   the gather over those slots: candidates numbered in
//                    slot order, the threshold a weighted quantile of the
//                    subtrees' samples, then as gather_kernel
//   descend_kernel   other shapes, one workgroup per query head: the query's latent
//                    (round(q.W_h)), then level by level the children of every
//                    kept node are scored (one lane per child) and ranked
//                    within the wave (readlane compares); leaf list with CSR
//                    row starts and candidate prefix counts
//   gather_kernel    a query head's candidates split evenly over S
//                    workgroups; 16-byte lane loads of latent rows (a row is
//                    LPK lanes, reduced with DPP), fp32 dot, causal / sink /
//                    window mask, streaming top-k in LDS (radix-select
//                    compaction); with S > 1 the local lists are appended to
//                    one per-query-head array
//   merge_kernel     streaming top-k over that array, then the output row
//   flat_tau_kernel  query latents for the flat scan and a sampled threshold per
//                    query head (qproj_kernel: latents only, unsplit scans)
//   qproj_kernel     query latents for the flat scan
//   flat_kernel      full scan of one KV head's rows for its G query heads
//                    (each row read once for G heads), streaming top-k each
#include <limits.h>

#include <algorithm>

#include "select_device.h"

namespace lsa {

// ---------------------------------------------------------------------------
// descent
// ---------------------------------------------------------------------------

// Compact the non-negative entries of src[0..ns) into dst (order kept);
// returns the count.  Block-wide.
template <int BLOCK>
__device__ int compact_ids(const int* src, int ns, int* dst, int* wsum) {
  const int per = (ns + BLOCK - 1) / BLOCK;
  const int i0 = min(ns, (int)threadIdx.x * per), i1 = min(ns, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += src[i] >= 0;
  int total;
  int pos = block_exclusive_scan<BLOCK>(c, wsum, &total);
  for (int i = i0; i < i1; ++i)
    if (src[i] >= 0) dst[pos++] = src[i];
  __syncthreads();
  return total;
}

// compact_ids, moving the companion values ca[i], cb[i] of every kept entry
// along with it (into da, db).  Block-wide.
template <int BLOCK>
__device__ int compact_ids_with(const int* src, const int* ca, const int* cb, int ns, int* dst, int* da, int* db,
                                int* wsum) {
  const int per = (ns + BLOCK - 1) / BLOCK;
  const int i0 = min(ns, (int)threadIdx.x * per), i1 = min(ns, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += src[i] >= 0;
  int total;
  int pos = block_exclusive_scan<BLOCK>(c, wsum, &total);
  for (int i = i0; i < i1; ++i)
    if (src[i] >= 0) {
      dst[pos] = src[i];
      da[pos] = ca[i];
      db[pos] = cb[i];
      ++pos;
    }
  __syncthreads();
  return total;
}

// Mark the `need` largest of the unique nonzero keys the wave holds (J per
// lane): bit-serial radix select with ballots, from the top bit down, until
// the undecided keys are exactly the ones still needed.  in[j] gets the
// selected lanes of slot j.
template <int J>
__device__ __forceinline__ void wave_select_top(const u64* key, int need, u64* in) {
  u64 cand[J];
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    cand[j] = __ballot(key[j] != 0ull);
    in[j] = 0ull;
    ncand += __popcll(cand[j]);
  }
  if (ncand <= need) {
#pragma unroll
    for (int j = 0; j < J; ++j) in[j] = cand[j];
    return;
  }
  int remaining = need;
  for (int bit = 63; bit >= 0; --bit) {
    u64 ones[J];
    int c1 = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      ones[j] = __ballot((key[j] >> bit) & 1ull) & cand[j];
      c1 += __popcll(ones[j]);
    }
    ncand = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (c1 >= remaining) {
        cand[j] = ones[j];                   // the best `remaining` all have this bit
      } else {
        in[j] |= ones[j];                    // all of these are in
        cand[j] &= ~ones[j];
      }
      ncand += __popcll(cand[j]);
    }
    if (c1 < remaining) remaining -= c1;
    if (ncand == remaining) break;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) in[j] |= cand[j];
}

// Mark the `need` largest of the nonzero 32-bit keys the wave holds (J per
// lane; equal keys rank by slot j, then by lane): bit-serial select with
// ballots from the top bit down until the undecided keys are exactly the
// ones still needed; keys equal in all 32 bits take the lowest (j, lane).
template <int J>
__device__ __forceinline__ void wave_select_top32(const uint32_t* key, int need, u64* in) {
  u64 cand[J];
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    cand[j] = __ballot(key[j] != 0u);
    in[j] = 0ull;
    ncand += __popcll(cand[j]);
  }
  if (ncand <= need) {
#pragma unroll
    for (int j = 0; j < J; ++j) in[j] = cand[j];
    return;
  }
  int remaining = need;
  for (int bit = 31; bit >= 0 && ncand > remaining; --bit) {
    u64 ones[J];
    int c1 = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      ones[j] = __ballot((key[j] >> bit) & 1u) & cand[j];
      c1 += __popcll(ones[j]);
    }
    ncand = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (c1 >= remaining) {
        cand[j] = ones[j];                   // the best `remaining` all have this bit
      } else {
        in[j] |= ones[j];                    // all of these are in
        cand[j] &= ~ones[j];
      }
      ncand += __popcll(cand[j]);
    }
    if (c1 < remaining) remaining -= c1;
  }
  // cand: keys still tied over every bit; the first `remaining` in (j, lane) order
#pragma unroll
  for (int j = 0; j < J; ++j) {
    u64 c = cand[j];
    while (c != 0ull && remaining > 0) {
      const u64 low = c & (~c + 1ull);
      in[j] |= low;
      c ^= low;
      --remaining;
    }
  }
}

// One parent's children at a level with fanout <= 64: their scoring
// centroids are one contiguous block of rows.  LPK lanes read a row (16 bytes
// each, so a load instruction covers KPW whole rows) and reduce their partial
// dots with DPP; each lane then takes its own child's score and the wave
// ranks them.  Loads past the last child re-read the last row (its score is
// dropped), so every load is unconditional.
template <typename LT, int DL>
struct ChildBlock {
  static constexpr int E = Lat<LT>::PER16;
  static constexpr int LPK = DL / E;        // lanes per centroid row
  static constexpr int KPW = 64 / LPK;      // rows per load instruction
  static constexpr int NR = 64 / KPW;       // load rounds for up to 64 children
  uint4 v[NR];
  int o0, o1;                               // CSR range of child `lane`

  // Wave-wide: issue the loads of node `parent`'s children at level lev.
  __device__ __forceinline__ void load(const SelArgs& a, int lev, int h, int64_t parent) {
    const int lane = threadIdx.x & 63, lig = lane % LPK, g = lane / LPK;
    const int F = a.F[lev];
    const LT* cs = (const LT*)a.cscore[lev] + (size_t)h * a.P[lev] * DL;
    const int* off = a.off[lev] + (size_t)h * (a.P[lev] + 1);
    const int64_t node0 = parent * F;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = min(r * KPW + g, F - 1);
      v[r] = *(const uint4*)(cs + (node0 + c) * DL + lig * E);
    }
    const int c = min(lane, F - 1);
    o0 = off[node0 + c];
    o1 = off[node0 + c + 1];
  }

  // Wave-wide: the parent's best bs children (ties to the lower id) into
  // out[0..bs) in child order, -1 padded, and (when orow is given) each
  // kept child's first CSR row and row count into orow / ocnt at the same
  // places.  q: the query latent (LDS).
  __device__ __forceinline__ void pick(const float* q, int F, int bs, int64_t parent, int* out,
                                       int* orow = nullptr, int* ocnt = nullptr) const {
    const int lane = threadIdx.x & 63, lig = lane % LPK;
    QSlice<LT> qv;
    qv.load(q + lig * E);
    float part[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) part[r] = group_sum_lead<LPK>(qv.dot(v[r]));
    // child `lane` is row g' = lane % KPW of round lane / KPW, summed at lane g' * LPK
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float x = __shfl(part[r], (lane % KPW) * LPK, 64);
      if (lane / KPW == r) sc = x;
    }
    const uint32_t key = (lane < F && o1 > o0) ? order_u32(sc) : 0u;
    u64 in[1];
    wave_select_top32<1>(&key, bs, in);
    if ((in[0] >> lane) & 1ull) {
      const int pos = (int)mbcnt64(in[0]);
      out[pos] = (int)(parent * F + lane);
      if (orow) {
        orow[pos] = o0;
        ocnt[pos] = o1 - o0;
      }
    }
    for (int r = __popcll(in[0]) + lane; r < bs; r += 64) out[r] = -1;
  }
};

// One level of a per-parent descent with every fanout <= 64: for each parent
// fa[i] (i < nf) the best min(b, F) children go to fb[i * bs ..] in child
// order, -1 padded.  A wave loads two parents' rows before it scores either
// (bf16 rows, or fp32 rows at d_l = 32), so their round trips overlap.
// Block-wide (no barrier inside).
template <typename LT, int DL, int NW>
__device__ __forceinline__ void small_level(const SelArgs& a, int lev, int h, const float* q, const int* fa, int nf,
                                            int* fb, int* orow = nullptr, int* ocnt = nullptr) {
  using CB = ChildBlock<LT, DL>;
  const int w = threadIdx.x >> 6;
  const int F = a.F[lev];
  const int bs = min(a.b, F);
  if constexpr (CB::NR <= 8) {
    for (int i = w; i < nf; i += 2 * NW) {
      const bool two = i + NW < nf;
      CB x, y;
      x.load(a, lev, h, fa[i]);
      y.load(a, lev, h, fa[two ? i + NW : i]);
      x.pick(q, F, bs, fa[i], fb + i * bs, orow ? orow + i * bs : nullptr, ocnt ? ocnt + i * bs : nullptr);
      if (two)
        y.pick(q, F, bs, fa[i + NW], fb + (i + NW) * bs, orow ? orow + (i + NW) * bs : nullptr,
               ocnt ? ocnt + (i + NW) * bs : nullptr);
    }
  } else {
    // fp32 rows at d_l = 64: two parents' rows would not fit the registers
    for (int i = w; i < nf; i += NW) {
      CB x;
      x.load(a, lev, h, fa[i]);
      x.pick(q, F, bs, fa[i], fb + i * bs, orow ? orow + i * bs : nullptr, ocnt ? ocnt + i * bs : nullptr);
    }
  }
}

// SMALL: a per-parent beam and every fanout <= 64 (the only branch compiled
// in; the general branches would raise the register count past the budget)
template <typename KT, typename LT, int DL, int BLOCK, bool SMALL>
__global__ __launch_bounds__(BLOCK) void descend_kernel(SelArgs a) {
  constexpr int NW = BLOCK / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float qin[256 + kQSlices * DL];
  __shared__ float q[DL];
  __shared__ int wsum[NW];
  __shared__ unsigned long long wbest[NW];
  __shared__ RadixScratch rs;
  int* fa = (int*)smem;                   // frontier
  int* fb = fa + a.nl_cap;                // next frontier slots, then the leaf prefix counts
  const size_t off_gk = ((size_t)(2 * a.nl_cap + 1) * 4 + 7) / 8 * 8;
  unsigned long long* gk = (unsigned long long*)(smem + off_gk);                       // global beam keys
  unsigned long long* sk = gk + (a.beam == LSA_BEAM_GLOBAL ? (size_t)a.b * 256 : 0);   // sample keys

  const int64_t qh = a.qh0 + blockIdx.x;
  const int hq = (int)(qh % a.Hq);
  const int h = hq / a.G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (!check_index_first(a)) {               // block-uniform: nothing past the header is read
    if (a.out_leaves)
      for (int i = threadIdx.x; i < a.nl_cap; i += BLOCK) a.out_leaves[qh * a.nl_cap + i] = -1;
    return;
  }
  query_latent<KT, LT, DL>(a, qh, h, qin, q);
  if (threadIdx.x == 0) {
    fa[0] = 0;
    if (a.part_n) a.part_n[qh] = 0u;
  }
  __syncthreads();
  int nf = 1;
  for (int lev = 0; lev < a.L; ++lev) {
    const int F = a.F[lev];
    const LT* cs = (const LT*)a.cscore[lev] + (size_t)h * a.P[lev] * DL;
    const int* off = a.off[lev] + (size_t)h * (a.P[lev] + 1);
    if constexpr (SMALL) {
      small_level<LT, DL, NW>(a, lev, h, q, fa, nf, fb);
      __syncthreads();
      nf = compact_ids<BLOCK>(fb, nf * min(a.b, F), fa, wsum);
    } else if (a.beam == LSA_BEAM_PER_PARENT) {
      const int bs = min(a.b, F);
      for (int i = w; i < nf; i += NW) {
        const int par = fa[i];
        u64 key[4];
        int nne = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = j * 64 + lane;
          key[j] = 0ull;
          if (c < F) {
            const int64_t node = (int64_t)par * F + c;
            const int o0 = off[node], o1 = off[node + 1];
            const float sc = row_dot<LT, DL>(cs + node * DL, q);   // loads issued with the offsets
            if (o1 > o0) key[j] = rank_key(sc, (int)node);
          }
          nne += __popcll(__ballot(key[j] != 0ull));
        }
        // the parent's best bs children (keys are unique), kept in child order
        u64 in[4];
        wave_select_top<4>(key, bs, in);
        int slot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((in[j] >> lane) & 1ull) fb[i * bs + slot + (int)mbcnt64(in[j])] = rank_key_index(key[j]);
          slot += __popcll(in[j]);
        }
        for (int r = min(nne, bs) + lane; r < bs; r += 64) fb[i * bs + r] = -1;
      }
      __syncthreads();
      nf = compact_ids<BLOCK>(fb, nf * bs, fa, wsum);
    } else {
      const int ns = nf * F;
      for (int i = threadIdx.x; i < ns; i += BLOCK) {
        const int par = fa[i / F], c = i % F;
        const int64_t node = (int64_t)par * F + c;
        gk[i] = off[node + 1] > off[node] ? rank_key(row_dot<LT, DL>(cs + node * DL, q), (int)node) : 0ull;
      }
      __syncthreads();
      int r = 0;
      for (; r < a.b; ++r) {
        u64 best = 0ull;
        for (int i = threadIdx.x; i < ns; i += BLOCK) best = gk[i] > best ? gk[i] : best;
        best = wave_max_u64(best);
        if (lane == 0) wbest[w] = best;
        __syncthreads();
        u64 bm = wbest[0];
        for (int ww = 1; ww < NW; ++ww) bm = wbest[ww] > bm ? wbest[ww] : bm;
        if (bm == 0ull) break;                      // block-uniform
        for (int i = threadIdx.x; i < ns; i += BLOCK)
          if (gk[i] == bm) gk[i] = 0ull;
        if (threadIdx.x == 0) fb[r] = rank_key_index(bm);
        __syncthreads();
      }
      for (int rr = r + threadIdx.x; rr < a.b; rr += BLOCK) fb[rr] = -1;
      __syncthreads();
      nf = compact_ids<BLOCK>(fb, a.b, fa, wsum);
    }
  }
  if (a.leafid) {
    // the kept leaves in ascending id order (the per-parent frontier already
    // is; a global beam's is in score order: each leaf's rank is the number
    // of smaller ids, ids being distinct)
    int* lid = a.leafid + qh * a.nl_cap;
    for (int i = threadIdx.x; i < nf; i += BLOCK) {
      int rank = i;
      if (a.beam == LSA_BEAM_GLOBAL) {
        rank = 0;
        for (int j2 = 0; j2 < nf; ++j2) rank += fa[j2] < fa[i] ? 1 : 0;
      }
      lid[rank] = fa[i];
    }
    __syncthreads();
  }
  // leaf list: CSR row starts and exclusive prefix of member counts
  const int* offL = a.off[a.L - 1] + (size_t)h * (a.P[a.L - 1] + 1);
  int* lrow = a.leafrow + qh * a.nl_cap;
  int* lpre = a.leafpre + qh * (a.nl_cap + 1);
  if (a.out_leaves) {
    int* ol = a.out_leaves + qh * a.nl_cap;
    for (int i = threadIdx.x; i < a.nl_cap; i += BLOCK) ol[i] = i < nf ? fa[i] : -1;
  }
  const int per = (nf + BLOCK - 1) / BLOCK;
  const int i0 = min(nf, (int)threadIdx.x * per), i1 = min(nf, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += offL[fa[i] + 1] - offL[fa[i]];
  int total;
  int run = block_exclusive_scan<BLOCK>(c, wsum, &total);
  for (int i = i0; i < i1; ++i) {
    const int leaf = fa[i];
    const int r0 = offL[leaf];
    lrow[i] = r0;
    lpre[i] = run;
    fa[i] = r0;                 // from here on fa holds the leaves' first CSR rows
    fb[i] = run;
    run += offL[leaf + 1] - r0;
  }
  if (threadIdx.x == 0) {
    lpre[nf] = total;
    fb[nf] = total;
    a.nleaf[qh] = nf;
  }
  if (!a.tau) return;
  // Sampled threshold: score NS candidates spread evenly over the leaf list
  // and keep the r-th best sample key, r chosen so that about 2k candidates
  // are expected above it.  The gather appends only keys above this value;
  // a query head that ends with fewer than k such keys is redone without it.
  __syncthreads();
  const int t = (int)(qh / a.Hq);
  const int p = a.q_pos[t];
  u64 tau = 0ull;
  if (p >= 0 && (int64_t)p < a.Npos && (int64_t)total > 4 * (int64_t)a.k) {
    // every wave scores 64 of BLOCK evenly spaced candidates and keeps its
    // r-th best (r = expected share of 2k); tau is the median wave value
    const int64_t NS = BLOCK;
    const int r = (int)((2LL * a.k * 64 + total - 1) / total);
    const int64_t o = (int64_t)threadIdx.x * total / NS;
    int lo_i = 0, hi_i = nf;   // fb[lo_i] <= o < fb[hi_i]
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (fb[mid] <= o) lo_i = mid; else hi_i = mid;
    }
    const int row = fa[lo_i] + (int)(o - fb[lo_i]);
    const int j = a.perm[(size_t)h * a.N + row];
    // the wave's 64 sample rows are read LPK lanes per row (16-byte slices,
    // whole rows per load instruction) and the partial dots reduced with
    // DPP; lane L then takes the score of sample L
    constexpr int E = Lat<LT>::PER16, LPK = DL / E, KPW = 64 / LPK, NR = 64 / KPW;
    const int lig = lane % LPK, g = lane / LPK;
    QSlice<LT> qv;
    qv.load(q + lig * E);
    const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
    uint4 v[NR];
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const int rw = __shfl(row, rr * KPW + g, 64);
      v[rr] = *(const uint4*)(latb + (size_t)rw * DL + lig * E);
    }
    float sc = 0.f;
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const float part = group_sum_lead<LPK>(qv.dot(v[rr]));
      const float x = __shfl(part, (lane % KPW) * LPK, 64);
      if (lane / KPW == rr) sc = x;
    }
    const uint32_t key = (j >= a.sink && j <= p - a.window) ? order_u32(sc) : 0u;
    const int nvalid = __popcll(__ballot(key != 0u));
    u64 wt = 0ull;
    if (r < nvalid) {
      u64 in[1];
      wave_select_top32<1>(&key, r, in);
      // the r-th best score of the wave's samples, as the smallest rank key
      // of that score
      uint32_t m = ((in[0] >> lane) & 1ull) ? key : 0xFFFFFFFFu;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, o, 64));
      wt = (u64)m << 32;
    }
    if (lane == 0) sk[w] = wt;
    __syncthreads();
    if (w == 0) {
      // median of the NW wave values: lane i ranks value i (ties by lane)
      const u64 x = lane < NW ? sk[lane] : ~0ull;
      int rank = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const u64 o = __shfl(x, i, 64);
        rank += (o < x || (o == x && i < lane)) ? 1 : 0;
      }
      if (lane < NW && rank == (NW - 1) / 2) a.tau[qh] = x;
    }
    return;
  }
  if (threadIdx.x == 0) a.tau[qh] = tau;
}

// query latents (and a cleared append counter) for the flat scan
template <typename KT, typename LT, int DL>
__global__ __launch_bounds__(256) void qproj_kernel(SelArgs a) {
  __shared__ float qin[256 + kQSlices * DL];
  __shared__ float q[DL];
  const int64_t qh = a.qh0 + blockIdx.x;
  const int h = (int)(qh % a.Hq) / a.G;
  if (!check_index_first(a)) return;
  query_latent<KT, LT, DL>(a, qh, h, qin, q);
  if (threadIdx.x == 0 && a.part_n) a.part_n[qh] = 0u;
}

template <typename LT, int DL, int M, int U, int BLOCK>
__global__ __launch_bounds__(BLOCK) void gather_kernel(SelArgs a) {
  constexpr int CAP = M * BLOCK;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh, base_sh;
  u64* buf = (u64*)smem;
  int* lpre = (int*)(buf + CAP);
  int* lrow = lpre + a.nl_cap + 1;
  int* lid = lrow + a.nl_cap;                 // appended mode: the leaves, ascending

  __shared__ float qs[DL];
  const int64_t qh = a.qh0 + blockIdx.y;
  const int s = blockIdx.x;
  const int t = (int)(qh / a.Hq), hq = (int)(qh % a.Hq), h = hq / a.G;
  // None of these loads depends on another (the leaf lists are read to
  // their capacity, not to the list length), so they are all issued before
  // the first LDS store and share one round trip.
  const int p = a.q_pos[t];
  const int bad = *a.status;
  const int nl = a.nleaf[qh];
  const u64 thr0 = a.tau ? a.tau[qh] : 0ull;
  {
    constexpr int R = 3;
    const int np = a.nl_cap + 1;
    const int* gp = a.leafpre + qh * np;
    const int* gr = a.leafrow + qh * a.nl_cap;
    int vp[R], vr[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = threadIdx.x + j * BLOCK;
      vp[j] = i < np ? gp[i] : 0;
      vr[j] = i < a.nl_cap ? gr[i] : 0;
    }
    const float qv = threadIdx.x < DL ? a.qlat[qh * DL + threadIdx.x] : 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int i = threadIdx.x + j * BLOCK;
      if (i < np) lpre[i] = vp[j];
      if (i < a.nl_cap) lrow[i] = vr[j];
    }
    if (threadIdx.x < DL) qs[threadIdx.x] = qv;
    for (int i = threadIdx.x + R * BLOCK; i < np; i += BLOCK) lpre[i] = gp[i];
    for (int i = threadIdx.x + R * BLOCK; i < a.nl_cap; i += BLOCK) lrow[i] = gr[i];
    if (a.leafid)
      for (int i = threadIdx.x; i < a.nl_cap; i += BLOCK) lid[i] = a.leafid[qh * a.nl_cap + i];
  }
  if (bad || p < 0 || (int64_t)p >= a.Npos) {
    if (a.S == 1)
      write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
    return;
  }
  const int clo = a.sink, chi = p - a.window;
  __syncthreads();
  const int64_t total = lpre[nl];
  const int64_t lo = total * s / a.S, hi = total * (s + 1) / a.S;
  // appended keys: this workgroup's share of the pool's slots
  const int64_t plo = (int64_t)a.app_n * s / a.S, phi = (int64_t)a.app_n * (s + 1) / a.S;
  int n = gather_stream<LT, DL, M, U, BLOCK>(a, qh, h, clo, chi, lpre, lrow, nl, lo, hi, thr0, buf, &n_sh, &rs, qs);
  if (a.app_n > 0) n = pool_stream<LT, DL, M, BLOCK>(a, h, clo, chi, lid, nl, plo, phi, thr0, buf, n, &n_sh, &rs, qs);
  if (a.S == 1 && n < a.k && thr0 != 0ull) {
    // the sampled threshold let fewer than k keys through: redo without it
    n = gather_stream<LT, DL, M, U, BLOCK>(a, qh, h, clo, chi, lpre, lrow, nl, lo, hi, 0ull, buf, &n_sh, &rs, qs);
    if (a.app_n > 0) n = pool_stream<LT, DL, M, BLOCK>(a, h, clo, chi, lid, nl, plo, phi, 0ull, buf, n, &n_sh, &rs, qs);
  }
  if (a.S > 1) {
    if (n > a.k) {
      topk_compact<BLOCK, M>(buf, n, a.k, &rs);
      n = a.k;
    }
    append_part<BLOCK>(a, qh, buf, n, &base_sh);
  } else {
    write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                              a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs);
  }
}

// ---------------------------------------------------------------------------
// split descent: one workgroup per kept level-1 node of a query head
// ---------------------------------------------------------------------------

constexpr int kSplitBlock = 256;

// Workgroup (g, query head): the query latent, the root's best children (the
// same in every workgroup of the query head), then the descent below the g-th
// of them.  Its leaves fill the query head's leaf slots [g sub, (g+1) sub)
// (sub = b^(L-1), ascending ids, empty slots marked), so the slots of all the
// workgroups list the kept leaves in ascending order.  It also scores
// kSplitSamples candidates spread evenly over its own leaves (the gather
// derives its threshold from them, each sample standing for its share of the
// subtree's candidates).  Per-parent beam, fanouts <= 64.
template <typename KT, typename LT, int DL>
__global__ __launch_bounds__(kSplitBlock) void descend_split_kernel(SelArgs a) {
  constexpr int BLOCK = kSplitBlock, NW = BLOCK / 64;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float qin[256 + kQSlices * DL];
  __shared__ float q[DL];
  __shared__ int wsum[NW];
  const int sub = a.nl_cap / a.G1;
  const int nfb = max(sub, a.G1) + 1;       // the root's kept children, a level's slots, or the prefix
  int* fa = (int*)smem;                     // frontier: leaf ids at the end   [sub]
  int* fb = fa + sub;                       // next frontier slots; then the prefix of leaf sizes   [nfb]
  int* lr = fb + nfb;                       // first CSR row of each frontier node (leaf)   [sub]
  int* ln = lr + sub;                       // its row count   [sub]
  int* fr = ln + sub;                       // first CSR row of each next-frontier slot   [nfb]
  int* fc = fr + nfb;                       // its row count   [nfb]
  // (a child's CSR range comes with its centroid row, so the leaves' ranges
  // need no loads of their own)
  const int64_t qh = a.qh0 + blockIdx.y;
  const int g = blockIdx.x;
  const int hq = (int)(qh % a.Hq), h = hq / a.G, t = (int)(qh / a.Hq);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (!check_index_first(a)) return;        // block-uniform; the gather reads the status
  const int p = a.q_pos[t];
  // level 1: the root's children do not depend on the query, so wave 0 loads
  // them before the query latent (their round trip overlaps the projection's)
  ChildBlock<LT, DL> root;
  if (w == 0) root.load(a, 0, h, 0);
  query_latent<KT, LT, DL>(a, qh, h, qin, q);
  if (g == 0 && threadIdx.x == 0 && a.part_n) a.part_n[qh] = 0u;   // the gather's lists (S > 1 only)
  // the root's kept children, ascending; this workgroup takes the g-th
  if (w == 0) root.pick(q, a.F[0], min(a.b, a.F[0]), 0, fb, fr, fc);
  __syncthreads();
  const int my = fb[g];
  const int myr = fr[g], myn = fc[g];
  __syncthreads();
  int nf = 0;
  if (my >= 0) {                            // block-uniform
    if (threadIdx.x == 0) {
      fa[0] = my;
      lr[0] = myr;
      ln[0] = myn;
    }
    __syncthreads();
    nf = 1;
    for (int lev = 1; lev < a.L; ++lev) {
      small_level<LT, DL, NW>(a, lev, h, q, fa, nf, fb, fr, fc);
      __syncthreads();
      nf = compact_ids_with<BLOCK>(fb, fr, fc, nf * min(a.b, a.F[lev]), fa, lr, ln, wsum);
    }
  }
  // the leaf slots and the exclusive prefix of the leaves' sizes
  int* srow = a.slot_row + qh * a.nl_cap + (int64_t)g * sub;
  int* sn = a.slot_n + qh * a.nl_cap + (int64_t)g * sub;
  int* sleaf = a.slot_leaf + qh * a.nl_cap + (int64_t)g * sub;
  const int per = (sub + BLOCK - 1) / BLOCK;
  const int i0 = min(sub, (int)threadIdx.x * per), i1 = min(sub, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) {
    if (i < nf) {
      srow[i] = lr[i];
      sn[i] = ln[i];
      sleaf[i] = fa[i];
      c += ln[i];
    } else {
      // an empty slot repeats the workgroup's last leaf (none: past every
      // id), so the slots' leaf ids stay non-decreasing across workgroups
      srow[i] = -1;
      sn[i] = 0;
      sleaf[i] = nf > 0 ? fa[nf - 1] : INT_MAX;
    }
  }
  int ng;
  int run = block_exclusive_scan<BLOCK>(c, wsum, &ng);
  for (int i = i0; i < min(i1, nf); ++i) {
    fb[i] = run;
    run += ln[i];
  }
  if (threadIdx.x == 0) {
    fb[nf] = ng;
    a.smpn[qh * a.G1 + g] = ng;
  }
  __syncthreads();
  if (w != 0) return;
  // wave 0: the samples, lane l taking candidate l n_g / min(n_g, kSplitSamples)
  constexpr int E = Lat<LT>::PER16, LPK = DL / E, KPW = 64 / LPK, NR = 64 / KPW;
  const int ns = min(ng, kSplitSamples);
  int row = 0, j = -1;
  if (ns > 0) {
    const int o = (int)((int64_t)min(lane, ns - 1) * ng / ns);
    int lo_i = 0, hi_i = nf;                // fb[lo_i] <= o < fb[hi_i]
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (fb[mid] <= o) lo_i = mid; else hi_i = mid;
    }
    row = lr[lo_i] + (o - fb[lo_i]);
    j = a.perm[(size_t)h * a.N + row];
  }
  uint32_t key = 0u;
  if (ns > 0) {
    const int lig = lane % LPK, gg = lane / LPK;
    QSlice<LT> qv;
    qv.load(q + lig * E);
    const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
    uint4 v[NR];
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const int rw = __shfl(row, rr * KPW + gg, 64);
      v[rr] = *(const uint4*)(latb + (size_t)rw * DL + lig * E);
    }
    float sc = 0.f;
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) {
      const float part = group_sum_lead<LPK>(qv.dot(v[rr]));
      const float x = __shfl(part, (lane % KPW) * LPK, 64);
      if (lane / KPW == rr) sc = x;
    }
    const bool cand = lane < ns && p >= 0 && (int64_t)p < a.Npos && j >= a.sink && j <= p - a.window;
    key = cand ? order_u32(sc) : 0u;
  }
  a.smp[(qh * a.G1 + g) * kSplitSamples + lane] = key;
}

// LDS scratch of block_weighted_threshold.
struct ThrScratch {
  uint32_t hist[4][256];       // per-wave weighted histograms
  uint32_t lo[4], hi[4];
  int d;
  uint32_t above;
};

// Block-wide (256 threads): the largest tau such that the sample keys at or
// above it weigh at least `target`.  Thread t holds NS keys (0 = none) and
// their weights (integers: the sums are exact, so every workgroup that runs
// this on the same samples gets the same tau).  Two passes of 8-bit digits
// below the bits all the keys share, each a per-wave histogram in LDS (the
// digits spread the keys, so the atomics rarely collide), summed over the
// waves; the lower bits of tau stay 0, so the keys at or above it weigh at
// least the target.  0 when all the samples weigh less.
template <int NS>
__device__ uint32_t block_weighted_threshold(const uint32_t* key, const uint32_t* wt, uint32_t target,
                                             ThrScratch* sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (key[j] != 0u) {
      lo = min(lo, key[j]);
      hi = max(hi, key[j]);
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  if (lane == 0) {
    sc->lo[w] = lo;
    sc->hi[w] = hi;
  }
  for (int i = lane; i < 256; i += 64) sc->hist[w][i] = 0u;
  __syncthreads();
  lo = min(min(sc->lo[0], sc->lo[1]), min(sc->lo[2], sc->lo[3]));
  hi = max(max(sc->hi[0], sc->hi[1]), max(sc->hi[2], sc->hi[3]));
  if (hi == 0u) return 0u;                   // block-uniform: no sample
  const int top = lo == hi ? 0 : 32 - __clz((int)(lo ^ hi));       // bits [0, top) differ
  uint32_t mask = top >= 32 ? 0u : ~0u << top;
  uint32_t prefix = lo & mask;
  uint32_t need = target;
  for (int pass = 0, hb = top; pass < 2 && hb > 0; ++pass) {
    const int lb = hb > 8 ? hb - 8 : 0;
    const uint32_t dmask = (1u << (hb - lb)) - 1u;
    if (pass > 0) {
      for (int i = lane; i < 256; i += 64) sc->hist[w][i] = 0u;
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&sc->hist[w][(key[j] >> lb) & dmask], wt[j]);
    __syncthreads();
    {
      const uint32_t t = sc->hist[0][threadIdx.x] + sc->hist[1][threadIdx.x] + sc->hist[2][threadIdx.x] +
                         sc->hist[3][threadIdx.x];
      __syncthreads();
      sc->hist[0][threadIdx.x] = t;
    }
    __syncthreads();
    if (w == 0) {
      // lane l owns bins 4l..4l+3; weight above a bin comes from higher lanes
      const uint32_t h0 = sc->hist[0][4 * lane], h1 = sc->hist[0][4 * lane + 1], h2 = sc->hist[0][4 * lane + 2],
                     h3 = sc->hist[0][4 * lane + 3];
      const uint32_t s4 = h0 + h1 + h2 + h3;
      uint32_t incl = s4;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = (uint32_t)__shfl_down((int)incl, o, 64);
        if (lane + o < 64) incl += x;
      }
      const uint32_t above = incl - s4;
      if (lane == 0) sc->d = -1;
      if (above < need && need <= incl) {
        uint32_t acc = above;
        int d;
        if (acc + h3 >= need) d = 4 * lane + 3;
        else if ((acc += h3) + h2 >= need) d = 4 * lane + 2;
        else if ((acc += h2) + h1 >= need) d = 4 * lane + 1;
        else { acc += h1; d = 4 * lane; }
        sc->d = d;
        sc->above = acc;
      }
    }
    __syncthreads();
    const int d = sc->d;
    const uint32_t ab = sc->above;
    __syncthreads();
    if (d < 0) return pass == 0 ? 0u : prefix;    // block-uniform: less weight than the target
    prefix |= (uint32_t)d << lb;
    mask |= dmask << lb;
    need -= ab;
    hb = lb;
  }
  return prefix;
}

// The gather of the split descent.  Its first loads take the query head's
// leaf slots, the subtrees' samples and the query latent together.  The
// candidates are numbered in slot order (an empty slot is a leaf of no key),
// and the threshold is the weighted sample quantile with about 2k candidates
// expected above it: a sample of subtree g stands for
// n_g / min(n_g, kSplitSamples) candidates.  Every workgroup of the query head
// computes the same value.  The candidates are split over S workgroups as in
// gather_kernel (with S > 1 merge_kernel takes the appended lists; workgroup
// 0 leaves it the leaf list and the threshold, for its exact re-score).
template <typename LT, int DL, int M, int U, int BLOCK>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(3))) void gather_split_kernel(SelArgs a) {
  constexpr int CAP = M * BLOCK;
  constexpr int NSB = kSplitMaxB * kSplitSamples / BLOCK; // samples per thread
  constexpr int MAXPER = 4096 / BLOCK;                    // leaf slots per thread, at most
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh, base_sh;
  __shared__ int wsum[BLOCK / 64];
  __shared__ ThrScratch tsc;
  __shared__ int gsz[kSplitMaxB];
  __shared__ float qs[DL];
  u64* buf = (u64*)smem;
  int* lpre = (int*)(buf + CAP);            // [nl_cap + 1] candidates before each slot
  int* lrow = lpre + a.nl_cap + 1;          // [nl_cap] first CSR row of each slot's leaf
  int* lid = lrow + a.nl_cap;               // [nl_cap] leaf id of each slot, non-decreasing
  const int64_t qh = a.qh0 + blockIdx.y;
  const int s = blockIdx.x;
  const int t = (int)(qh / a.Hq), hq = (int)(qh % a.Hq), h = hq / a.G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nlc = a.nl_cap;
  const int per = (nlc + BLOCK - 1) / BLOCK;
  const int i0 = min(nlc, (int)threadIdx.x * per);
  const bool want_lid = a.app_n > 0 || (s == 0 && a.out_leaves);
  // the first loads, independent of one another: position, status, this
  // thread's leaf slots, (wave 0) the samples and their subtree's size, the
  // query latent
  const int p = a.q_pos[t];
  const int bad = *a.status;
  int vn[MAXPER], vr[MAXPER];
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    const int i = i0 + j;
    const bool in = j < per && i < nlc;
    vn[j] = in ? a.slot_n[qh * nlc + i] : 0;
    vr[j] = in ? a.slot_row[qh * nlc + i] : -1;
  }
  const int nsmp = a.G1 * kSplitSamples;
  uint32_t sk[NSB];
#pragma unroll
  for (int j = 0; j < NSB; ++j) {
    const int i = threadIdx.x + j * BLOCK;
    sk[j] = i < nsmp ? a.smp[qh * nsmp + i] : 0u;
  }
  const int gn = (int)threadIdx.x < a.G1 ? a.smpn[qh * a.G1 + threadIdx.x] : 0;
  const float qv = threadIdx.x < DL ? a.qlat[qh * DL + threadIdx.x] : 0.f;
  if ((int)threadIdx.x < a.G1) gsz[threadIdx.x] = gn;
  if (want_lid)
    for (int i = threadIdx.x; i < nlc; i += BLOCK) lid[i] = a.slot_leaf[qh * nlc + i];
  if (threadIdx.x < DL) qs[threadIdx.x] = qv;
  if (bad || p < 0 || (int64_t)p >= a.Npos) {   // block-uniform
    if (s == 0) {
      write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
      if (a.out_leaves)
        for (int i = threadIdx.x; i < nlc; i += BLOCK) a.out_leaves[qh * nlc + i] = -1;
    }
    return;
  }
  // candidates before each slot
  int sz = 0;
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) sz += vn[j];
  int total32;
  int run = block_exclusive_scan<BLOCK>(sz, wsum, &total32);
#pragma unroll
  for (int j = 0; j < MAXPER; ++j)
    if (j < per && i0 + j < nlc) {
      lrow[i0 + j] = vr[j];
      lpre[i0 + j] = run;
      run += vn[j];
    }
  if (threadIdx.x == 0) lpre[nlc] = total32;
  const int64_t total = total32;
  __syncthreads();
  const int nl = nlc;
  if (s == 0) {
    // the leaf list for the merge kernel's exact re-score
    for (int i = threadIdx.x; i <= nlc; i += BLOCK) a.leafpre[qh * (nlc + 1) + i] = lpre[i];
    for (int i = threadIdx.x; i < nlc; i += BLOCK) a.leafrow[qh * nlc + i] = lrow[i];
    if (a.leafid)
      for (int i = threadIdx.x; i < nlc; i += BLOCK) a.leafid[qh * nlc + i] = lid[i];
    if (threadIdx.x == 0) a.nleaf[qh] = nlc;
    if (a.out_leaves) {
      // the kept leaves, ascending, then -1
      int c = 0;
#pragma unroll
      for (int j = 0; j < MAXPER; ++j) c += vn[j] > 0 ? 1 : 0;
      int nv;
      int pos = block_exclusive_scan<BLOCK>(c, wsum, &nv);
#pragma unroll
      for (int j = 0; j < MAXPER; ++j)
        if (vn[j] > 0) a.out_leaves[qh * nlc + pos++] = lid[i0 + j];
      for (int i = nv + threadIdx.x; i < nlc; i += BLOCK) a.out_leaves[qh * nlc + i] = -1;
    }
  }
  // threshold: the weighted quantile of the samples with about 2k candidates
  // above, computed by wave 0 once the first rows' loads are in flight
  auto late = [&](u64) -> u64 {
    uint32_t tau = 0u;
    if (total > 4 * (int64_t)a.k) {          // block-uniform
      // a sample of subtree g weighs n_g / min(n_g, kSplitSamples) candidates, in 1/16 units
      uint32_t wt[NSB];
#pragma unroll
      for (int j = 0; j < NSB; ++j) {
        const int g = (int)(threadIdx.x + j * BLOCK) / kSplitSamples;
        const int ng = g < a.G1 ? gsz[g] : 0;
        const int nsg = min(ng, kSplitSamples);
        wt[j] = nsg > 0 ? (uint32_t)((uint64_t)ng * 16u / (uint64_t)nsg) : 0u;
      }
      tau = block_weighted_threshold<NSB>(sk, wt, (uint32_t)a.k * 32u, &tsc);
    }
    return (u64)tau << 32;
  };
  const int clo = a.sink, chi = p - a.window;
  const int64_t lo = total * s / a.S, hi = total * (s + 1) / a.S;
  const int64_t plo = (int64_t)a.app_n * s / a.S, phi = (int64_t)a.app_n * (s + 1) / a.S;
  u64 thr0 = 0ull;
  auto late_keep = [&](u64 t) -> u64 {
    thr0 = late(t);
    return thr0;
  };
  int n = gather_stream<LT, DL, M, U, BLOCK>(a, qh, h, clo, chi, lpre, lrow, nl, lo, hi, 0ull, buf, &n_sh, &rs, qs,
                                             late_keep);
  if (s == 0 && threadIdx.x == 0) a.tau[qh] = thr0;   // for the merge kernel's exact re-score
  if (a.app_n > 0) n = pool_stream<LT, DL, M, BLOCK>(a, h, clo, chi, lid, nl, plo, phi, thr0, buf, n, &n_sh, &rs, qs);
  int32_t* orow = a.out_idx + qh * a.width;
  float* srow = a.out_scores ? a.out_scores + qh * a.k : nullptr;
  if (a.S == 1) {
    if (n < a.k && thr0 != 0ull) {
      // the threshold let fewer than k keys through: redo without it
      n = gather_stream<LT, DL, M, U, BLOCK>(a, qh, h, clo, chi, lpre, lrow, nl, lo, hi, 0ull, buf, &n_sh, &rs, qs);
      if (a.app_n > 0) n = pool_stream<LT, DL, M, BLOCK>(a, h, clo, chi, lid, nl, plo, phi, 0ull, buf, n, &n_sh, &rs, qs);
    }
    write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, orow, srow, &rs);
    return;
  }
  if (n > a.k) {
    topk_compact<BLOCK, M>(buf, n, a.k, &rs);
    n = a.k;
  }
  append_part<BLOCK>(a, qh, buf, n, &base_sh);
}

// r-th largest of the nonzero keys[0..n) in LDS (0 if fewer than r): three
// histogram passes over 11, 11 and 10-bit digits from the top.  Block-wide.
template <int BLOCK>
__device__ uint32_t block_kth_u32(const uint32_t* keys, int n, int r, uint32_t* hist, int* dsel, uint32_t* asel) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0u, pmask = 0u, need = (uint32_t)r;
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0), nb = pass < 2 ? 2048 : 1024;
    for (int i = threadIdx.x; i < 2048; i += BLOCK) hist[i] = 0u;
    if (threadIdx.x == 0) *dsel = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += BLOCK) {
      const uint32_t v = keys[i];
      if (v != 0u && (v & pmask) == prefix) atomicAdd(&hist[(v >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns bins [32 l, 32 l + 32); counts above come from higher lanes
      uint32_t hb[32], sum = 0u;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        hb[i] = hist[32 * lane + i];
        sum += hb[i];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = (uint32_t)__shfl_down((int)incl, o, 64);
        if (lane + o < 64) incl += x;
      }
      const uint32_t above = incl - sum;
      if (above < need && need <= incl) {
        uint32_t acc = above;
        for (int i = 31; i >= 0; --i) {
          if (acc + hb[i] >= need) {
            *dsel = 32 * lane + i;
            *asel = acc;
            break;
          }
          acc += hb[i];
        }
      }
    }
    __syncthreads();
    const int d = *dsel;
    const uint32_t ab = *asel;
    __syncthreads();
    if (d < 0) return 0u;                       // fewer than r keys
    prefix |= (uint32_t)d << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= ab;
  }
  return prefix;
}

// Query latents for the full scan, and a sampled threshold per query head:
// NS rows of the KV head at a fixed stride (CSR order spreads them over every
// leaf) are scored, whole rows per load instruction; the exact r-th best
// candidate sample, r chosen so that about `target` candidates are expected
// at or above it, gives the threshold the scan appends above.  A query head
// with at most 2 target candidates takes none.
template <typename KT, typename LT, int DL>
__global__ __launch_bounds__(1024) void flat_tau_kernel(SelArgs a, int NS, int target) {
  constexpr int BLOCK = 1024, NW = BLOCK / 64;
  constexpr int E = Lat<LT>::PER16, LPK = DL / E, KPW = 64 / LPK;
  constexpr int UB = 8;                          // sample rows in flight per lane group
  extern __shared__ __align__(16) uint32_t skey[];   // [NS]
  __shared__ uint32_t hist[2048];
  __shared__ float qin[256 + kQSlices * DL];
  __shared__ float q[DL];
  __shared__ int dsel, nv_sh;
  __shared__ uint32_t asel;
  const int64_t qh = a.qh0 + blockIdx.x;
  const int h = (int)(qh % a.Hq) / a.G;
  if (!check_index_first(a)) return;
  query_latent<KT, LT, DL>(a, qh, h, qin, q);
  if (threadIdx.x == 0 && a.part_n) a.part_n[qh] = 0u;
  const int p = a.q_pos[qh / a.Hq];
  const int64_t n_cand = (p >= 0 && (int64_t)p < a.N) ? max(0, p - a.window - a.sink + 1) : 0;
  if (n_cand <= 2 * (int64_t)target) {
    if (threadIdx.x == 0) a.tau[qh] = 0ull;
    return;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  QSlice<LT> qv;
  qv.load(q + lig * E);
  const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
  const int* permb = a.perm + (size_t)h * a.N;
  const int clo = a.sink, chi = p - a.window;
  if (threadIdx.x == 0) nv_sh = 0;
  __syncthreads();
  int nv = 0;
  for (int base = w * KPW * UB; base < NS; base += NW * KPW * UB) {
    uint4 v[UB];
    int si[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      si[u] = base + u * KPW + g;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (si[u] < NS) v[u] = *(const uint4*)(latb + ((int64_t)si[u] * a.N / NS) * DL + lig * E);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const float sc = group_sum_lead<LPK>(qv.dot(v[u]));
      if (lig == 0 && si[u] < NS) {
        const int j = permb[(int64_t)si[u] * a.N / NS];
        const bool c = j >= clo && j <= chi;
        skey[si[u]] = c ? order_u32(sc) : 0u;
        nv += c ? 1 : 0;
      }
    }
  }
  atomicAdd(&nv_sh, nv);
  __syncthreads();
  const int64_t r = ((int64_t)target * nv_sh + n_cand - 1) / n_cand;
  uint32_t kth = 0u;
  if (r >= 1 && r <= nv_sh) kth = block_kth_u32<BLOCK>(skey, NS, (int)r, hist, &dsel, &asel);
  if (threadIdx.x == 0) a.tau[qh] = (u64)kth << 32;
}

// ---------------------------------------------------------------------------
// merge: streaming top-k over a query head's appended local lists
// ---------------------------------------------------------------------------

// Two histogram passes over the keys (12-bit digits of the rank key, from the
// top) find a prefix that every key of the best k reaches; one more pass
// appends only the keys at or above it, and the streaming compaction picks
// the exact best k among them.
template <typename LT, int DL, int BLOCK, int M>
__global__ __launch_bounds__(BLOCK) void merge_kernel(SelArgs a) {
  constexpr int CAP = M * BLOCK;
  constexpr int R = 8;                       // loads in flight per thread
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ uint32_t hist[4096];
  __shared__ int n_sh, d_sh;
  __shared__ uint32_t above_sh, hd_sh;
  u64* buf = (u64*)smem;
  const int64_t qh = a.qh0 + blockIdx.x;
  const int t = (int)(qh / a.Hq);
  // the list's first CAP / 2 places are loaded together with its count
  // (clamped into the query head's region of the workspace, masked by the
  // count where used), the rest once the count is known and only up to it:
  // a list usually holds about 2k keys, and loading all CAP places made the
  // first barrier wait for twice the bytes
  const u64* src = a.part_keys + qh * a.part_cap;
  u64 pre[M];
#pragma unroll
  for (int j = 0; j < M / 2; ++j) pre[j] = src[min((int64_t)threadIdx.x + (int64_t)j * BLOCK, a.part_cap - 1)];
  // these loads are independent as well: issue them together
  const int n_in = (int)a.part_n[qh];
#pragma unroll
  for (int j = M / 2; j < M; ++j) {
    const int64_t i = (int64_t)threadIdx.x + (int64_t)j * BLOCK;
    pre[j] = i < n_in ? src[min(i, a.part_cap - 1)] : 0ull;
  }
  const u64 thr0 = a.tau ? a.tau[qh] : 0ull;
  const int p = a.q_pos[t];
  const int bad = *a.status;
  if (bad || p < 0 || (int64_t)p >= a.Npos) {
    write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
    return;
  }
  if (n_in < a.k && thr0 != 0ull && !a.nleaf) {
    // full scan: the sampled threshold let fewer than k keys through; scan
    // every row of the KV head here, without it
    int* lpre = (int*)(buf + CAP);
    int* lrow = lpre + 2;
    if (threadIdx.x == 0) {
      lpre[0] = 0;
      lpre[1] = (int)a.N;
      lrow[0] = 0;
    }
    __syncthreads();
    const int h = (int)(qh % a.Hq) / a.G;
    int n = gather_stream<LT, DL, M, 4, BLOCK>(a, qh, h, a.sink, p - a.window, lpre, lrow, 1, 0, a.N, 0ull, buf,
                                               &n_sh, &rs);
    write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                              a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs);
    return;
  }
  if (n_in < a.k && thr0 != 0ull && a.nleaf) {
    // the sampled threshold let fewer than k keys through: score every
    // candidate of this query head here, without it
    int* lpre = (int*)(buf + CAP);
    int* lrow = lpre + a.nl_cap + 1;
    int* lid = lrow + a.nl_cap;
    const int nl = a.nleaf[qh];
    for (int i = threadIdx.x; i <= nl; i += BLOCK) lpre[i] = a.leafpre[qh * (a.nl_cap + 1) + i];
    for (int i = threadIdx.x; i < nl; i += BLOCK) lrow[i] = a.leafrow[qh * a.nl_cap + i];
    if (a.leafid)
      for (int i = threadIdx.x; i < nl; i += BLOCK) lid[i] = a.leafid[qh * a.nl_cap + i];
    __syncthreads();
    const int h = (int)(qh % a.Hq) / a.G;
    int n = gather_stream<LT, DL, M, 4, BLOCK>(a, qh, h, a.sink, p - a.window, lpre, lrow, nl, 0, lpre[nl], 0ull,
                                               buf, &n_sh, &rs);
    if (a.app_n > 0)
      n = pool_stream<LT, DL, M, BLOCK>(a, h, a.sink, p - a.window, lid, nl, 0, a.app_n, 0ull, buf, n, &n_sh, &rs,
                                        a.qlat + qh * DL);
    write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                              a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs);
    return;
  }
  if (n_in <= CAP) {
    // everything fits the registers, loaded above: one selection
    write_top_k_row<BLOCK, M>(buf, n_in, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                              a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs, nullptr, pre);
    return;
  }
  u64 lowest = 0ull;                         // keys below this are never needed
  if (n_in > 8 * a.k) {
    uint32_t need = (uint32_t)a.k;
    u64 prefix = 0ull;
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = 52 - 12 * pass;
      const u64 pmask = pass == 0 ? 0ull : (0xFFFull << 52);
      for (int i = threadIdx.x; i < 4096; i += BLOCK) hist[i] = 0u;
      __syncthreads();
      for (int base = 0; base < n_in; base += BLOCK * R) {
        u64 v[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int e = base + j * BLOCK + threadIdx.x;
          v[j] = e < n_in ? src[e] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (v[j] != 0ull && (v[j] & pmask) == prefix) atomicAdd(&hist[(uint32_t)(v[j] >> shift) & 0xFFFu], 1u);
      }
      __syncthreads();
      find_digit<BLOCK>(hist, need, rs.wsum, &d_sh, &above_sh, &hd_sh);
      prefix |= (u64)d_sh << shift;
      need -= above_sh;
      const bool done = hd_sh == need;
      __syncthreads();
      if (done || pass == 1) break;
    }
    lowest = prefix;                         // the best k all have key >= prefix
  }
  if (threadIdx.x == 0) n_sh = 0;
  __syncthreads();
  u64 thr = lowest == 0ull ? 0ull : lowest - 1ull;
  for (int base = 0; base < n_in; base += BLOCK * R) {
    u64 v[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int e = base + j * BLOCK + threadIdx.x;
      v[j] = e < n_in ? src[e] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      wave_append(v[j] > thr, v[j], buf, &n_sh);
      if ((j & 1) == 1) {                    // room check every two appends
        __syncthreads();
        if (n_sh + 2 * BLOCK > CAP) {
          thr = topk_compact<BLOCK, M>(buf, n_sh, a.k, &rs);
          if (threadIdx.x == 0) n_sh = a.k;
          __syncthreads();
        }
      }
    }
  }
  __syncthreads();
  int n = n_sh;
  write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                            a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs);
}

// ---------------------------------------------------------------------------
// flat full scan: rows of KV head h for its NQ = G query heads at token t
// ---------------------------------------------------------------------------

template <typename LT, int DL, int M, int U, int NQ>
__global__ __launch_bounds__(1024) void flat_kernel(SelArgs a) {
  constexpr int BLOCK = 1024, NW = BLOCK / 64;
  constexpr int CAP = M * BLOCK;
  constexpr int E = Lat<LT>::PER16;
  constexpr int LPK = DL / E;
  constexpr int KPW = 64 / LPK;
  constexpr int ROUND = NW * KPW * U;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh[NQ];
  __shared__ int base_sh;
  u64* bufs = (u64*)smem;   // NQ x CAP

  const int s = blockIdx.x;
  const int t = blockIdx.y / a.Hkv, h = blockIdx.y % a.Hkv;
  const int p = a.q_pos[t];
  const int bad = *a.status;
  const int64_t qh_base = (int64_t)t * a.Hq + (int64_t)h * a.G;
  if (bad || p < 0 || (int64_t)p >= a.N) {
    if (a.S == 1)
      for (int j = 0; j < NQ; ++j) {
        const int64_t qh = qh_base + j;
        write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
      }
    return;
  }
  const int clo = a.sink, chi = p - a.window;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  QSlice<LT> qv[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) qv[j].load(a.qlat + (qh_base + j) * DL + lig * E);
  if (threadIdx.x < NQ) n_sh[threadIdx.x] = 0;
  __syncthreads();
  const int64_t lo = a.N * s / a.S, hi = a.N * (s + 1) / a.S;
  const int64_t wlen = (hi - lo + NW - 1) / NW;
  const int64_t wlo = lo + w * wlen, whi = min(hi, wlo + wlen);
  const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
  const int* permb = a.perm + (size_t)h * a.N;
  u64 thr[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) thr[j] = a.tau ? a.tau[qh_base + j] : 0ull;
  const int64_t rounds = (wlen + KPW * U - 1) / (KPW * U);
  uint4 v[U], vn[U];
  int idx[U], idxn[U];
  auto fetch = [&](int64_t r, uint4* vv, int* ii) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = wlo + (r * U + u) * KPW + g;
      vv[u] = make_uint4(0u, 0u, 0u, 0u);
      ii[u] = -1;
      if (row < whi) {
        vv[u] = *(const uint4*)(latb + row * DL + lig * E);
        ii[u] = permb[row];
      }
    }
  };
  if (rounds > 0) fetch(0, v, idx);
  for (int64_t r = 0; r < rounds; ++r) {
    if (r + 1 < rounds) fetch(r + 1, vn, idxn);
    bool cand[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cand[u] = lig == 0 && idx[u] >= clo && idx[u] <= chi;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      bool pr[U];
      u64 ky[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float sc = group_sum_lead<LPK>(qv[j].dot(v[u]));
        ky[u] = cand[u] ? rank_key(sc, idx[u]) : 0ull;
        pr[u] = cand[u] && ky[u] > thr[j];
      }
      wave_append_many<U>(pr, ky, bufs + j * CAP, &n_sh[j]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = vn[u];
      idx[u] = idxn[u];
    }
    // the barrier of every round also keeps the waves' streams in step,
    // which reads faster than letting them drift apart
    {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        if (n_sh[j] + ROUND > CAP) {
          const int n = n_sh[j];
          const u64 t2 = topk_compact<BLOCK, M>(bufs + j * CAP, n, a.k, &rs);
          thr[j] = t2 > thr[j] ? t2 : thr[j];
          if (threadIdx.x == 0) n_sh[j] = a.k;
          __syncthreads();
        }
      }
    }
  }
  __syncthreads();
  for (int j = 0; j < NQ; ++j) {
    const int64_t qh = qh_base + j;
    u64* buf = bufs + j * CAP;
    int n = n_sh[j];
    if (a.S > 1) {
      if (n > a.k) {
        topk_compact<BLOCK, M>(buf, n, a.k, &rs);
        n = a.k;
      }
      append_part<BLOCK>(a, qh, buf, n, &base_sh);
    } else {
      write_top_k_row<BLOCK, M>(buf, n, a.k, CAP, p, a.sink, a.window, a.out_idx + qh * a.width,
                                a.out_scores ? a.out_scores + qh * a.k : nullptr, &rs);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

int ipow(int b, int e) {
  int r = 1;
  for (int i = 0; i < e; ++i) r *= b;
  return r;
}

// entries per thread of a streaming buffer whose capacity must reach `need`
int pick_m(int need, int block) {
  int m = 1;
  while (m * block < need) m <<= 1;
  return m;
}

constexpr int kMergeBlock = 1024;
constexpr int kSplitM = 8;                 // 1024-thread split buffer: 8192 keys
constexpr int kFlatU = 4;
constexpr int kFlatR = 40;                 // samples expected above a full-scan threshold

struct SelWs {
  int* status;
  int* leafid;
  int* slot_row;
  int* slot_n;
  int* slot_leaf;
  unsigned int* smp;
  int* smpn;
  float* qlat;
  int* leafrow;
  int* leafpre;
  int* nleaf;
  unsigned long long* part_keys;
  unsigned int* part_n;
  unsigned long long* tau;
};

size_t carve_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, int32_t T,
                    int32_t Hq, bool flat, void* base, SelWs* out) {
  Carver c(base);
  SelWs w;
  const int64_t qh = (int64_t)T * Hq;
  w.status = c.take<int>(64);                 // byte 0 of the workspace (lsa.h)
  w.qlat = c.take<float>((size_t)(qh * d.d_latent));
  w.leafrow = w.leafpre = w.nleaf = nullptr;
  w.leafid = nullptr;
  w.slot_row = w.slot_n = w.slot_leaf = w.smpn = nullptr;
  w.smp = nullptr;
  w.tau = nullptr;
  if (!flat && pl.g1 > 0) {
    w.slot_row = c.take<int>((size_t)(qh * pl.nl_cap));
    w.slot_n = c.take<int>((size_t)(qh * pl.nl_cap));
    w.slot_leaf = c.take<int>((size_t)(qh * pl.nl_cap));
    w.smp = c.take<unsigned int>((size_t)(qh * pl.g1 * kSplitSamples));
    w.smpn = c.take<int>((size_t)(qh * pl.g1));
    w.leafrow = c.take<int>((size_t)(qh * pl.nl_cap));
    w.leafpre = c.take<int>((size_t)(qh * (pl.nl_cap + 1)));
    w.nleaf = c.take<int>((size_t)qh);
    if (pl.appended) w.leafid = c.take<int>((size_t)(qh * pl.nl_cap));
    w.tau = c.take<unsigned long long>((size_t)qh);
  } else {
    if (!flat) {
      w.leafrow = c.take<int>((size_t)(qh * pl.nl_cap));
      w.leafpre = c.take<int>((size_t)(qh * (pl.nl_cap + 1)));
      w.nleaf = c.take<int>((size_t)qh);
      if (pl.appended) w.leafid = c.take<int>((size_t)(qh * pl.nl_cap));
    }
    w.tau = c.take<unsigned long long>((size_t)qh);
  }
  const int S = flat ? pl.flat_splits : pl.splits;
  w.part_keys = nullptr;
  w.part_n = nullptr;
  if (S > 1) {
    w.part_keys = c.take<unsigned long long>((size_t)(qh * S * p.k));
    w.part_n = c.take<unsigned int>((size_t)qh);
  }
  if (out) *out = w;
  return align_up(c.used);
}

template <typename KERNEL>
void allow_lds(KERNEL* k, size_t bytes) {
  if (bytes > 64 * 1024) (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename LT, int DL, int M>
void launch_merge(SelArgs a, int64_t QH, int64_t chunk, hipStream_t st) {
  auto mk = merge_kernel<LT, DL, kMergeBlock, M>;
  const size_t mlds = (size_t)M * kMergeBlock * 8 + ((size_t)a.nl_cap * 3 + 2) * 4;
  allow_lds(mk, mlds);
  for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
    a.qh0 = q0;
    const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
    hipLaunchKernelGGL(mk, dim3((unsigned)nq), dim3(kMergeBlock), mlds, st, a);
  }
}

// capacity >= k + four appends' room, and >= 2k so the final sort fits:
// 8 keys per thread cover every k up to kMaxK
static_assert(kMaxK + 4 * kMergeBlock <= 8 * kMergeBlock && 2 * kMaxK <= 8 * kMergeBlock, "merge capacity");
template <typename LT, int DL>
void merge_all(const SelArgs& a, int k, int64_t QH, int64_t chunk, hipStream_t st) {
  (void)k;
  launch_merge<LT, DL, 8>(a, QH, chunk, st);
}

template <typename KT, typename LT, int DL>
int run_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, const void* index,
               const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
               float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, bool flat, char* err,
               size_t errlen, const AppendView& app) {
  const Layout L = compute_layout(d);
  const char* blob = (const char*)index;
  SelWs w;
  carve_select(d, p, pl, T, Hq, flat, ws, &w);
  SelArgs a;
  memset(&a, 0, sizeof(a));
  a.lat = blob + L.latent;
  a.perm = (const int*)(blob + L.perm);
  a.N = d.n_keys;
  a.Hkv = d.n_kv_heads;
  a.G = Hq / d.n_kv_heads;
  a.Hq = Hq;
  a.T = T;
  a.d_head = d.d_head;
  a.queries = queries;
  a.W = (const float*)(blob + L.W);
  a.qlat = w.qlat;
  a.q_pos = q_pos;
  a.sink = p.sink;
  a.window = p.window;
  a.k = p.k;
  a.width = p.sink + p.k + p.window;
  a.L = d.n_levels;
  for (int l = 0; l < d.n_levels; ++l) {
    a.cscore[l] = blob + L.cscore[l];
    a.off[l] = (const int*)(blob + L.offsets[l]);
    a.F[l] = d.fanout[l];
    a.P[l] = L.nodes[l + 1];
  }
  a.b = p.b;
  a.beam = p.beam;
  a.nl_cap = pl.nl_cap;
  a.leafrow = w.leafrow;
  a.leafpre = w.leafpre;
  a.nleaf = w.nleaf;
  a.out_leaves = out_leaves;
  a.part_keys = w.part_keys;
  a.part_n = w.part_n;
  a.tau = w.tau;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  a.qh0 = 0;
  set_header_check(a, d, L, index, w.status);
  a.Npos = d.n_keys;
  a.leafid = w.leafid;
  a.G1 = pl.g1;
  a.slot_row = w.slot_row;
  a.slot_n = w.slot_n;
  a.slot_leaf = w.slot_leaf;
  a.smp = w.smp;
  a.smpn = w.smpn;
  if (app.on && app.n > 0) {
    const PoolLayout PL = pool_layout(d, app.cap);
    a.app_leaf = (const int*)((const char*)app.pool + PL.leaf);
    a.app_lat = (const char*)app.pool + PL.latent;
    a.app_cap = app.cap;
    a.app_n = app.n;
    a.Npos = d.n_keys + app.n;
  }
  const int64_t QH = (int64_t)T * Hq;

#define LSA_CHECK(what)                                                              \
  do {                                                                               \
    hipError_t e_ = hipGetLastError();                                               \
    if (e_ != hipSuccess) {                                                          \
      snprintf(err, errlen, "%s launch failed: %s", what, hipGetErrorString(e_));    \
      return LSA_ERR_HIP;                                                            \
    }                                                                                \
  } while (0)

  const int64_t chunk = 32768;   // query heads per grid (grid.y limit)
  if (!flat && pl.g1 > 0) {
    // split descent, the gather over its leaf slots, then the merge of the
    // gather's splits
    a.S = pl.splits;
    a.part_cap = (int64_t)a.S * p.k;
    const int sub = pl.nl_cap / pl.g1;
    auto dk = descend_split_kernel<KT, LT, DL>;
    const size_t dlds = ((size_t)3 * sub + 3 * ((size_t)std::max(sub, pl.g1) + 1)) * 4;
    prof_begin(LSA_STAGE_DESCEND, st);
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
      a.qh0 = q0;
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
      hipLaunchKernelGGL(dk, dim3((unsigned)pl.g1, (unsigned)nq), dim3(kSplitBlock), dlds, st, a);
    }
    prof_end(LSA_STAGE_DESCEND, st);
    LSA_CHECK("descend");
    constexpr int U = 8, GB = 256;
    const int KPWG = 64 / (DL * (int)sizeof(LT) / 16);
    const int roundg = std::max((GB / 64) * KPWG * U, GB);
    const int needg = p.k + roundg > 2 * p.k ? p.k + roundg : 2 * p.k;
    const int M = pick_m(needg, GB);
#define LSA_GATHER_SPLIT(MV)                                                                    \
  {                                                                                             \
    auto gk = gather_split_kernel<LT, DL, MV, U, GB>;                                           \
    const size_t glds = (size_t)MV * GB * 8 + ((size_t)pl.nl_cap * 3 + 2) * 4;                  \
    allow_lds(gk, glds);                                                                        \
    prof_begin(LSA_STAGE_GATHER, st);                                                           \
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {                                                \
      a.qh0 = q0;                                                                               \
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;                                     \
      hipLaunchKernelGGL(gk, dim3((unsigned)a.S, (unsigned)nq), dim3(GB), glds, st, a);         \
    }                                                                                           \
    prof_end(LSA_STAGE_GATHER, st);                                                             \
  }
    switch (M) {
      case 1: case 2: LSA_GATHER_SPLIT(2) break;
      case 4: LSA_GATHER_SPLIT(4) break;
      case 8: LSA_GATHER_SPLIT(8) break;
      case 16: LSA_GATHER_SPLIT(16) break;
      default: LSA_GATHER_SPLIT(32) break;
    }
#undef LSA_GATHER_SPLIT
    LSA_CHECK("gather");
    if (a.S > 1) {
      prof_begin(LSA_STAGE_MERGE, st);
      merge_all<LT, DL>(a, p.k, QH, chunk, st);
      prof_end(LSA_STAGE_MERGE, st);
      LSA_CHECK("merge");
    }
    return LSA_OK;
  }
  if (!flat) {
    a.S = pl.splits;
    a.part_cap = (int64_t)a.S * p.k;
    constexpr int DB = 1024;
    const size_t dlds = ((size_t)(2 * pl.nl_cap + 1) * 4 + 7) / 8 * 8 +
                        (p.beam == LSA_BEAM_GLOBAL ? (size_t)p.b * 256 * 8 : 0) + (size_t)DB * 8;
    bool small = p.beam == LSA_BEAM_PER_PARENT;
    for (int l = 0; l < d.n_levels; ++l) small = small && d.fanout[l] <= 64;
    auto dk = small ? descend_kernel<KT, LT, DL, DB, true> : descend_kernel<KT, LT, DL, DB, false>;
    allow_lds(dk, dlds);
    prof_begin(LSA_STAGE_DESCEND, st);
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
      a.qh0 = q0;
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
      hipLaunchKernelGGL(dk, dim3((unsigned)nq), dim3(DB), dlds, st, a);
    }
    prof_end(LSA_STAGE_DESCEND, st);
    LSA_CHECK("descend");
    constexpr int U = 8;
    const int GB = 256;
    const int KPWG = 64 / (DL * (int)sizeof(LT) / 16);
    // room for a round of appends above k (a round of the pool scan is one key per thread)
    const int roundg = std::max((GB / 64) * KPWG * U, GB);
    const int needg = p.k + roundg > 2 * p.k ? p.k + roundg : 2 * p.k;
    const int M = pick_m(needg, GB);
#define LSA_GATHER(MV, BV)                                                                      \
  {                                                                                             \
    auto gk = gather_kernel<LT, DL, MV, U, BV>;                                                 \
    const size_t glds = (size_t)MV * BV * 8 + ((size_t)pl.nl_cap * 3 + 2) * 4;                  \
    allow_lds(gk, glds);                                                                        \
    prof_begin(LSA_STAGE_GATHER, st);                                                           \
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {                                                \
      a.qh0 = q0;                                                                               \
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;                                     \
      hipLaunchKernelGGL(gk, dim3((unsigned)a.S, (unsigned)nq), dim3(BV), glds, st, a);         \
    }                                                                                           \
    prof_end(LSA_STAGE_GATHER, st);                                                             \
  }
    if (GB == 1024) {
      switch (M) {
        case 1: case 2: LSA_GATHER(2, 1024) break;
        case 4: LSA_GATHER(4, 1024) break;
        default: LSA_GATHER(8, 1024) break;
      }
    } else {
      switch (M) {
        case 1: case 2: LSA_GATHER(2, 256) break;
        case 4: LSA_GATHER(4, 256) break;
        case 8: LSA_GATHER(8, 256) break;
        case 16: LSA_GATHER(16, 256) break;
        default: LSA_GATHER(32, 256) break;
      }
    }
#undef LSA_GATHER
    LSA_CHECK("gather");
    if (a.S > 1) {
      prof_begin(LSA_STAGE_MERGE, st);
      merge_all<LT, DL>(a, p.k, QH, chunk, st);
      prof_end(LSA_STAGE_MERGE, st);
      LSA_CHECK("merge");
    }
    return LSA_OK;
  }
  // flat
  a.S = pl.flat_splits;
  a.part_cap = (int64_t)a.S * p.k;
  const int G = a.G;
  prof_begin(LSA_STAGE_PROJECT, st);
  if (a.S > 1) {
    // sampled thresholds: enough samples that about kFlatR of them are
    // expected above the threshold, which aims at >= 8k candidates
    int64_t ns = 2048;
    while (ns < 16384 && ns * 8 * (int64_t)p.k < (int64_t)kFlatR * d.n_keys) ns <<= 1;
    const int64_t tg = std::max<int64_t>(8 * (int64_t)p.k, ((int64_t)kFlatR * d.n_keys + ns - 1) / ns);
    const int target = (int)std::min<int64_t>(tg, (int64_t)1 << 30);
    auto tk = flat_tau_kernel<KT, LT, DL>;
    const size_t tlds = (size_t)ns * 4;
    allow_lds(tk, tlds);
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
      a.qh0 = q0;
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
      hipLaunchKernelGGL(tk, dim3((unsigned)nq), dim3(1024), tlds, st, a, (int)ns, target);
    }
  } else {
    // one workgroup per (token, KV head) writes its rows itself: no threshold
    a.tau = nullptr;
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
      a.qh0 = q0;
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
      hipLaunchKernelGGL((qproj_kernel<KT, LT, DL>), dim3((unsigned)nq), dim3(256), 0, st, a);
    }
  }
  prof_end(LSA_STAGE_PROJECT, st);
  a.qh0 = 0;
  LSA_CHECK("query projection");
  const int KPWF = 64 / (DL * (int)sizeof(LT) / 16);
  const int needf = p.k + 16 * KPWF * kFlatU > 2 * p.k ? p.k + 16 * KPWF * kFlatU : 2 * p.k;
  const int MF = pick_m(needf, 1024);
  const int64_t TH = (int64_t)T * d.n_kv_heads;
  const int64_t fchunk = (chunk / d.n_kv_heads) * d.n_kv_heads;   // whole tokens per grid
#define LSA_FLAT(MV, NQV)                                                                         \
  {                                                                                               \
    auto fk = flat_kernel<LT, DL, MV, kFlatU, NQV>;                                               \
    const size_t flds = (size_t)NQV * MV * 1024 * 8;                                              \
    if (flds > 160 * 1024) {                                                                      \
      snprintf(err, errlen, "flat scan: k = %d with %d query heads per KV head exceeds LDS", p.k, NQV); \
      return LSA_ERR_UNSUPPORTED;                                                                 \
    }                                                                                             \
    allow_lds(fk, flds);                                                                          \
    for (int64_t r0 = 0; r0 < TH; r0 += fchunk) {                                                 \
      const int64_t nr = TH - r0 < fchunk ? TH - r0 : fchunk;                                     \
      SelArgs b2 = a;                                                                             \
      const int64_t t0 = r0 / d.n_kv_heads;                                                       \
      b2.q_pos = a.q_pos + t0;                                                                    \
      b2.qlat = a.qlat + t0 * (int64_t)Hq * DL;                                                   \
      b2.out_idx = a.out_idx + t0 * (int64_t)Hq * a.width;                                        \
      b2.out_scores = a.out_scores ? a.out_scores + t0 * (int64_t)Hq * a.k : nullptr;             \
      b2.part_keys = a.part_keys ? a.part_keys + t0 * (int64_t)Hq * a.part_cap : nullptr;         \
      b2.part_n = a.part_n ? a.part_n + t0 * (int64_t)Hq : nullptr;                               \
      hipLaunchKernelGGL(fk, dim3((unsigned)a.S, (unsigned)nr), dim3(1024), flds, st, b2);        \
    }                                                                                             \
  }
#define LSA_FLAT_NQ(MV)                                                        \
  switch (G) {                                                                 \
    case 1: LSA_FLAT(MV, 1) break;                                             \
    case 2: LSA_FLAT(MV, 2) break;                                             \
    case 4: LSA_FLAT(MV, 4) break;                                             \
    default: snprintf(err, errlen, "flat scan supports 1, 2 or 4 query heads per KV head"); return LSA_ERR_UNSUPPORTED; \
  }
  prof_begin(LSA_STAGE_FLAT, st);
  switch (MF) {
    case 1: LSA_FLAT_NQ(1) break;
    case 2: LSA_FLAT_NQ(2) break;
    case 4: LSA_FLAT_NQ(4) break;
    default: LSA_FLAT_NQ(8) break;
  }
  prof_end(LSA_STAGE_FLAT, st);
#undef LSA_FLAT_NQ
#undef LSA_FLAT
  LSA_CHECK("flat scan");
  if (a.S > 1) {
    prof_begin(LSA_STAGE_MERGE, st);
    merge_all<LT, DL>(a, p.k, QH, chunk, st);
    prof_end(LSA_STAGE_MERGE, st);
    LSA_CHECK("merge");
  }
  return LSA_OK;
#undef LSA_CHECK
}

}  // namespace

SelectPlan plan_select(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq, bool flat,
                       bool appended) {
  SelectPlan pl;
  pl.qh = (int64_t)T * Hq;
  pl.appended = appended && !flat;
  pl.nl_cap = p.beam == LSA_BEAM_GLOBAL ? p.b : ipow(p.b, d.n_levels);
  const Layout L = compute_layout(d);
  const double avg_leaf = (double)d.n_keys / (double)L.nodes[d.n_levels];
  const double expect = avg_leaf * pl.nl_cap;
  // few query heads: split each over S workgroups so that the grid is one
  // round of resident workgroups (the 256-thread gather holds 3 per CU: 768
  // on 256 CUs; a fourth would run alone in a second round), each with at
  // least 512 candidates; the sampled threshold keeps every split's append
  // list short
  int S = 1;
  if (pl.qh < 768) {
    S = (int)((768 + pl.qh - 1) / pl.qh);
    const int by_work = (int)(expect / 512.0);
    S = S < by_work ? S : by_work;
    S = S < 1 ? 1 : (S > 64 ? 64 : S);
  }
  pl.splits = S;
  // split descent: per-parent beam, fanouts <= 64, at most kSplitMaxB kept
  // level-1 nodes (one workgroup each); not for the node-major path
  pl.g1 = 0;
  if (!flat && p.beam == LSA_BEAM_PER_PARENT && p.b <= kSplitMaxB) {
    bool ok = true;
    for (int l = 0; l < d.n_levels; ++l) ok = ok && d.fanout[l] <= 64;
    if (ok) pl.g1 = p.b;
  }
  const int64_t th = (int64_t)T * d.n_kv_heads;
  int64_t sf = (256 + th - 1) / th;
  const int64_t by_rows = d.n_keys / 8192;
  sf = sf < by_rows ? sf : by_rows;
  sf = sf < 1 ? 1 : (sf > 1024 ? 1024 : sf);
  pl.flat_splits = (int)sf;
  pl.bytes = carve_select(d, p, pl, T, Hq, flat, nullptr, nullptr);
  memset(&pl.pf, 0, sizeof(pl.pf));
  memset(&pl.fs, 0, sizeof(pl.fs));
  if (!flat && !pl.appended) {
    pl.pf = plan_prefill(d, p, T, Hq);
    if (pl.pf.ok) {
      pl.bytes = pl.pf.bytes;
      pl.g1 = 0;
    }
  } else if (flat) {
    pl.fs = plan_flat_tiled(d, p, T, Hq);
    if (pl.fs.ok) pl.bytes = pl.fs.bytes;
  }
  return pl;
}

int launch_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, const void* index,
                  const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                  float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, bool flat, char* err,
                  size_t errlen, const AppendView& app) {
  if (!flat && pl.pf.ok)
    return launch_prefill(d, p, pl.pf, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, err, errlen);
  if (flat && pl.fs.ok)
    return launch_flat_tiled(d, p, pl.fs, index, queries, q_pos, T, Hq, out_idx, out_scores, ws, st, err, errlen);
  const bool kb = d.key_dtype == LSA_BF16, lb = d.latent_dtype == LSA_BF16;
#define LSA_RUN(KT, LT, DLV) \
  return run_select<KT, LT, DLV>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, flat, err, errlen, app)
  if (d.d_latent == 64) {
    if (kb && lb) LSA_RUN(bf16_t, bf16_t, 64);
    if (kb) LSA_RUN(bf16_t, float, 64);
    if (lb) LSA_RUN(float, bf16_t, 64);
    LSA_RUN(float, float, 64);
  }
  if (kb && lb) LSA_RUN(bf16_t, bf16_t, 32);
  if (kb) LSA_RUN(bf16_t, float, 32);
  if (lb) LSA_RUN(float, bf16_t, 32);
  LSA_RUN(float, float, 32);
#undef LSA_RUN
}

}  // namespace lsa
