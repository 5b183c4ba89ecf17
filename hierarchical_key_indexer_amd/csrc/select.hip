// Selection for gfx950: centroid descent, gather-and-score, top-k, assembly,
// and the full-scan baseline.
//
// Steps 2 and 3 of "How does LSA work?" (page "Latent Sparse Attention (LSA):
// The 72.4x and 22.7x Speedups, and What They Compare Against"): a query
// scores the bucket centroids first, drills into the selected buckets, and
// attends to the selected long-range keys plus the attention sink and a local
// window.  The full scan is the "old indexer" of the flowchart on "Latent
// Sparse Attention: tree search over keys for 10M-token context".
//
//   descend_kernel   one workgroup per query head: level-by-level centroid
//                    dot products, wave-wide top-b per parent; leaf list with
//                    CSR row starts and candidate prefix counts
//   gather_kernel    a query head's candidates split evenly over S
//                    workgroups; 16-byte lane loads of latent rows (a row is
//                    LPK lanes), fp32 dot, causal/sink/window mask, streaming
//                    top-k in LDS (radix-select compaction)
//   merge_kernel     top-k over the S partial lists, then the output row
//   flat_kernel      full scan of one KV head's rows for its G query heads
//                    (each row read once for G heads), streaming top-k each
#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

struct SelArgs {
  const void* lat;             // [Hkv][N][DL] CSR latent
  const int* perm;             // [Hkv][N]
  int64_t N;
  int Hkv, G, Hq, T;
  const float* qlat;           // [T*Hq][DL]
  const int* q_pos;            // [T]
  int sink, window, k, width;
  const void* cscore[kMaxLevels];
  const int* off[kMaxLevels];
  int F[kMaxLevels];
  int64_t P[kMaxLevels];
  int L, b, beam, nl_cap;
  int* leafrow;                // [QH][nl_cap]
  int* leafpre;                // [QH][nl_cap+1]
  int* nleaf;                  // [QH]
  int* out_leaves;             // [QH][nl_cap] or null
  int S;                       // workgroups per query head (gather) or per (t, KV head) (flat)
  unsigned long long* part_keys;  // [QH][S][k]
  int* part_cnt;               // [QH][S]
  int32_t* out_idx;            // [QH][width]
  float* out_scores;           // [QH][k] or null
  int64_t qh0;                 // first query head of this launch
};

template <typename LT, int DL>
__device__ __forceinline__ float row_dot(const LT* row, const float* q) {
  const uint4* r = (const uint4*)row;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < DL / Lat<LT>::PER16; ++i) acc += Lat<LT>::dot16(r[i], q + i * Lat<LT>::PER16);
  return acc;
}

// ---------------------------------------------------------------------------
// descent
// ---------------------------------------------------------------------------

// Compact the non-negative entries of src[0..ns) into dst (order kept);
// returns the count.  Block-wide, 256 threads.
__device__ int compact_ids(const int* src, int ns, int* dst, int* wsum) {
  const int per = (ns + 255) / 256;
  const int i0 = min(ns, (int)threadIdx.x * per), i1 = min(ns, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += src[i] >= 0;
  int total;
  int pos = block_exclusive_scan<256>(c, wsum, &total);
  for (int i = i0; i < i1; ++i)
    if (src[i] >= 0) dst[pos++] = src[i];
  __syncthreads();
  return total;
}

template <typename LT, int DL>
__global__ __launch_bounds__(256) void descend_kernel(SelArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float q[DL];
  __shared__ int wsum[4];
  __shared__ unsigned long long wbest[4];
  int* fa = (int*)smem;                   // frontier
  int* fb = fa + a.nl_cap;                // next frontier slots
  unsigned long long* gk = (unsigned long long*)(fb + a.nl_cap + (a.nl_cap & 1));  // global beam keys

  const int64_t qh = a.qh0 + blockIdx.x;
  const int hq = (int)(qh % a.Hq);
  const int h = hq / a.G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < DL; i += 256) q[i] = a.qlat[qh * DL + i];
  if (threadIdx.x == 0) fa[0] = 0;
  __syncthreads();
  int nf = 1;
  for (int lev = 0; lev < a.L; ++lev) {
    const int F = a.F[lev];
    const LT* cs = (const LT*)a.cscore[lev] + (size_t)h * a.P[lev] * DL;
    const int* off = a.off[lev] + (size_t)h * (a.P[lev] + 1);
    if (a.beam == LSA_BEAM_PER_PARENT) {
      const int bs = min(a.b, F);
      for (int i = w; i < nf; i += 4) {
        const int par = fa[i];
        unsigned long long key[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = j * 64 + lane;
          key[j] = 0ull;
          if (c < F) {
            const int64_t node = (int64_t)par * F + c;
            if (off[node + 1] > off[node]) key[j] = rank_key(row_dot<LT, DL>(cs + node * DL, q), (int)node);
          }
        }
        int r = 0;
        for (; r < bs; ++r) {
          unsigned long long best = key[0];
#pragma unroll
          for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
          const unsigned long long wm = wave_max_u64(best);
          if (wm == 0ull) break;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key[j] == wm) key[j] = 0ull;
          if (lane == 0) fb[i * bs + r] = rank_key_index(wm);
        }
        for (int rr = r + lane; rr < bs; rr += 64) fb[i * bs + rr] = -1;
      }
      __syncthreads();
      nf = compact_ids(fb, nf * bs, fa, wsum);
    } else {
      const int ns = nf * F;
      for (int i = threadIdx.x; i < ns; i += 256) {
        const int par = fa[i / F], c = i % F;
        const int64_t node = (int64_t)par * F + c;
        gk[i] = off[node + 1] > off[node] ? rank_key(row_dot<LT, DL>(cs + node * DL, q), (int)node) : 0ull;
      }
      __syncthreads();
      int r = 0;
      for (; r < a.b; ++r) {
        unsigned long long best = 0ull;
        for (int i = threadIdx.x; i < ns; i += 256) best = gk[i] > best ? gk[i] : best;
        best = wave_max_u64(best);
        if (lane == 0) wbest[w] = best;
        __syncthreads();
        unsigned long long bm = wbest[0];
        for (int ww = 1; ww < 4; ++ww) bm = wbest[ww] > bm ? wbest[ww] : bm;
        if (bm == 0ull) break;                      // block-uniform
        for (int i = threadIdx.x; i < ns; i += 256)
          if (gk[i] == bm) gk[i] = 0ull;
        if (threadIdx.x == 0) fb[r] = rank_key_index(bm);
        __syncthreads();
      }
      for (int rr = r + threadIdx.x; rr < a.b; rr += 256) fb[rr] = -1;
      __syncthreads();
      nf = compact_ids(fb, a.b, fa, wsum);
    }
  }
  // leaf list: CSR row starts and exclusive prefix of member counts
  const int* offL = a.off[a.L - 1] + (size_t)h * (a.P[a.L - 1] + 1);
  int* lrow = a.leafrow + qh * a.nl_cap;
  int* lpre = a.leafpre + qh * (a.nl_cap + 1);
  const int per = (nf + 255) / 256;
  const int i0 = min(nf, (int)threadIdx.x * per), i1 = min(nf, i0 + per);
  int c = 0;
  for (int i = i0; i < i1; ++i) c += offL[fa[i] + 1] - offL[fa[i]];
  int total;
  int run = block_exclusive_scan<256>(c, wsum, &total);
  for (int i = i0; i < i1; ++i) {
    const int leaf = fa[i];
    lrow[i] = offL[leaf];
    lpre[i] = run;
    run += offL[leaf + 1] - offL[leaf];
  }
  if (threadIdx.x == 0) {
    lpre[nf] = total;
    a.nleaf[qh] = nf;
  }
  if (a.out_leaves) {
    int* ol = a.out_leaves + qh * a.nl_cap;
    for (int i = threadIdx.x; i < a.nl_cap; i += 256) ol[i] = i < nf ? fa[i] : -1;
  }
}

// ---------------------------------------------------------------------------
// streaming top-k helpers
// ---------------------------------------------------------------------------

// Append the keys with pred set to the LDS buffer (one LDS atomic per wave).
__device__ __forceinline__ void wave_append(bool pred, unsigned long long key, unsigned long long* buf, int* n) {
  const uint64_t bal = __ballot(pred);
  if (bal == 0ull) return;
  int base = 0;
  if (lane_id() == 0) base = atomicAdd(n, __popcll(bal));
  base = __shfl(base, 0, 64);
  if (pred) buf[base + mbcnt64(bal)] = key;
}

// ---------------------------------------------------------------------------
// gather-and-score
// ---------------------------------------------------------------------------

template <typename LT, int DL, int M, int U>
__global__ __launch_bounds__(256) void gather_kernel(SelArgs a) {
  constexpr int BLOCK = 256;
  constexpr int CAP = M * BLOCK;
  constexpr int E = Lat<LT>::PER16;              // latent elements per lane load
  constexpr int LPK = DL / E;                    // lanes per key
  constexpr int KPW = 64 / LPK;                  // keys per wave per load
  constexpr int ROUND = 4 * KPW * U;             // candidates per round
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh;
  unsigned long long* buf = (unsigned long long*)smem;
  int* lpre = (int*)(buf + CAP);
  int* lrow = lpre + a.nl_cap + 1;

  const int64_t qh = a.qh0 + blockIdx.y;
  const int s = blockIdx.x;
  const int t = (int)(qh / a.Hq), hq = (int)(qh % a.Hq), h = hq / a.G;
  const int p = a.q_pos[t];
  if (p < 0 || (int64_t)p >= a.N) {
    if (a.S > 1) {
      if (threadIdx.x == 0) a.part_cnt[qh * a.S + s] = 0;
    } else {
      write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
    }
    return;
  }
  const int clo = a.sink, chi = p - a.window;
  const int nl = a.nleaf[qh];
  for (int i = threadIdx.x; i <= nl; i += BLOCK) lpre[i] = a.leafpre[qh * (a.nl_cap + 1) + i];
  for (int i = threadIdx.x; i < nl; i += BLOCK) lrow[i] = a.leafrow[qh * a.nl_cap + i];
  if (threadIdx.x == 0) n_sh = 0;
  __syncthreads();
  const int64_t total = lpre[nl];
  const int64_t lo = total * s / a.S, hi = total * (s + 1) / a.S;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  const int64_t wlen = (hi - lo + 3) / 4;
  const int64_t wlo = lo + w * wlen, whi = min(hi, wlo + wlen);
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = a.qlat[qh * DL + lig * E + e];
  // first leaf of this wave's range (largest i with lpre[i] <= wlo)
  int cur = 0;
  {
    int lo_i = 0, hi_i = nl;   // lpre[lo_i] <= wlo < lpre[hi_i]
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (lpre[mid] <= wlo) lo_i = mid; else hi_i = mid;
    }
    cur = lo_i;
  }
  const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
  const int* permb = a.perm + (size_t)h * a.N;
  unsigned long long thr = 0ull;
  const int64_t rounds = (wlen + KPW * U - 1) / (KPW * U);
  for (int64_t r = 0; r < rounds; ++r) {
    uint4 v[U];
    int idx[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = wlo + (r * U + u) * KPW + g;
      ok[u] = o < whi;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      idx[u] = -1;
      if (ok[u]) {
        while (lpre[cur + 1] <= o) ++cur;
        const int64_t row = lrow[cur] + (o - lpre[cur]);
        v[u] = *(const uint4*)(latb + row * DL + lig * E);
        idx[u] = permb[row];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = group_sum<LPK>(Lat<LT>::dot16(v[u], qv));
      const bool cand = ok[u] && lig == LPK - 1 && idx[u] >= clo && idx[u] <= chi;
      const unsigned long long key = cand ? rank_key(sc, idx[u]) : 0ull;
      wave_append(cand && key > thr, key, buf, &n_sh);
    }
    __syncthreads();
    if (n_sh + ROUND > CAP) {
      const int n = n_sh;
      const unsigned long long t2 = topk_compact<BLOCK, M>(buf, n, a.k, &rs);
      if (threadIdx.x == 0) n_sh = a.k;
      thr = t2;
      __syncthreads();
    }
  }
  __syncthreads();
  int n = n_sh;
  if (n > a.k) {
    topk_compact<BLOCK, M>(buf, n, a.k, &rs);
    n = a.k;
  }
  if (a.S > 1) {
    unsigned long long* dst = a.part_keys + (qh * a.S + s) * (int64_t)a.k;
    for (int i = threadIdx.x; i < n; i += BLOCK) dst[i] = buf[i];
    if (threadIdx.x == 0) a.part_cnt[qh * a.S + s] = n;
  } else {
    write_selection_row<BLOCK>(buf, n, CAP, p, a.sink, a.k, a.window, a.out_idx + qh * a.width,
                               a.out_scores ? a.out_scores + qh * a.k : nullptr);
  }
}

// ---------------------------------------------------------------------------
// merge of the S partial lists of one query head
// ---------------------------------------------------------------------------

template <int M>
__global__ __launch_bounds__(256) void merge_kernel(SelArgs a) {
  constexpr int BLOCK = 256;
  constexpr int CAP = M * BLOCK;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh;
  unsigned long long* buf = (unsigned long long*)smem;
  const int64_t qh = a.qh0 + blockIdx.x;
  const int t = (int)(qh / a.Hq);
  const int p = a.q_pos[t];
  if (p < 0 || (int64_t)p >= a.N) {
    write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
    return;
  }
  if (threadIdx.x == 0) n_sh = 0;
  __syncthreads();
  unsigned long long thr = 0ull;
  for (int s = 0; s < a.S; ++s) {
    const int cnt = a.part_cnt[qh * a.S + s];
    if (n_sh + cnt > CAP) {           // block-uniform (n_sh read after a barrier)
      thr = topk_compact<BLOCK, M>(buf, n_sh, a.k, &rs);
      if (threadIdx.x == 0) n_sh = a.k;
      __syncthreads();
    }
    const unsigned long long* src = a.part_keys + (qh * a.S + s) * (int64_t)a.k;
    for (int i0 = 0; i0 < cnt; i0 += BLOCK) {
      const int i = i0 + threadIdx.x;
      const unsigned long long key = i < cnt ? src[i] : 0ull;
      wave_append(key > thr, key, buf, &n_sh);
    }
    __syncthreads();
  }
  int n = n_sh;
  if (n > a.k) {
    topk_compact<BLOCK, M>(buf, n, a.k, &rs);
    n = a.k;
  }
  write_selection_row<BLOCK>(buf, n, CAP, p, a.sink, a.k, a.window, a.out_idx + qh * a.width,
                             a.out_scores ? a.out_scores + qh * a.k : nullptr);
}

// ---------------------------------------------------------------------------
// flat full scan: rows of KV head h for its NQ = G query heads at token t
// ---------------------------------------------------------------------------

template <typename LT, int DL, int M, int U, int NQ>
__global__ __launch_bounds__(512) void flat_kernel(SelArgs a) {
  constexpr int BLOCK = 512, NW = BLOCK / 64;
  constexpr int CAP = M * BLOCK;
  constexpr int E = Lat<LT>::PER16;
  constexpr int LPK = DL / E;
  constexpr int KPW = 64 / LPK;
  constexpr int ROUND = NW * KPW * U;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh[NQ];
  unsigned long long* bufs = (unsigned long long*)smem;   // NQ x CAP

  const int s = blockIdx.x;
  const int t = blockIdx.y / a.Hkv, h = blockIdx.y % a.Hkv;
  const int p = a.q_pos[t];
  const int64_t qh_base = (int64_t)t * a.Hq + (int64_t)h * a.G;
  if (p < 0 || (int64_t)p >= a.N) {
    for (int j = 0; j < NQ; ++j) {
      const int64_t qh = qh_base + j;
      if (a.S > 1) {
        if (threadIdx.x == 0) a.part_cnt[qh * a.S + s] = 0;
      } else {
        write_invalid_row<BLOCK>(a.width, a.k, a.out_idx + qh * a.width, a.out_scores ? a.out_scores + qh * a.k : nullptr);
      }
    }
    return;
  }
  const int clo = a.sink, chi = p - a.window;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  float qv[NQ][E];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) qv[j][e] = a.qlat[(qh_base + j) * DL + lig * E + e];
  if (threadIdx.x < NQ) n_sh[threadIdx.x] = 0;
  __syncthreads();
  const int64_t lo = a.N * s / a.S, hi = a.N * (s + 1) / a.S;
  const int64_t wlen = (hi - lo + NW - 1) / NW;
  const int64_t wlo = lo + w * wlen, whi = min(hi, wlo + wlen);
  const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
  const int* permb = a.perm + (size_t)h * a.N;
  unsigned long long thr[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) thr[j] = 0ull;
  const int64_t rounds = (wlen + KPW * U - 1) / (KPW * U);
  for (int64_t r = 0; r < rounds; ++r) {
    uint4 v[U];
    int idx[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = wlo + (r * U + u) * KPW + g;
      ok[u] = row < whi;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      idx[u] = -1;
      if (ok[u]) {
        v[u] = *(const uint4*)(latb + row * DL + lig * E);
        idx[u] = permb[row];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool cand = ok[u] && lig == LPK - 1 && idx[u] >= clo && idx[u] <= chi;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const float sc = group_sum<LPK>(Lat<LT>::dot16(v[u], qv[j]));
        const unsigned long long key = cand ? rank_key(sc, idx[u]) : 0ull;
        wave_append(cand && key > thr[j], key, bufs + j * CAP, &n_sh[j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (n_sh[j] + ROUND > CAP) {
        const int n = n_sh[j];
        thr[j] = topk_compact<BLOCK, M>(bufs + j * CAP, n, a.k, &rs);
        if (threadIdx.x == 0) n_sh[j] = a.k;
        __syncthreads();
      }
    }
  }
  __syncthreads();
  for (int j = 0; j < NQ; ++j) {
    const int64_t qh = qh_base + j;
    unsigned long long* buf = bufs + j * CAP;
    int n = n_sh[j];
    if (n > a.k) {
      topk_compact<BLOCK, M>(buf, n, a.k, &rs);
      n = a.k;
    }
    if (a.S > 1) {
      unsigned long long* dst = a.part_keys + (qh * a.S + s) * (int64_t)a.k;
      for (int i = threadIdx.x; i < n; i += BLOCK) dst[i] = buf[i];
      if (threadIdx.x == 0) a.part_cnt[qh * a.S + s] = n;
    } else {
      write_selection_row<BLOCK>(buf, n, CAP, p, a.sink, a.k, a.window, a.out_idx + qh * a.width,
                                 a.out_scores ? a.out_scores + qh * a.k : nullptr);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int launch_project_queries(const lsa_index_desc& d, const void* queries, int32_t T, int32_t Hq, const float* W,
                           float* out, hipStream_t st);

namespace {

int ipow(int b, int e) {
  int r = 1;
  for (int i = 0; i < e; ++i) r *= b;
  return r;
}

// entries per thread of the streaming buffer: capacity >= 2k
int pick_m(int k, int block) {
  int m = 1;
  while (m * block < 2 * k) m <<= 1;
  return m;
}

struct SelWs {
  float* qlat;
  int* leafrow;
  int* leafpre;
  int* nleaf;
  unsigned long long* part_keys;
  int* part_cnt;
};

size_t carve_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, int32_t T,
                    int32_t Hq, bool flat, void* base, SelWs* out) {
  Carver c(base);
  SelWs w;
  const int64_t qh = (int64_t)T * Hq;
  w.qlat = c.take<float>((size_t)(qh * d.d_latent));
  w.leafrow = w.leafpre = w.nleaf = nullptr;
  if (!flat) {
    w.leafrow = c.take<int>((size_t)(qh * pl.nl_cap));
    w.leafpre = c.take<int>((size_t)(qh * (pl.nl_cap + 1)));
    w.nleaf = c.take<int>((size_t)qh);
  }
  const int S = flat ? pl.flat_splits : pl.splits;
  w.part_keys = nullptr;
  w.part_cnt = nullptr;
  if (S > 1) {
    w.part_keys = c.take<unsigned long long>((size_t)(qh * S * p.k));
    w.part_cnt = c.take<int>((size_t)(qh * S));
  }
  if (out) *out = w;
  return align_up(c.used);
}

template <typename KERNEL>
void allow_lds(KERNEL* k, size_t bytes) {
  if (bytes > 64 * 1024) (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename LT, int DL>
int run_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, const void* index,
               const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
               float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, bool flat, char* err,
               size_t errlen) {
  const Layout L = compute_layout(d);
  const char* blob = (const char*)index;
  SelWs w;
  carve_select(d, p, pl, T, Hq, flat, ws, &w);
  int rc = launch_project_queries(d, queries, T, Hq, (const float*)(blob + L.W), w.qlat, st);
  if (rc != LSA_OK) {
    snprintf(err, errlen, "query projection launch failed");
    return rc;
  }
  SelArgs a;
  memset(&a, 0, sizeof(a));
  a.lat = blob + L.latent;
  a.perm = (const int*)(blob + L.perm);
  a.N = d.n_keys;
  a.Hkv = d.n_kv_heads;
  a.G = Hq / d.n_kv_heads;
  a.Hq = Hq;
  a.T = T;
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
  a.part_cnt = w.part_cnt;
  a.out_idx = out_idx;
  a.out_scores = out_scores;
  a.qh0 = 0;
  const int64_t QH = (int64_t)T * Hq;
  const int M = pick_m(p.k, 256);

#define LSA_CHECK(what)                                                              \
  do {                                                                               \
    hipError_t e_ = hipGetLastError();                                               \
    if (e_ != hipSuccess) {                                                          \
      snprintf(err, errlen, "%s launch failed: %s", what, hipGetErrorString(e_));    \
      return LSA_ERR_HIP;                                                            \
    }                                                                                \
  } while (0)

  const int64_t chunk = 32768;   // query heads per grid (grid.y limit)
  if (!flat) {
    a.S = pl.splits;
    const size_t dlds = align_up((size_t)pl.nl_cap * 2 * 4 + 8, 16) +
                        (p.beam == LSA_BEAM_GLOBAL ? (size_t)p.b * 256 * 8 : 0);
    auto dk = descend_kernel<LT, DL>;
    allow_lds(dk, dlds);
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {
      a.qh0 = q0;
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;
      hipLaunchKernelGGL(dk, dim3((unsigned)nq), dim3(256), dlds, st, a);
    }
    LSA_CHECK("descend");
    constexpr int U = 4;
#define LSA_GATHER(MV)                                                                          \
  {                                                                                             \
    auto gk = gather_kernel<LT, DL, MV, U>;                                                     \
    const size_t glds = (size_t)MV * 256 * 8 + ((size_t)pl.nl_cap * 2 + 2) * 4;                 \
    allow_lds(gk, glds);                                                                        \
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {                                                \
      a.qh0 = q0;                                                                               \
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;                                     \
      hipLaunchKernelGGL(gk, dim3((unsigned)a.S, (unsigned)nq), dim3(256), glds, st, a);        \
    }                                                                                           \
    if (a.S > 1) {                                                                              \
      auto mk = merge_kernel<MV>;                                                               \
      const size_t mlds = (size_t)MV * 256 * 8;                                                 \
      allow_lds(mk, mlds);                                                                      \
      for (int64_t q0 = 0; q0 < QH; q0 += chunk) {                                              \
        a.qh0 = q0;                                                                             \
        const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;                                   \
        hipLaunchKernelGGL(mk, dim3((unsigned)nq), dim3(256), mlds, st, a);                     \
      }                                                                                         \
    }                                                                                           \
  }
    switch (M) {
      case 1: case 2: LSA_GATHER(2) break;
      case 4: LSA_GATHER(4) break;
      case 8: LSA_GATHER(8) break;
      case 16: LSA_GATHER(16) break;
      default: LSA_GATHER(32) break;
    }
#undef LSA_GATHER
    LSA_CHECK("gather");
    return LSA_OK;
  }
  // flat
  a.S = pl.flat_splits;
  const int G = a.G;
  const int MF = pick_m(p.k, 512);
  const int64_t TH = (int64_t)T * d.n_kv_heads;
  const int64_t fchunk = (chunk / d.n_kv_heads) * d.n_kv_heads;   // whole tokens per grid
  constexpr int UF = 4;
#define LSA_FLAT(MV, NQV)                                                                         \
  {                                                                                               \
    auto fk = flat_kernel<LT, DL, MV, UF, NQV>;                                                   \
    const size_t flds = (size_t)NQV * MV * 512 * 8;                                               \
    allow_lds(fk, flds);                                                                          \
    for (int64_t r0 = 0; r0 < TH; r0 += fchunk) {                                                 \
      const int64_t nr = TH - r0 < fchunk ? TH - r0 : fchunk;                                     \
      SelArgs b2 = a;                                                                             \
      b2.q_pos = a.q_pos + r0 / d.n_kv_heads;                                                     \
      b2.qlat = a.qlat + (r0 / d.n_kv_heads) * (int64_t)Hq * DL;                                  \
      b2.out_idx = a.out_idx + (r0 / d.n_kv_heads) * (int64_t)Hq * a.width;                       \
      b2.out_scores = a.out_scores ? a.out_scores + (r0 / d.n_kv_heads) * (int64_t)Hq * a.k : nullptr; \
      b2.part_keys = a.part_keys ? a.part_keys + (r0 / d.n_kv_heads) * (int64_t)Hq * a.S * a.k : nullptr; \
      b2.part_cnt = a.part_cnt ? a.part_cnt + (r0 / d.n_kv_heads) * (int64_t)Hq * a.S : nullptr;  \
      hipLaunchKernelGGL(fk, dim3((unsigned)a.S, (unsigned)nr), dim3(512), flds, st, b2);         \
    }                                                                                             \
  }
#define LSA_FLAT_NQ(MV)                                                        \
  switch (G) {                                                                 \
    case 1: LSA_FLAT(MV, 1) break;                                             \
    case 2: LSA_FLAT(MV, 2) break;                                             \
    case 4: LSA_FLAT(MV, 4) break;                                             \
    default: snprintf(err, errlen, "flat scan supports 1, 2 or 4 query heads per KV head"); return LSA_ERR_UNSUPPORTED; \
  }
  switch (MF) {
    case 1: LSA_FLAT_NQ(1) break;
    case 2: LSA_FLAT_NQ(2) break;
    case 4: LSA_FLAT_NQ(4) break;
    default: LSA_FLAT_NQ(8) break;
  }
#undef LSA_FLAT_NQ
#undef LSA_FLAT
  LSA_CHECK("flat scan");
  if (a.S > 1) {
#define LSA_MERGE(MV)                                                                   \
  {                                                                                     \
    auto mk = merge_kernel<MV>;                                                         \
    const size_t mlds = (size_t)MV * 256 * 8;                                           \
    allow_lds(mk, mlds);                                                                \
    for (int64_t q0 = 0; q0 < QH; q0 += chunk) {                                        \
      a.qh0 = q0;                                                                       \
      const int64_t nq = QH - q0 < chunk ? QH - q0 : chunk;                             \
      hipLaunchKernelGGL(mk, dim3((unsigned)nq), dim3(256), mlds, st, a);               \
    }                                                                                   \
  }
    switch (M) {
      case 1: case 2: LSA_MERGE(2) break;
      case 4: LSA_MERGE(4) break;
      case 8: LSA_MERGE(8) break;
      case 16: LSA_MERGE(16) break;
      default: LSA_MERGE(32) break;
    }
#undef LSA_MERGE
    LSA_CHECK("merge");
  }
  return LSA_OK;
#undef LSA_CHECK
}

}  // namespace

SelectPlan plan_select(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq, bool flat) {
  SelectPlan pl;
  pl.qh = (int64_t)T * Hq;
  pl.nl_cap = p.beam == LSA_BEAM_GLOBAL ? p.b : ipow(p.b, d.n_levels);
  const Layout L = compute_layout(d);
  const double avg_leaf = (double)d.n_keys / (double)L.nodes[d.n_levels];
  const double expect = avg_leaf * pl.nl_cap;
  int S = 1;
  if (pl.qh < 2048) {
    S = (int)((2048 + pl.qh - 1) / pl.qh);
    const int by_work = (int)(expect / 512.0);
    S = S < by_work ? S : by_work;
    S = S < 1 ? 1 : (S > 256 ? 256 : S);
  }
  pl.splits = S;
  const int64_t th = (int64_t)T * d.n_kv_heads;
  int64_t sf = (512 + th - 1) / th;
  const int64_t by_rows = d.n_keys / 4096;
  sf = sf < by_rows ? sf : by_rows;
  sf = sf < 1 ? 1 : (sf > 1024 ? 1024 : sf);
  pl.flat_splits = (int)sf;
  pl.bytes = carve_select(d, p, pl, T, Hq, flat, nullptr, nullptr);
  return pl;
}

int launch_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& pl, const void* index,
                  const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                  float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, bool flat, char* err,
                  size_t errlen) {
  const bool lb = d.latent_dtype == LSA_BF16;
  if (d.d_latent == 64) {
    if (lb) return run_select<bf16_t, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, flat, err, errlen);
    return run_select<float, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, flat, err, errlen);
  }
  if (lb) return run_select<bf16_t, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, flat, err, errlen);
  return run_select<float, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, flat, err, errlen);
}

}  // namespace lsa
