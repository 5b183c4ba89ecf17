// Device routines shared by the selection kernels of the per-query-head path
// (select.hip) and the node-major prefill path (prefill.hip): the argument
// block, the query latent, the LDS append helpers and the streaming
// gather-and-score over a query head's leaf list.
#pragma once

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {

struct SelArgs {
  const void* lat;             // [Hkv][N][DL] CSR latent
  const int* perm;             // [Hkv][N]
  int64_t N;
  int Hkv, G, Hq, T, d_head;
  const void* queries;         // [T][Hq][d_head] key dtype
  const float* W;              // [Hkv][d_head][DL]
  float* qlat;                 // [T*Hq][DL]
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
  unsigned long long* part_keys;  // [QH][part_cap] appended local top-k lists
  unsigned int* part_n;        // [QH] entries appended
  int64_t part_cap;
  unsigned long long* tau;     // [QH] sampled lower bound for the best k (0 = none)
  int32_t* out_idx;            // [QH][width]
  float* out_scores;           // [QH][k] or null
  int64_t qh0;                 // first query head of this launch
  const uint32_t* hdr;         // the blob's header
  uint32_t hx[kHeaderCheckWords];   // header words the descriptor implies
  int* status;                 // the call's device status (LSA_OK / LSA_ERR_BAD_INDEX)
  int64_t Npos;                // valid query positions: [0, Npos) (N plus the appended keys)
  const int* app_leaf;         // [Hkv][app_cap] leaf of each appended key, -1 = none (null: no pool)
  const void* app_lat;         // [Hkv][app_cap][DL] latent of each appended key
  int64_t app_cap;
  int app_n;                   // appended keys in use: positions N .. N + app_n - 1
  int* leafid;                 // [QH][nl_cap] the selected leaves, ascending (appended mode)
  // split descent (one workgroup per kept level-1 node) and its gather
  int G1;                      // level-1 nodes kept per query head = workgroups per query head
  int* slot_row;               // [QH][nl_cap] first CSR row of each leaf slot
  int* slot_n;                 // [QH][nl_cap] keys of the slot's leaf, 0 = no leaf
  int* slot_leaf;              // [QH][nl_cap] leaf id, -1 = no leaf
  unsigned int* smp;           // [QH][G1][kSplitSamples] sampled candidate score keys (0 = none)
  int* smpn;                   // [QH][G1] candidates under each kept level-1 node
};

constexpr int kSplitSamples = 64;   // threshold samples per kept level-1 node
constexpr int kSplitMaxB = 16;      // split descent: at most 16 kept level-1 nodes

// Wave-wide: does the blob's header hold the expected words hx (magic,
// version, shape fields, total size, a zero build status)?  Reads the first
// kHeaderCheckWords words of the blob and nothing else.
__device__ __forceinline__ bool header_words_match(const uint32_t* hdr, const uint32_t* hx) {
  const int lane = lane_id();
  uint32_t want = 0u;
#pragma unroll
  for (int i = 0; i < kHeaderCheckWords; ++i)
    if (lane == i) want = hx[i];
  const bool cmp = lane < kHeaderCheckWords && ((kHeaderCheckMask >> lane) & 1u);
  const uint32_t got = cmp ? hdr[lane] : want;
  return __ballot(got != want) == 0ull;
}

__device__ __forceinline__ bool header_matches(const SelArgs& a) { return header_words_match(a.hdr, a.hx); }

// Host: what the kernels of a call compare the blob's header with, and where
// the call's status word lives.
inline void set_header_check(SelArgs& a, const lsa_index_desc& d, const Layout& L, const void* index,
                             int* status) {
  const BlobHeader want = make_header(d, L);
  a.hdr = (const uint32_t*)index;
  for (int i = 0; i < kHeaderCheckWords; ++i) a.hx[i] = want.w[i];
  a.status = status;
}

// First kernel of a select call: the header check, whose result workgroup 0
// leaves in the status word for the kernels that follow.
__device__ __forceinline__ bool check_index_first(const SelArgs& a) {
  const bool ok = header_matches(a);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.status = ok ? LSA_OK : LSA_ERR_BAD_INDEX;
  return ok;
}

template <typename LT, int DL>
__device__ __forceinline__ float row_dot(const LT* row, const float* q) {
  const uint4* r = (const uint4*)row;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < DL / Lat<LT>::PER16; ++i) acc += Lat<LT>::dot16(r[i], q + i * Lat<LT>::PER16);
  return acc;
}

// q~ = round_latent(q . W_h) into q_out (LDS) and the workspace.  d_head is
// cut into kQSlices slices; thread (slice, j) sums one slice of output j and
// the slice sums are added in slice order, so every kernel that projects a
// query gets the same bits (needs blockDim >= kQSlices * DL).  qin holds
// d_head + kQSlices * DL floats of LDS.
constexpr int kQSlices = 4;

template <typename KT, typename LT, int DL>
__device__ __forceinline__ void query_latent(const SelArgs& a, int64_t qh, int h, float* qin, float* q_out) {
  const KT* qrow = (const KT*)a.queries + qh * a.d_head;
  float* part = qin + a.d_head;
  const bool pj = threadIdx.x < kQSlices * DL;
  const int j = threadIdx.x % DL, sl = threadIdx.x / DL;
  const int per = a.d_head / kQSlices;
  const float* Wh = a.W + (size_t)h * a.d_head * DL + j;
  // the first 32 weights of the thread's slice do not depend on the query:
  // their loads are issued first and overlap the query's round trip
  constexpr int kW0 = 32;
  const int n0 = per < kW0 ? per : kW0;
  float w0[kW0];
  if (pj) {
#pragma unroll
    for (int u = 0; u < kW0; ++u) w0[u] = Wh[(size_t)(sl * per + (u < n0 ? u : n0 - 1)) * DL];
  }
  for (int i = threadIdx.x; i < a.d_head; i += blockDim.x) qin[i] = KeyLoad<KT>::get(qrow, i);
  __syncthreads();
  if (pj) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kW0; ++u)
      if (u < n0) acc = fmaf(qin[sl * per + u], w0[u], acc);
    for (int i = sl * per + n0; i < (sl + 1) * per; i += 8) {   // per is a multiple of 8
      float wv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) wv[u] = Wh[(size_t)(i + u) * DL];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(qin[i + u], wv[u], acc);
    }
    part[sl * DL + j] = acc;
  }
  __syncthreads();
  if (threadIdx.x < DL) {
    float v = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < kQSlices; ++k2) v += part[k2 * DL + threadIdx.x];
    v = Lat<LT>::PER16 == 8 ? round_to_bf16(v) : v;
    q_out[threadIdx.x] = v;
    a.qlat[qh * DL + threadIdx.x] = v;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// streaming top-k helpers
// ---------------------------------------------------------------------------

// Append the keys with pred set to the LDS buffer (one LDS atomic per wave).
__device__ __forceinline__ void wave_append(bool pred, u64 key, u64* buf, int* n) {
  const u64 bal = __ballot(pred);
  if (bal == 0ull) return;
  int base = 0;
  if (lane_id() == 0) base = atomicAdd(n, __popcll(bal));
  base = __shfl(base, 0, 64);
  if (pred) buf[base + mbcnt64(bal)] = key;
}

// Append the keys with pred[u] set (up to U <= 15 per lane) with one LDS
// atomic per wave: the lane's exclusive offset comes from bit-plane ballots
// of its count.
template <int U>
__device__ __forceinline__ void wave_append_many(const bool* pred, const u64* key, u64* buf, int* n) {
  static_assert(U <= 15, "four bit planes");
  constexpr int PL = U < 2 ? 1 : U < 4 ? 2 : U < 8 ? 3 : 4;
  int c = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) c += pred[u] ? 1 : 0;
  int tot = 0, pre = 0;
#pragma unroll
  for (int b = 0; b < PL; ++b) {
    const u64 bb = __ballot((c >> b) & 1);
    tot += __popcll(bb) << b;
    pre += (int)mbcnt64(bb) << b;
  }
  if (tot == 0) return;
  int base = 0;
  if (lane_id() == 0) base = atomicAdd(n, tot);
  base = __builtin_amdgcn_readfirstlane(base);
  int pos = base + pre;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (pred[u]) buf[pos++] = key[u];
}

// Append this workgroup's n local keys to the query head's array.
template <int BLOCK>
__device__ void append_part(const SelArgs& a, int64_t qh, const u64* buf, int n, int* base_sh) {
  if (threadIdx.x == 0) *base_sh = (int)atomicAdd(&a.part_n[qh], (unsigned)n);
  __syncthreads();
  u64* dst = a.part_keys + qh * a.part_cap + *base_sh;
  for (int i = threadIdx.x; i < n; i += BLOCK) dst[i] = buf[i];
}

// ---------------------------------------------------------------------------
// gather-and-score
// ---------------------------------------------------------------------------

// The threshold of a gather, known before it starts.
struct FixedThr {
  __device__ __forceinline__ u64 operator()(u64 thr) const { return thr; }
};

// Score candidates [lo, hi) of a query head's leaf list (CSR rows of KV head
// h; lpre / lrow in LDS) and append the rank keys above thr to buf, keeping
// at most the best k when the buffer fills (streaming radix-select
// compaction).  Returns the number of keys left in buf.  The query latent is
// read from qsrc when given (visible to the block), else from a.qlat.
// `late(thr)` gives the threshold actually used; it runs once the first rows'
// loads are in flight (block-wide; it may synchronise the block), so a
// threshold computed there costs no round trip of its own.  Block-wide.
template <typename LT, int DL, int M, int U, int BLOCK, typename Late = FixedThr>
__device__ int gather_stream(const SelArgs& a, int64_t qh, int h, int clo, int chi, const int* lpre,
                             const int* lrow, int nl, int64_t lo, int64_t hi, u64 thr, u64* buf, int* n_sh,
                             RadixScratch* rs, const float* qsrc = nullptr, Late late = Late()) {
  constexpr int NW = BLOCK / 64;
  constexpr int CAP = M * BLOCK;
  constexpr int E = Lat<LT>::PER16;              // latent elements per lane load
  constexpr int LPK = DL / E;                    // lanes per key
  constexpr int KPW = 64 / LPK;                  // keys per wave per load
  constexpr int ROUND = NW * KPW * U;            // candidates per round
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  if (threadIdx.x == 0) *n_sh = 0;
  __syncthreads();
  const int64_t wlen = (hi - lo + NW - 1) / NW;
  const int64_t wlo = lo + w * wlen, whi = min(hi, wlo + wlen);
  QSlice<LT> qv;
  qv.load((qsrc ? qsrc : a.qlat + qh * DL) + lig * E);   // qsrc: the latent already in LDS
  // first leaf of this wave's range (largest i with lpre[i] <= wlo); the
  // current leaf's candidate range [cb, nb) and first row stay in registers,
  // so LDS is read only when a candidate crosses into a later leaf
  int cur = 0;
  {
    int lo_i = 0, hi_i = nl;
    while (hi_i - lo_i > 1) {
      const int mid = (lo_i + hi_i) >> 1;
      if (lpre[mid] <= wlo) lo_i = mid; else hi_i = mid;
    }
    cur = lo_i;
  }
  int cb = lpre[cur], nb = lpre[cur + 1], crow = lrow[cur];
  const LT* latb = (const LT*)a.lat + (size_t)h * a.N * DL;
  const int* permb = a.perm + (size_t)h * a.N;
  const int64_t rounds = (wlen + KPW * U - 1) / (KPW * U);
  const bool fits = hi - lo <= CAP;
  uint4 v[U], vn[U];
  int idx[U], idxn[U];
  auto fetch = [&](int64_t r, uint4* vv, int* ii) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = wlo + (r * U + u) * KPW + g;
      vv[u] = make_uint4(0u, 0u, 0u, 0u);
      ii[u] = -1;
      if (o < whi) {
        while (nb <= o) {
          ++cur;
          cb = nb;
          nb = lpre[cur + 1];
          crow = lrow[cur];
        }
        const int64_t row = crow + (o - cb);
        vv[u] = *(const uint4*)(latb + row * DL + lig * E);
        ii[u] = permb[row];
      }
    }
  };
  if (rounds > 0) fetch(0, v, idx);
  thr = late(thr);
  for (int64_t r = 0; r < rounds; ++r) {
    if (r + 1 < rounds) fetch(r + 1, vn, idxn);
    bool pr[U];
    u64 ky[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = group_sum_lead<LPK>(qv.dot(v[u]));
      const bool cand = lig == 0 && idx[u] >= clo && idx[u] <= chi;
      ky[u] = cand ? rank_key(sc, idx[u]) : 0ull;
      pr[u] = cand && ky[u] > thr;
    }
    wave_append_many<U>(pr, ky, buf, n_sh);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = vn[u];
      idx[u] = idxn[u];
    }
    if (fits) continue;          // every candidate of the range fits: no compaction
    __syncthreads();
    if (*n_sh + ROUND > CAP) {
      const int n = *n_sh;
      thr = topk_compact<BLOCK, M>(buf, n, a.k, rs);
      if (threadIdx.x == 0) *n_sh = a.k;
      __syncthreads();
    }
  }
  __syncthreads();
  return *n_sh;
}

// Appended keys: score the pool slots [s0, s1) of KV head h whose key joined
// one of the query's leaves (lid, ascending, nl of them) and whose position
// N + slot lies in [clo, chi], and append their rank keys above thr to buf
// after its first n entries, compacting to the best k when it fills.  One
// thread per slot: the 4-byte leaf ids are read for every slot, a latent row
// only for a member (few: a query keeps a small share of the leaves).  q is
// the query latent (fp32, visible to the block).  Needs CAP >= k + BLOCK.
// Returns the number of keys in buf.  Block-wide.
template <typename LT, int DL, int M, int BLOCK>
__device__ int pool_stream(const SelArgs& a, int h, int clo, int chi, const int* lid, int nl, int64_t s0,
                           int64_t s1, u64 thr, u64* buf, int n, int* n_sh, RadixScratch* rs, const float* q) {
  constexpr int CAP = M * BLOCK;
  const int* leafs = a.app_leaf + (size_t)h * a.app_cap;
  const LT* lats = (const LT*)a.app_lat + (size_t)h * a.app_cap * DL;
  __syncthreads();
  if (threadIdx.x == 0) *n_sh = n;
  for (int64_t base = s0; base < s1; base += BLOCK) {
    __syncthreads();
    if (*n_sh + BLOCK > CAP) {                 // block-uniform
      const int nn = *n_sh;
      thr = topk_compact<BLOCK, M>(buf, nn, a.k, rs);
      if (threadIdx.x == 0) *n_sh = a.k;
      __syncthreads();
    }
    const int64_t slot = base + threadIdx.x;
    bool pr = false;
    u64 key = 0ull;
    if (slot < s1) {
      const int leaf = leafs[slot];
      const int64_t j = a.N + slot;
      if (leaf >= 0 && nl > 0 && j >= clo && j <= chi) {
        int lo_i = 0, hi_i = nl;               // largest lo_i with lid[lo_i] <= leaf
        while (hi_i - lo_i > 1) {
          const int mid = (lo_i + hi_i) >> 1;
          if (lid[mid] <= leaf) lo_i = mid; else hi_i = mid;
        }
        if (lid[lo_i] == leaf) {
          key = rank_key(row_dot<LT, DL>(lats + slot * DL, q), (int)j);
          pr = key > thr;
        }
      }
    }
    wave_append(pr, key, buf, n_sh);
  }
  __syncthreads();
  return *n_sh;
}

// Over a 256-bin histogram (lane l owns bins 4l..4l+3), the bin that holds
// the need-th unit of weight counted from the top, and in *above the weight of
// the bins above it; -1 if the histogram holds less than need.  Wave-wide.
__device__ __forceinline__ int wave_find_bin(const u64* hist, u64 need, u64* above_out) {
  const int lane = threadIdx.x & 63;
  u64 hb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hb[i] = hist[4 * lane + i];
  const u64 sum = hb[0] + hb[1] + hb[2] + hb[3];
  u64 incl = sum;   // over lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 x = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += x;
  }
  const u64 above = incl - sum;
  const bool mine = above < need && need <= incl;
  int d = -1;
  u64 ab = 0ull;
  if (mine) {
    u64 acc = above;
    for (int i = 3; i >= 0; --i) {
      if (acc + hb[i] >= need) {
        d = 4 * lane + i;
        ab = acc;
        break;
      }
      acc += hb[i];
    }
  }
  const u64 bal = __ballot(mine);
  if (bal == 0ull) return -1;
  const int src = __ffsll((long long)bal) - 1;
  *above_out = __shfl(ab, src, 64);
  return __shfl(d, src, 64);
}

// Find, in a 4096-bin histogram of 12-bit digits, the bin that holds the
// need-th largest key: *d_out gets the bin, *above_out the keys in higher
// bins, *hd_out the keys in the bin.  Block-wide (BLOCK divides 4096).
template <int BLOCK>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, int* wsum, int* d_out,
                                           uint32_t* above_out, uint32_t* hd_out) {
  // thread t owns bins [4t, 4t+4); counts above a bin come from a scan that
  // runs from the highest thread down
  constexpr int PER = 4096 / BLOCK;
  const int t = threadIdx.x;
  uint32_t hb[PER];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    hb[i] = hist[t * PER + i];
    s += hb[i];
  }
  int total;
  // exclusive scan in reversed thread order = keys in bins of higher threads
  const int rev_t = BLOCK - 1 - t;
  (void)rev_t;
  const uint32_t above_t = (uint32_t)block_exclusive_scan_rev<BLOCK>((int)s, wsum, &total);
  if (above_t < need && need <= above_t + s) {
    uint32_t acc = above_t;
    for (int i = PER - 1; i >= 0; --i) {
      if (acc + hb[i] >= need) {
        *d_out = t * PER + i;
        *above_out = acc;
        *hd_out = hb[i];
        break;
      }
      acc += hb[i];
    }
  }
  __syncthreads();
}


}  // namespace lsa
