// Node-major selection for large query batches (prefill chunks) on gfx950.
//
// Same result as the per-query-head path of select.hip (steps 2 and 3 of "How
// does LSA work?" on the page "Latent Sparse Attention (LSA): The 72.4x and
// 22.7x Speedups, and What They Compare Against": score the bucket centroids,
// keep the best buckets level by level, score the keys of the kept leaves,
// keep the best k), computed the other way round: every tree node is visited
// once per call with all the query heads that kept its parent, so a node's
// children (and a leaf's keys) are read once per batch instead of once per
// query head, and the scores come from bf16 matrix-core tiles.
//
//   pf_qproj_kernel     query latents, fp32 and bf16 copies
//   pf_level_count      one level of the descent: a workgroup takes one parent
//                       node and the query heads ("rows") that kept it; the
//                       parent's children are the A operand of a 32x32x16 bf16
//                       MFMA, 32 rows the B operand; every row keeps its best
//                       b children (insertion network over the lane's 32
//                       scores, merged with the partner lane); per-child
//                       counts are added to global counters
//   pf_level_scatter    the rows of every kept child are written to the
//                       child's list (the next level's groups); at the last
//                       level also the per-row leaf slots
//   pf_sample, pf_gather  leaf-major scoring: one item is (leaf, 32 rows),
//                       32 keys of the leaf are the A operand of a 32x32x16
//                       bf16 MFMA, the rows' latents the B operand.  The
//                       sample pass keeps the first s scores of every (row,
//                       leaf); the main pass counts each row's keys at or
//                       above its threshold, reserves their places with one
//                       atomic per row and writes them
//   pf_tau_kernel       per row, a threshold from the weighted samples such
//                       that about 1.5k candidates are expected above it
//   pf_merge_fast       per row, the exact best k of the appended keys and the
//                       output row, for the usual row (its keys fit the
//                       registers, no re-score); any other row goes on a list
//   pf_merge_kernel     the rows on that list: a row whose threshold let fewer
//                       than k keys through (or whose list overflowed) is
//                       scored again in full from its leaf list
#include <limits.h>

#include <type_traits>

#include "select_device.h"

namespace lsa {

typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kPfBlock = 256;        // level and gather workgroups: 4 waves
constexpr int kPfNW = kPfBlock / 64;
constexpr int kPfMergeBlock = 256;
constexpr int kPfMergeFbGrid = 1024; // workgroups of the block merge over the rows the usual-row merge left
constexpr int kPfMinRows = 256;      // query heads per KV head for this path
constexpr int kPfMaxB = 16;
constexpr int kPfMaxF = 64;
constexpr float kPfTarget = 1.5f;    // expected appended keys per row, in units of k
constexpr int kPfSampleR = 100;      // samples expected above the threshold
constexpr int kPfStage = 512;        // staged appends per wave in the gather

struct PfArgs {
  SelArgs s;                   // index, queries, outputs; s.qlat fp32 latents; s.part_keys / part_n appends
  uint16_t* qlat16;            // [R][DL] bf16 bits of the query latents
  int64_t R;                   // rows = T * Hq
  int TG;                      // rows per KV head = T * G
  // level being scored: lev = e - 1 indexes cscore / off / F / P; parents at depth e - 1
  int lev;
  int be;                      // children kept per parent at this level, min(b, F_e)
  int sub;                     // leaf slots under one depth-e slot
  int CH;                      // workgroups per parent
  int64_t P_par;               // parents per KV head, P_{e-1}
  const uint32_t* pstart;      // [Hkv * P_{e-1}] list starts in the parents' entries (null: root)
  const uint32_t* pcnt;        // [Hkv * P_{e-1}] list lengths (null: root)
  const int2* Eprev;           // parents' entries (row, slot) (null: root)
  int2* Enext;                 // children's entries
  u64* mask;                   // per parent entry: the children kept (bit c)
  uint32_t* ccnt;              // [Hkv * P_e] child list lengths
  uint32_t* cfill;             // [Hkv * P_e] fill counters
  uint32_t* cstart;            // [Hkv * P_e] child list starts
  int32_t* lf;                 // [R][nl] leaf of every slot, -1 for none
  int nl;                      // leaf slots per row, prod of the be
  // gather
  int spl;                     // samples per (row, leaf)
  int spl4;                    // spl rounded up to a multiple of 4 (the stride of smp)
  int shalf;                   // 1: only leaves with an even child index are sampled
  uint16_t* smp;               // [R][nl][spl4] top 16 bits of order(score), 0 = not a candidate
  float* tauf;                 // [R] score threshold, -inf = none
  int64_t cap;                 // append capacity per row
  uint32_t* fb_rows;           // [R] rows the usual-row merge leaves to the block merge
  uint32_t* fb_n;              // their count (cleared by the query projection)
  // row-tiled full scan
  bool flat;                   // every key in [sink, p - window] is a candidate of every row
  int64_t ns;                  // sampled keys per KV head
  int64_t fs_keys;             // keys per split
  int fs_split;                // key splits per (KV head, row block)
  int fs_rb;                   // row blocks per KV head
};

__device__ __forceinline__ int2 pf_entry(const PfArgs& a, int64_t pos, int h) {
  if (a.Eprev) return a.Eprev[pos];
  const int64_t i = pos - (int64_t)h * a.TG;
  return make_int2((int)((i / a.s.G) * a.s.Hq + (int64_t)h * a.s.G + i % a.s.G), 0);
}

// the parent's list: [start, start + n) of the parents' entries
__device__ __forceinline__ void pf_parent(const PfArgs& a, int64_t gp, int h, int64_t* start, int* n) {
  if (a.pstart) {
    *start = a.pstart[gp];
    *n = (int)a.pcnt[gp];
  } else {
    *start = (int64_t)h * a.TG;
    *n = a.TG;
  }
}

// Workgroup -> (parent, chunk).  Workgroups are dealt to the 8 XCDs in turn;
// when the KV heads divide evenly, all workgroups of a KV head are mapped to
// one XCD, so that head's query latents and list heads stay in that XCD's L2.
__device__ __forceinline__ void pf_block(const PfArgs& a, int64_t* gp, int* ch) {
  const int64_t b = blockIdx.x;
  const int64_t per_head = a.P_par * a.CH;
  int64_t logical = b;
  if (a.s.Hkv % 8 == 0) {
    const int64_t x = b % 8, q = b / 8;
    logical = (x + 8 * (q / per_head)) * per_head + q % per_head;
  }
  *gp = logical / a.CH;
  *ch = (int)(logical % a.CH);
}

// Append counter of a row, stored head-major (KV head, token, group member)
// so one KV head's counters share no cache line with another head's.
__device__ __forceinline__ uint32_t* pf_count_of(const PfArgs& a, int64_t row) {
  const int64_t t = row / a.s.Hq, hq = row % a.s.Hq;
  const int64_t h = hq / a.s.G, g = hq % a.s.G;
  return a.s.part_n + (h * a.s.T + t) * a.s.G + g;
}

__device__ __forceinline__ v8s as_v8s(const uint4& u) { return __builtin_bit_cast(v8s, u); }

// In-order LDS traffic of one wave, kept in program order by the compiler.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ u64 shfl_xor_u64(u64 v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((u64)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// query latents
// ---------------------------------------------------------------------------

template <typename KT, int DL>
__global__ __launch_bounds__(256) void pf_qproj_kernel(PfArgs a) {
  __shared__ float qin[256 + kQSlices * DL];
  __shared__ float q[DL];
  const int64_t row = blockIdx.x;
  const int h = (int)(row % a.s.Hq) / a.s.G;
  if (row == 0 && threadIdx.x == 0) *a.fb_n = 0u;
  if (!check_index_first(a.s)) return;       // nothing past the header is read
  query_latent<KT, bf16_t, DL>(a.s, row, h, qin, q);
  if (threadIdx.x < DL) a.qlat16[row * DL + threadIdx.x] = (uint16_t)(__float_as_uint(q[threadIdx.x]) >> 16);
  if (threadIdx.x == 0) *pf_count_of(a, row) = 0u;
}

// ---------------------------------------------------------------------------
// descent, one level
// ---------------------------------------------------------------------------

template <int DL, int NT, int BMAX>
__global__ __launch_bounds__(kPfBlock) __attribute__((amdgpu_waves_per_eu(3))) void pf_level_count(PfArgs a) {
  constexpr int KS = DL / 16;                    // k-steps of 16 latent dims
  __shared__ uint32_t lcnt[kPfMaxF];
  if (*a.s.status != LSA_OK) return;
  int64_t gp;
  int ch;
  pf_block(a, &gp, &ch);
  const int h = (int)(gp / a.P_par);
  const int64_t par = gp % a.P_par;
  const int F = a.s.F[a.lev];
  const int64_t Pe = a.s.P[a.lev];
  int64_t start;
  int n;
  pf_parent(a, gp, h, &start, &n);
  const int ntiles = (n + 31) / 32;
  if (ch * kPfNW >= ntiles) return;              // workgroup-uniform
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  if (threadIdx.x < kPfMaxF) lcnt[threadIdx.x] = 0u;
  // children of the parent: non-empty mask and the A operand
  const int64_t child0 = par * F;
  const int* off = a.s.off[a.lev] + (size_t)h * (Pe + 1);
  bool ne = false;
  if (lane < F) ne = off[child0 + lane + 1] > off[child0 + lane];
  const u64 ne_mask = __ballot(ne);
  const bf16_t* cs = (const bf16_t*)a.s.cscore[a.lev] + ((size_t)h * Pe + child0) * DL;
  v8s A[NT][KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = 32 * t + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (c < F) u = *(const uint4*)(cs + (size_t)c * DL + 16 * s + 8 * half);
      A[t][s] = as_v8s(u);
    }
  }
  __syncthreads();
  // A wave's tiles are pipelined: the list entries (rows) two tiles ahead,
  // and where the registers allow (BMAX <= 8) the rows' latents (the B
  // operand) one tile ahead, so a tile's operands are in registers when its
  // turn comes.  A tile past the end has no rows.
  constexpr bool PREQ = BMAX <= 8;
  const int stride = a.CH * kPfNW;
  auto row_of = [&](int tt) {
    const int r = tt * 32 + l32;
    return (tt < ntiles && r < n) ? pf_entry(a, start + r, h).x : -1;
  };
  auto latents_of = [&](int row, uint4* q) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      q[s] = make_uint4(0u, 0u, 0u, 0u);
      if (row >= 0) q[s] = *(const uint4*)(a.qlat16 + (size_t)row * DL + 16 * s + 8 * half);
    }
  };
  int ti = ch * kPfNW + w;
  int row_c = row_of(ti), row_n = row_of(ti + stride);
  uint4 qc[KS];
  if constexpr (PREQ) latents_of(row_c, qc);
  for (; ti < ntiles; ti += stride) {
    const int r_in = ti * 32 + l32;
    const bool valid = r_in < n;
    const int64_t pos = start + r_in;
    uint4 qn[KS];
    if constexpr (PREQ) latents_of(row_n, qn);
    else latents_of(row_c, qc);
    const int row_nn = row_of(ti + 2 * stride);
    v16f acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const v8s Bv = as_v8s(qc[s]);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[t][s], Bv, acc[t], 0, 0, 0);
    }
    // lane holds row l32 against children 32t + 8(i/4) + 4 half + i%4
    // the lane's BMAX best scores, descending: one v_med3 per entry and score
    // (an empty child is -inf here and key 0 below; the keys are taken from
    // the scores again where they are compared, so they hold no registers)
    auto key_of = [&](int t, int i) {
      const int c = 32 * t + 8 * (i >> 2) + 4 * half + (i & 3);
      return ((ne_mask >> c) & 1ull) ? order_u32(acc[t][i]) : 0u;
    };
    float tf[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) tf[j] = -__builtin_huge_valf();
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = 32 * t + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool nec = (ne_mask >> c) & 1ull;
        const float v = nec ? acc[t][i] : -__builtin_huge_valf();
#pragma unroll
        for (int j = BMAX - 1; j > 0; --j) tf[j] = __builtin_amdgcn_fmed3f(tf[j - 1], tf[j], v);
        tf[0] = fmaxf(tf[0], v);
      }
    uint32_t top[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) top[j] = tf[j] == -__builtin_huge_valf() ? 0u : order_u32(tf[j]);
    // the partner lane (lane ^ 32) holds the other children of the row
    uint32_t cm[BMAX];
#pragma unroll
    for (int j = 0; j < BMAX; ++j) {
      const uint32_t o = (uint32_t)__shfl_xor((int)top[BMAX - 1 - j], 32, 64);
      cm[j] = top[j] > o ? top[j] : o;
    }
#pragma unroll
    for (int hs = BMAX / 2; hs >= 1; hs >>= 1)
#pragma unroll
      for (int j = 0; j < BMAX; ++j)
        if ((j & hs) == 0) {
          const uint32_t x = cm[j], y = cm[j + hs];
          cm[j] = x > y ? x : y;
          cm[j + hs] = x > y ? y : x;
        }
    uint32_t theta = 0u;
#pragma unroll
    for (int j = 0; j < BMAX; ++j)
      if (j == a.be - 1) theta = cm[j];
    u64 gt = 0ull, eq = 0ull;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const u64 bit = 1ull << (32 * t + 8 * (i >> 2) + 4 * half + (i & 3));
        const uint32_t kv = key_of(t, i);
        gt |= kv > theta ? bit : 0ull;
        eq |= kv == theta ? bit : 0ull;
      }
    gt |= shfl_xor_u64(gt, 32);
    eq |= shfl_xor_u64(eq, 32);
    u64 sel = gt;
    if (theta != 0u) {
      // ties at the b-th score: the lowest child ids
      int need = a.be - __popcll(gt);
      while (need > 0 && eq != 0ull) {
        const u64 low = eq & (~eq + 1ull);
        sel |= low;
        eq ^= low;
        --need;
      }
    }
    if (half == 0 && valid) {
      a.mask[pos] = sel;
      u64 m = sel;
      while (m != 0ull) {
        const int c = __ffsll((long long)m) - 1;
        atomicAdd(&lcnt[c], 1u);
        m &= m - 1ull;
      }
    }
    if constexpr (PREQ) {
#pragma unroll
      for (int s = 0; s < KS; ++s) qc[s] = qn[s];
    }
    row_c = row_n;
    row_n = row_nn;
  }
  __syncthreads();
  if (threadIdx.x < F && lcnt[threadIdx.x] != 0u)
    atomicAdd(&a.ccnt[(size_t)h * Pe + child0 + threadIdx.x], lcnt[threadIdx.x]);
}

template <int BMAX>
__global__ __launch_bounds__(kPfBlock) void pf_level_scatter(PfArgs a) {
  __shared__ uint32_t lcnt[kPfMaxF], lbase[kPfMaxF], lfill[kPfMaxF], cst[kPfMaxF];
  if (*a.s.status != LSA_OK) return;
  int64_t gp;
  int ch;
  pf_block(a, &gp, &ch);
  const int h = (int)(gp / a.P_par);
  const int64_t par = gp % a.P_par;
  const int F = a.s.F[a.lev];
  const int64_t Pe = a.s.P[a.lev];
  int64_t start;
  int n;
  pf_parent(a, gp, h, &start, &n);
  // rows in tiles of 64, one per lane (the level kernel's tiles are 32 rows)
  const int ntiles = (n + 63) / 64;
  const int64_t cbase = (int64_t)h * Pe + par * F;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (ch == 0 && ntiles == 0) {
    // a parent nobody kept: its children's lists are empty
    if (threadIdx.x < F) a.cstart[cbase + threadIdx.x] = (uint32_t)(a.be * start);
    return;
  }
  if (ch * kPfNW >= ntiles) return;              // workgroup-uniform
  if (w == 0) {
    const uint32_t c = lane < F ? a.ccnt[cbase + lane] : 0u;
    uint32_t incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = (uint32_t)__shfl_up((int)incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane < kPfMaxF) {
      cst[lane] = (uint32_t)(a.be * start) + incl - c;
      lcnt[lane] = 0u;
      lfill[lane] = 0u;
    }
    if (ch == 0 && lane < F) a.cstart[cbase + lane] = (uint32_t)(a.be * start) + incl - c;
  }
  __syncthreads();
  for (int ti = ch * kPfNW + w; ti < ntiles; ti += a.CH * kPfNW) {
    const int r_in = ti * 64 + lane;
    if (r_in < n) {
      u64 m = a.mask[start + r_in];
      while (m != 0ull) {
        atomicAdd(&lcnt[__ffsll((long long)m) - 1], 1u);
        m &= m - 1ull;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < F && lcnt[threadIdx.x] != 0u) lbase[threadIdx.x] = atomicAdd(&a.cfill[cbase + threadIdx.x], lcnt[threadIdx.x]);
  __syncthreads();
  const bool last = a.lev == a.s.L - 1;
  const int be = a.be;                           // <= BMAX: at most be children are kept
  for (int ti = ch * kPfNW + w; ti < ntiles; ti += a.CH * kPfNW) {
    const int r_in = ti * 64 + lane;
    if (r_in < n) {
      const int64_t pos = start + r_in;
      const int2 e = pf_entry(a, pos, h);
      u64 m = a.mask[pos];
      // the kept children in ascending order; their places in the child
      // lists are all reserved before any is used, so the LDS atomics go
      // out back to back
      int cs[BMAX];
#pragma unroll
      for (int j = 0; j < BMAX; ++j) {
        cs[j] = m != 0ull ? __ffsll((long long)m) - 1 : -1;
        m &= m - 1ull;
      }
      uint32_t dst[BMAX];
#pragma unroll
      for (int j = 0; j < BMAX; ++j) dst[j] = cs[j] >= 0 ? atomicAdd(&lfill[cs[j]], 1u) : 0u;
      int nk = 0;
#pragma unroll
      for (int j = 0; j < BMAX; ++j)
        if (cs[j] >= 0) {
          const int c = cs[j];
          a.Enext[cst[c] + lbase[c] + dst[j]] = make_int2(e.x, e.y * be + j);
          ++nk;
        }
      int32_t* lfr = a.lf + (size_t)e.x * a.nl + (size_t)e.y * be * a.sub;
      if (last) {
        // the leaf of each of the entry's be slots (-1 for an empty one):
        // consecutive, so whole 16-byte stores when be is a multiple of 4
        int lv[BMAX];
#pragma unroll
        for (int j = 0; j < BMAX; ++j) lv[j] = cs[j] >= 0 ? (int)(par * F + cs[j]) : -1;
        if ((be & 3) == 0) {
#pragma unroll
          for (int j = 0; j < BMAX; j += 4)
            if (j < be) *(int4*)(lfr + j) = make_int4(lv[j], lv[j + 1], lv[j + 2], lv[j + 3]);
        } else {
#pragma unroll
          for (int j = 0; j < BMAX; ++j)
            if (j < be) lfr[j] = lv[j];
        }
      } else {
        // slots left empty (fewer than be non-empty children) and their subtrees
        for (int j = nk; j < be; ++j)
          for (int64_t q = 0; q < a.sub; ++q) lfr[(int64_t)j * a.sub + q] = -1;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// leaf-major gather
// ---------------------------------------------------------------------------

// Items of a workgroup: (leaf c of the parent, tile i of 32 of the leaf's
// rows).  Keys are the A operand and rows the B operand, so a lane holds one
// row (its threshold and causal limit stay in registers) against 16 keys of
// every 32-key tile.  Main mode runs once over the leaf's key tiles and
// stages the keys at or above their row's threshold in the wave's LDS; at
// the end of the item one atomic per row reserves their places in the rows'
// lists.  Sample mode scores the first key tile and keeps the first spl
// scores of every row.
template <int DL, bool SAMPLE>
__device__ __forceinline__ void pf_gather_body(PfArgs a) {
  constexpr int KS = DL / 16;
  constexpr int RP = DL * 2 / 16;                  // 16-byte parts per key row
  constexpr int PL = 32 * RP / 64;                 // 16-byte parts per lane and 32-key tile
  // main mode: keys at or above a row's threshold are staged per wave (rank
  // key and the row's lane, 0..31) and flushed at the end of every item
  constexpr int SST = SAMPLE ? 1 : kPfStage;
  constexpr int SE = SST / 64;
  __shared__ __align__(16) unsigned char ktile[kPfNW][32 * DL * 2];
  __shared__ u64 skey[kPfNW][SST];
  __shared__ uint8_t srl[kPfNW][SST];
  __shared__ uint32_t scnt[kPfNW][32];
  __shared__ int srow[kPfNW][32];
  __shared__ uint32_t tpre[kPfMaxF + 1];
  __shared__ uint32_t lst[kPfMaxF], lcn[kPfMaxF];
  __shared__ int o0s[kPfMaxF], o1s[kPfMaxF];
  if (*a.s.status != LSA_OK) return;
  const int lev = a.s.L - 1;
  int64_t gp;
  int ch;
  pf_block(a, &gp, &ch);
  const int h = (int)(gp / a.P_par);
  const int64_t par = gp % a.P_par;
  const int F = a.s.F[lev];
  const int64_t Pe = a.s.P[lev];
  const int64_t cbase = (int64_t)h * Pe + par * F;
  const int* offL = a.s.off[lev] + (size_t)h * (Pe + 1);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  if (w == 0) {
    // the sample pass may skip the leaves with an odd child index
    const bool skip = SAMPLE && a.shalf && (lane & 1);
    const uint32_t c = (lane < F && !skip) ? a.ccnt[cbase + lane] : 0u;
    const uint32_t tl = (c + 31u) / 32u;
    uint32_t incl = tl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = (uint32_t)__shfl_up((int)incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane < F) {
      tpre[lane + 1] = incl;
      lst[lane] = a.cstart[cbase + lane];
      lcn[lane] = c;
      o0s[lane] = offL[par * F + lane];
      o1s[lane] = offL[par * F + lane + 1];
    }
    if (lane == 0) tpre[0] = 0u;
  }
  __syncthreads();
  const int items = (int)tpre[F];
  const int sink = a.s.sink;
  const bf16_t* latb = (const bf16_t*)a.s.lat + (size_t)h * a.s.N * DL;
  const int* permb = a.s.perm + (size_t)h * a.s.N;
  // item -> (leaf c of the parent, row tile i); this lane's entry (row,
  // slot) of the leaf's list, or (-1, 0) past the end of the leaf's rows
  auto item_of = [&](int itm, int* cc, int* ii) {
    int lo = 0, hi = F;                // tpre[lo] <= itm < tpre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int)tpre[mid] <= itm) lo = mid; else hi = mid;
    }
    *cc = lo;
    *ii = itm - (int)tpre[lo];
  };
  // this lane's entry of the item's row tile; a lane past the end of the
  // leaf's rows reads the leaf's last entry (dropped where it is used), so
  // the load is unconditional and may stay in flight
  auto entry_of = [&](int cc, int ii) {
    const int r_in = min(ii * 32 + l32, (int)lcn[cc] - 1);
    return a.Enext[lst[cc] + r_in];
  };
  // Key tiles: a tile is loaded coalesced (eight lanes per 128-byte key row;
  // a lane past the leaf reads its last key, masked by position where it is
  // scored), written to the wave's LDS tile with the 16-byte parts of row r
  // XOR-swizzled by r % 8, and read back as an MFMA operand (lane l32 takes
  // key l32's parts) with no bank conflicts.  The wave's LDS accesses
  // execute in order, so one tile buffer serves every tile.
  unsigned char* kl = ktile[w];
  auto put_parts = [&](const u32x4* P) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int c = lane + 64 * q, r = c / RP, pt = c % RP;
      *(u32x4*)(kl + r * RP * 16 + ((pt ^ (r & 7)) % RP) * 16) = P[q];
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto get_a = [&](v8s* A) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int pt = 2 * s + half;
      A[s] = as_v8s(*(const uint4*)(kl + l32 * RP * 16 + ((pt ^ (l32 & 7)) % RP) * 16));
    }
  };
  if constexpr (SAMPLE) {
    // Sample pass: the leaf's first key tile is scored against the item's
    // rows and the first spl scores of every row are kept.  The next item's
    // entries are loaded while the current item is scored (past the last
    // item, the current item's again).
    const int stride = a.CH * kPfNW;
    int2 enext = make_int2(0, 0);
    {
      const int it0 = ch * kPfNW + w;
      if (it0 < items) {
        int cc, ii;
        item_of(it0, &cc, &ii);
        enext = entry_of(cc, ii);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);             // vmcnt(0) only
    for (int it = ch * kPfNW + w; it < items; it += stride) {
      int c, i;
      item_of(it, &c, &i);
      const int2 ecur = enext;
      {
        int cn, in;
        item_of(it + stride < items ? it + stride : it, &cn, &in);
        enext = entry_of(cn, in);
      }
      // this lane's row (lanes l and l + 32 share row l % 32), -1 past the
      // end of the leaf's rows
      const int row = i * 32 + l32 < (int)lcn[c] ? ecur.x : -1;
      const int slot = ecur.y;
      const int o0 = o0s[c], o1 = o1s[c];
      // The key tile depends only on the leaf's range and the row data only
      // on the entry: every load below is unconditional (a lane with no row
      // reads row 0's data and drops it), so they all share one round trip.
      u32x4 PK[PL];
#pragma unroll
      for (int q = 0; q < PL; ++q) {
        const int cq = lane + 64 * q;
        const int krow = max(0, min(o0 + cq / RP, o1 - 1));   // in range for an empty leaf too
        PK[q] = *(const u32x4*)(latb + (size_t)krow * DL + (cq % RP) * 8);
      }
      const int jr = permb[max(0, min(o0 + l32, o1 - 1))];
      const int rq = row >= 0 ? row : 0;
      const int pq = a.s.q_pos[rq / a.s.Hq];
      // the rows' latents (the B operand, a missing row as zeros) come
      // coalesced through the LDS tile as well: one key tile per item makes
      // the row load as large as the key load
      v8s Bq[KS];
      {
        u32x4 P[PL];
#pragma unroll
        for (int q = 0; q < PL; ++q) {
          const int cq = lane + 64 * q;
          const int rr = __shfl(row, cq / RP, 64);
          P[q] = *(const u32x4*)(a.qlat16 + (size_t)(rr >= 0 ? rr : 0) * DL + (cq % RP) * 8);
          if (rr < 0) P[q] = u32x4{0u, 0u, 0u, 0u};
        }
        put_parts(P);
        get_a(Bq);
      }
      const int chi = (row >= 0 && pq >= 0 && (int64_t)pq < a.s.N) ? pq - a.s.window : -1;
      if (o1 <= o0) continue;
      put_parts(PK);
      v8s A[KS];
      get_a(A);
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bq[s], acc, 0, 0, 0);
      // lane holds row l32 against keys m = 8(r/4) + 4 half + r%4; key l32's
      // position as a candidate test value (INT_MAX for a missing key or one
      // inside the sink)
      const int jl = (o0 + l32 < o1 && jr >= sink) ? jr : INT_MAX;
      // registers 4g..4g+3 hold samples m0..m0+3 (m0 = 8g + 4 half): one
      // 8-byte store per group, zero past spl or for a non-candidate
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = 8 * g + 4 * half;
        u64 pk = 0ull;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int jm = __shfl(jl, m0 + cc, 64);
          const u64 v = (m0 + cc < a.spl && jm <= chi) ? (u64)(order_u32(acc[4 * g + cc]) >> 16) : 0ull;
          pk |= v << (16 * cc);
        }
        if (m0 < a.spl && row >= 0) *(u64*)(a.smp + ((size_t)row * a.nl + slot) * a.spl4 + m0) = pk;
      }
    }
  } else {
  // Main pass.  Every load is issued well before its use: an item's row
  // data (row latents, threshold, position) once at its start and awaited
  // at once, since every tile needs them; key tiles one ahead, the last tile
  // of an item fetching the next item's first, so a tile's keys arrive while
  // the tile before it is scored.  Entries hold rows only here.
  const int* Erow = (const int*)a.Enext;
  auto row_entry = [&](int cc, int ii) {
    const int r_in = min(ii * 32 + l32, (int)lcn[cc] - 1);
    return Erow[2 * (size_t)(lst[cc] + r_in)];
  };
  // key tile kt of the CSR range [lo, hi) (a lane past the range reads its
  // last key, masked by position where it is scored; the range is never
  // empty) and key l32's position
  auto load_tile = [&](int lo, int hi, int kt, u32x4* P, int* jraw) {
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int c = lane + 64 * q;
      const int krow = max(0, min(lo + 32 * kt + c / RP, hi - 1));
      P[q] = *(const u32x4*)(latb + (size_t)krow * DL + (c % RP) * 8);
    }
    *jraw = permb[max(0, min(lo + 32 * kt + l32, hi - 1))];
  };
  const int stride = a.CH * kPfNW;
  int it = ch * kPfNW + w;
  if (it >= items) return;
  // Staged entries -> the rows' append lists: per-row counts in LDS, one
  // global atomic per row reserves their places.  A flush is split so that
  // the atomics' round trip overlaps the next item's loads: flush_start (the
  // counts, the atomics issued, not awaited) ends an item, flush_finish (the
  // writes) runs in the next item once its loads are issued.  Until then the
  // staging buffers and row slots keep the finished item's entries.
  int pcnt = 0;                                    // entries of the pending flush (wave-uniform)
  uint32_t plp[SE];                                // their places among their row's entries
  uint32_t pc = 0u, graw = 0u;                     // this lane's row: its entries, the reserved base
  auto flush_start = [&](int cnt, int row) {
    if (half == 0) scnt[w][l32] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < SE; ++q) {
      const int e = lane + 64 * q;
      plp[q] = e < cnt ? atomicAdd(&scnt[w][srl[w][e]], 1u) : 0u;
    }
    wave_lds_sync();
    pc = half == 0 ? scnt[w][l32] : 0u;
    // a lane with nothing to reserve leaves its value undefined (it is not
    // read), so no merge with an older value has to wait for the atomic
    uint32_t got;
    if (pc != 0u) got = atomicAdd(pf_count_of(a, row), pc);
    graw = got;
    pcnt = cnt;
  };
  auto flush_finish = [&]() {
    if (half == 0) scnt[w][l32] = pc != 0u ? graw : 0u;
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < SE; ++q) {
      const int e = lane + 64 * q;
      if (e < pcnt) {
        const int rl = srl[w][e];
        const uint32_t pos = scnt[w][rl] + plp[q];
        if (pos < (uint32_t)a.cap) a.s.part_keys[(size_t)srow[w][rl] * a.cap + pos] = skey[w][e];
      }
    }
    wave_lds_sync();
    pcnt = 0;
  };
  int c, i;
  item_of(it, &c, &i);
  int ecur = row_entry(c, i);
  u32x4 PK[PL];
  int jr;
  load_tile(o0s[c], o1s[c], 0, PK, &jr);
  for (;;) {
    const int o0 = o0s[c], o1 = o1s[c];
    const int nkt = max(1, (o1 - o0 + 31) / 32);
    // the next item (this one again past the last)
    const int itn = it + stride < items ? it + stride : it;
    int cn, in;
    item_of(itn, &cn, &in);
    // this lane's row (lanes l and l + 32 share row l % 32); a lane past
    // the end of the leaf's rows has no row: nothing reaches its threshold
    // and it writes nothing
    const int row = i * 32 + l32 < (int)lcn[c] ? ecur : -1;
    const int rq = row >= 0 ? row : 0;
    const int pq = a.s.q_pos[rq / a.s.Hq];
    const float tq = a.tauf[rq];
    u32x4 Bu[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) Bu[s] = *(const u32x4*)(a.qlat16 + (size_t)rq * DL + 16 * s + 8 * half);
    const int enx = row_entry(cn, in);
    // every tile reads the row data: they are awaited here, once
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(Bu[s]));
    asm volatile("" ::"v"(pq), "v"(tq));
    v8s Bq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) Bq[s] = row >= 0 ? __builtin_bit_cast(v8s, Bu[s]) : v8s{0, 0, 0, 0, 0, 0, 0, 0};
    const int chi = (row >= 0 && pq >= 0 && (int64_t)pq < a.s.N) ? pq - a.s.window : -1;
    const float tau = row >= 0 ? tq : __builtin_huge_valf();
    // the smallest causal limit of the item's rows: a tile whose keys all
    // lie in [sink, that limit] needs no per-key range test
    int chimin = row >= 0 ? chi : INT_MAX;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) chimin = min(chimin, __shfl_xor(chimin, o, 64));
    // the previous item's appends; then this item's rows take the row slots
    if (pcnt > 0) flush_finish();
    if (half == 0) srow[w][l32] = row;
    int cnt = 0;                                   // staged entries (wave-uniform)
    auto flush = [&]() {
      flush_start(cnt, row);
      flush_finish();
      cnt = 0;
    };
    // key l32's position as a candidate test value: INT_MAX for a missing
    // key or one inside the sink
    auto pos_of = [&](int kt, int jraw) { return (o0 + 32 * kt + l32 < o1 && jraw >= sink) ? jraw : INT_MAX; };
    const int o0n = o0s[cn], o1n = o1s[cn];
    for (int kt = 0; kt < nkt; ++kt) {
      put_parts(PK);
      // key l32's position, taken before the next tile's loads reuse its
      // register (a copy of a register with a load in flight would wait for it)
      const int jl = pos_of(kt, jr);
      // the next tile: this item's, or after its last the next item's first
      const bool more = kt + 1 < nkt;
      load_tile(more ? o0 : o0n, more ? o1 : o1n, more ? kt + 1 : 0, PK, &jr);
      v8s A[KS];
      get_a(A);
      v16f acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bq[s], acc, 0, 0, 0);
      // results: lane holds row l32 against keys m = 8(r/4) + 4 half + r%4
      int js[16];
      auto positions = [&]() {
#pragma unroll
        for (int r = 0; r < 16; ++r) js[r] = __shfl(jl, 8 * (r >> 2) + 4 * half + (r & 3), 64);
      };
      const bool dirty = __ballot(jl > chimin) != 0ull;
      if (dirty) {
        // a key outside some row's range: its scores become NaN, which no
        // comparison passes and fmaxf ignores
        positions();
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (js[r] > chi) acc[r] = __builtin_nanf("");
      }
      float mx = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
      if (__ballot(mx >= tau) == 0ull) continue;
      if (!dirty) positions();
      // eight registers add at most 8 x 64 = kPfStage entries
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        u64 bal[8];
        int tot = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          bal[r] = __ballot(acc[8 * hb + r] >= tau);
          tot += __popcll(bal[r]);
        }
        if (tot == 0) continue;
        if (cnt + tot > SST) flush();
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (bal[r] == 0ull) continue;
          const float v = acc[8 * hb + r];
          if (v >= tau) {
            const int e = cnt + (int)mbcnt64(bal[r]);
            skey[w][e] = rank_key(v, js[8 * hb + r]);
            srl[w][e] = (uint8_t)l32;
          }
          cnt += __popcll(bal[r]);
        }
      }
    }
    // the atomics go out behind the next item's entry and first key tile
    // and are awaited together with that item's row data
    if (cnt > 0) flush_start(cnt, row);             // finished in the next item
    if (itn == it) break;
    it = itn;
    c = cn;
    i = in;
    ecur = enx;
  }
  if (pcnt > 0) flush_finish();
  }
}

// The two passes as kernels of their own: the sample pass holds few
// registers and runs six waves per SIMD; the main pass holds its row data,
// a prefetched key tile and the staging bookkeeping, and runs three.
template <int DL>
__global__ __launch_bounds__(kPfBlock) __attribute__((amdgpu_waves_per_eu(6))) void pf_sample(PfArgs a) {
  pf_gather_body<DL, true>(a);
}

template <int DL>
__global__ __launch_bounds__(kPfBlock) __attribute__((amdgpu_waves_per_eu(3))) void pf_gather(PfArgs a) {
  pf_gather_body<DL, false>(a);
}

// ---------------------------------------------------------------------------
// per-row threshold from the samples
// ---------------------------------------------------------------------------

// One wave per row.  A sample of leaf c stands for size_c / min(spl, size_c)
// candidates (fixed point, 4 fraction bits); the threshold is the largest
// 16-bit sample value whose weight at or above it reaches 1.5k, found with two
// 8-bit histogram passes.  A row whose leaves hold at most `cap` keys in all
// takes every candidate (no threshold).
// NG > 0: the row's slots fit one chunk (nl <= 64 kTauCL) and its samples
// NG groups of four (spl <= 4 NG); slots, leaf sizes and samples are then
// loaded once and kept in registers for both histogram passes.
template <int kTauCL, int NG>
__global__ __launch_bounds__(kPfBlock) void pf_tau_kernel(PfArgs a) {
  __shared__ u64 hist[kPfNW][256];
  if (*a.s.status != LSA_OK) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kPfNW + w;
  const bool live = row < a.R;
  const int lev = a.s.L - 1;
  const int64_t Pe = a.s.P[lev];
  int h = 0, p = -1;
  if (live) {
    h = (int)(row % a.s.Hq) / a.s.G;
    p = a.s.q_pos[row / a.s.Hq];
  }
  const int* offL = a.s.off[lev] + (size_t)h * (Pe + 1);
  const int32_t* lfr = a.lf + (size_t)(live ? row : 0) * a.nl;
  const uint16_t* sm = a.smp + (size_t)(live ? row : 0) * a.nl * a.spl4;
  const int FL = a.s.F[lev];
  auto sampled = [&](int leaf) { return !a.shalf || ((leaf % FL) & 1) == 0; };
  // a lane takes the row's slots lane, lane + 64, ... in chunks of kTauCL,
  // whose loads are issued together: slot -> leaf -> CSR range
  auto chunk = [&](int base, int* leaf, int* sz) {
#pragma unroll
    for (int j = 0; j < kTauCL; ++j) {
      const int sl = base + lane + 64 * j;
      leaf[j] = (live && sl < a.nl) ? lfr[sl] : -1;
    }
#pragma unroll
    for (int j = 0; j < kTauCL; ++j) sz[j] = leaf[j] >= 0 ? offL[leaf[j] + 1] - offL[leaf[j]] : 0;
  };
  int64_t tot = 0, tots = 0;                       // candidates of all / of the sampled leaves
  int cleaf[kTauCL], csz[kTauCL];                  // NG > 0: the row's only chunk
  for (int base = 0; base < a.nl; base += 64 * kTauCL) {
    int leaf[kTauCL], sz[kTauCL];
    chunk(base, leaf, sz);
#pragma unroll
    for (int j = 0; j < kTauCL; ++j) {
      tot += sz[j];
      if (leaf[j] >= 0 && sampled(leaf[j])) tots += sz[j];
      if (NG > 0) {
        cleaf[j] = leaf[j];
        csz[j] = sz[j];
      }
    }
  }
  // NG > 0: the samples, loaded once (as in the passes below)
  u64 cs4[NG > 0 ? NG : 1][kTauCL];
  if constexpr (NG > 0) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int j = 0; j < kTauCL; ++j) {
        const int g = 4 * gi, sl = lane + 64 * j;
        const bool use = cleaf[j] >= 0 && sampled(cleaf[j]) && g < min(csz[j], a.spl);
        cs4[gi][j] = use ? *(const u64*)(sm + (size_t)sl * a.spl4 + g) : 0ull;
      }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    tot += __shfl_xor(tot, o, 64);
    tots += __shfl_xor(tots, o, 64);
  }
  const bool want = live && p >= 0 && (int64_t)p < a.s.N && tot > a.cap;
  const u64 target = (u64)((double)kPfTarget * a.s.k * 16.0);
  int d1 = -1, d2 = -1;
  u64 ab1 = 0ull, ab2 = 0ull;
  for (int pass = 0; pass < 2; ++pass) {
    for (int b = lane; b < 256; b += 64) hist[w][b] = 0ull;
    __syncthreads();
    // one sample group: its samples' weights into the wave's histogram
    auto add_group = [&](int g, const int* leaf, const int* sz, const u64* s4) {
#pragma unroll
      for (int j = 0; j < kTauCL; ++j) {
        if (s4[j] == 0ull) continue;
        const int se = sz[j] < a.spl ? sz[j] : a.spl;
        // a sample stands for its share of the leaf, scaled up by the
        // candidates of the leaves that were not sampled
        const u64 wt = (u64)((double)sz[j] * 16.0 * (double)tot / ((double)se * (double)tots));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t v = (uint32_t)(s4[j] >> (16 * c)) & 0xFFFFu;
          if (v == 0u || g + c >= se) continue;
          if (pass == 0) atomicAdd(&hist[w][v >> 8], wt);
          else if ((int)(v >> 8) == d1) atomicAdd(&hist[w][v & 0xFFu], wt);
        }
      }
    };
    if (NG > 0 && want && (pass == 0 || d1 >= 0)) {
#pragma unroll
      for (int gi = 0; gi < (NG > 0 ? NG : 1); ++gi)
        if (4 * gi < a.spl) add_group(4 * gi, cleaf, csz, cs4[gi]);
    }
    if (NG == 0 && want && (pass == 0 || d1 >= 0))
      for (int base = 0; base < a.nl; base += 64 * kTauCL) {
        int leaf[kTauCL], sz[kTauCL];
        chunk(base, leaf, sz);
        // samples in groups of four (one 8-byte load per leaf and group)
        for (int g = 0; g < a.spl; g += 4) {
          u64 s4[kTauCL];
#pragma unroll
          for (int j = 0; j < kTauCL; ++j) {
            const int sl = base + lane + 64 * j;
            const bool use = leaf[j] >= 0 && sampled(leaf[j]) && g < min(sz[j], a.spl);
            s4[j] = use ? *(const u64*)(sm + (size_t)sl * a.spl4 + g) : 0ull;
          }
          add_group(g, leaf, sz, s4);
        }
      }
    __syncthreads();
    if (pass == 0) d1 = wave_find_bin(hist[w], target, &ab1);
    else if (d1 >= 0) d2 = wave_find_bin(hist[w], target - ab1, &ab2);
    __syncthreads();
  }
  float tf = -__builtin_huge_valf();
  if (want && d1 >= 0 && d2 >= 0) tf = order_u32_to_f32(((uint32_t)d1 << 24) | ((uint32_t)d2 << 16));
  if (live && lane == 0) a.tauf[row] = tf;
}

// ---------------------------------------------------------------------------
// per-row exact top-k and output
// ---------------------------------------------------------------------------

// One row by the whole workgroup, any case: the rows pf_merge_fast below
// leaves (a re-score, more appended keys than it holds, an uneven index
// spread).
template <int DL, int M>
__device__ __forceinline__ void pf_merge_row(const PfArgs& a, int64_t row, unsigned char* smem, RadixScratch& rs,
                                             int& n_sh, int* wsum) {
  constexpr int BLOCK = kPfMergeBlock, CAP = M * BLOCK;
  u64* buf = (u64*)smem;
  // one LDS block serves the leaf lists of a re-score (used while streaming
  // candidates) and then the index sort's scratch (used only afterwards)
  int* lpre = (int*)(buf + CAP);
  int* lrow = lpre + a.nl + 1;
  SortScratch& sort_ss = *(SortScratch*)(buf + CAP);
  const int t = (int)(row / a.s.Hq), h = (int)(row % a.s.Hq) / a.s.G;
  const int p = a.s.q_pos[t];
  if (*a.s.status != LSA_OK) {
    write_invalid_row<BLOCK>(a.s.width, a.s.k, a.s.out_idx + (size_t)row * a.s.width,
                             a.s.out_scores ? a.s.out_scores + (size_t)row * a.s.k : nullptr);
    if (a.s.out_leaves)
      for (int i = threadIdx.x; i < a.s.nl_cap; i += BLOCK) a.s.out_leaves[(size_t)row * a.s.nl_cap + i] = -1;
    return;
  }
  const int lev = a.s.L - 1;
  const int* offL = a.s.off[lev] + (size_t)h * (a.s.P[lev] + 1);
  const int32_t* lfr = a.lf + (size_t)row * a.nl;
  // the row's leaves in slot order (the out_leaves row, and for a re-score
  // the CSR row starts and candidate prefix counts); block-wide
  auto leaf_list = [&](bool lists, int* nlv_out, int* total_out) {
    const int per = (a.nl + BLOCK - 1) / BLOCK;
    const int i0 = min(a.nl, (int)threadIdx.x * per), i1 = min(a.nl, i0 + per);
    int c = 0, sz = 0;
    for (int i = i0; i < i1; ++i) {
      const int leaf = lfr[i];
      if (leaf >= 0) {
        ++c;
        if (lists) sz += offL[leaf + 1] - offL[leaf];
      }
    }
    int nlv, total = 0;
    int pos = block_exclusive_scan<BLOCK>(c, wsum, &nlv);
    int run = lists ? block_exclusive_scan<BLOCK>(sz, wsum, &total) : 0;
    int32_t* ol = a.s.out_leaves ? a.s.out_leaves + (size_t)row * a.s.nl_cap : nullptr;
    for (int i = i0; i < i1; ++i) {
      const int leaf = lfr[i];
      if (leaf < 0) continue;
      if (lists) {
        const int r0 = offL[leaf];
        lrow[pos] = r0;
        lpre[pos] = run;
        run += offL[leaf + 1] - r0;
      }
      if (ol) ol[pos] = leaf;
      ++pos;
    }
    if (lists && threadIdx.x == 0) lpre[nlv] = total;
    if (ol)
      for (int i = nlv + threadIdx.x; i < a.s.nl_cap; i += BLOCK) ol[i] = -1;
    __syncthreads();
    *nlv_out = nlv;
    *total_out = total;
  };
  int32_t* orow = a.s.out_idx + (size_t)row * a.s.width;
  float* srow = a.s.out_scores ? a.s.out_scores + (size_t)row * a.s.k : nullptr;
  const bool valid_p = p >= 0 && (int64_t)p < a.s.N;
  const int k = a.s.k;
  const int n_raw = (int)*pf_count_of(a, row);     // loaded with p, not after it
  const int n_in = valid_p ? n_raw : 0;
  const float tau = a.tauf[row];
  const bool rescore = valid_p && ((int64_t)n_in > a.cap || (n_in < k && tau > -__builtin_huge_valf()));
  int nlv = 0, total = 0;
  if (a.flat) {
    // a full scan's candidates are one range of the CSR latent
    if (rescore) {
      if (threadIdx.x == 0) {
        lrow[0] = 0;
        lpre[0] = 0;
        lpre[1] = (int)a.s.N;
      }
      __syncthreads();
      nlv = 1;
      total = (int)a.s.N;
    }
  } else if (rescore || a.s.out_leaves) {
    leaf_list(rescore, &nlv, &total);
  }
  if (!valid_p) {
    write_invalid_row<BLOCK>(a.s.width, a.s.k, orow, srow);
    return;
  }
  int n = 0;
  if (rescore) {
    // the threshold let fewer than k keys through, or the list overflowed:
    // score every candidate of the row
    n = gather_stream<bf16_t, DL, M, 4, BLOCK>(a.s, row, h, a.s.sink, p - a.s.window, lpre, lrow, nlv, 0, total,
                                               0ull, buf, &n_sh, &rs);
  } else if (n_in <= CAP) {
    // the appended keys fit the registers: they are read from the list by
    // the selection itself
    __syncthreads();                               // the lists are dead; the block becomes sort scratch
    write_top_k_row<BLOCK, M>(buf, n_in, k, CAP, p, a.s.sink, a.s.window, orow, srow, &rs, sort_ss,
                              a.s.part_keys + (size_t)row * a.cap);
    return;
  } else {
    // stream the appended keys through the buffer (CAP >= 2k), keeping the
    // best k whenever it fills before the end
    const u64* src = a.s.part_keys + (size_t)row * a.cap;
    for (int done = 0; done < n_in;) {
      const int take = min(CAP - n, n_in - done);
      for (int i = threadIdx.x; i < take; i += BLOCK) buf[n + i] = src[done + i];
      n += take;
      done += take;
      __syncthreads();
      if (done < n_in) {
        topk_compact<BLOCK, M>(buf, n, k, &rs);
        n = k;
      }
    }
  }
  __syncthreads();                                 // the lists are dead; the block becomes sort scratch
  write_top_k_row<BLOCK, M>(buf, n, k, CAP, p, a.s.sink, a.s.window, orow, srow, &rs, sort_ss);
}

template <int DL, int M>
__global__ __launch_bounds__(kPfMergeBlock) void pf_merge_kernel(PfArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ RadixScratch rs;
  __shared__ int n_sh, wsum[kPfMergeBlock / 64];
  const uint32_t nfb = min(*a.fb_n, (uint32_t)a.R);
  for (uint32_t i = blockIdx.x; i < nfb; i += gridDim.x) {
    __syncthreads();                               // the last row's LDS reads are done
    pf_merge_row<DL, M>(a, (int64_t)a.fb_rows[i], smem, rs, n_sh, wsum);
  }
}

// The usual row: its appended keys fit the registers (M per thread) and need
// no re-score.  Same result as pf_merge_row with less than half of its LDS
// and registers: the keys go from the list into registers, the selection
// runs on them there, and only the k kept keys pass through LDS (bucketed by
// index, then put in order in the same place), so six rows fit a CU at once
// (with M = 16) instead of three.  A row it does not take (a re-score, more
// keys than it holds, a bucket of more than 64 keys) goes to the block
// merge's list before anything of its top-k part is written.
template <int M>
__global__ __launch_bounds__(kPfMergeBlock) void pf_merge_fast(PfArgs a) {
  constexpr int BLOCK = kPfMergeBlock, CAP = M * BLOCK;
  extern __shared__ __align__(16) unsigned char smem[];   // k + 4 rank keys
  __shared__ RadixScratch rs;
  __shared__ SortScratch ss;
  u64* buf = (u64*)smem;
  const int64_t row = blockIdx.x;
  const int t = (int)(row / a.s.Hq);
  const int k = a.s.k;
  // independent loads, issued together
  const int status = *a.s.status;
  const int p = a.s.q_pos[t];
  const int n_raw = (int)*pf_count_of(a, row);
  const float tau = a.tauf[row];
  int32_t* orow = a.s.out_idx + (size_t)row * a.s.width;
  float* srow = a.s.out_scores ? a.s.out_scores + (size_t)row * k : nullptr;
  if (status != LSA_OK) {
    write_invalid_row<BLOCK>(a.s.width, k, orow, srow);
    if (a.s.out_leaves)
      for (int i = threadIdx.x; i < a.s.nl_cap; i += BLOCK) a.s.out_leaves[(size_t)row * a.s.nl_cap + i] = -1;
    return;
  }
  const bool valid_p = p >= 0 && (int64_t)p < a.s.N;
  const int n_in = valid_p ? n_raw : 0;
  const bool rescore = valid_p && ((int64_t)n_in > a.cap || (n_in < k && tau > -__builtin_huge_valf()));
  if (rescore || n_in > CAP) {                     // block-uniform
    if (threadIdx.x == 0) a.fb_rows[atomicAdd(a.fb_n, 1u)] = (uint32_t)row;
    return;
  }
  if (a.s.out_leaves && !a.flat && threadIdx.x < 64) {
    // the row's leaves in slot order, then -1 (wave 0; global writes only)
    int32_t* ol = a.s.out_leaves + (size_t)row * a.s.nl_cap;
    const int32_t* lfr = a.lf + (size_t)row * a.nl;
    const int lane = threadIdx.x;
    uint32_t base = 0;
    for (int i0 = 0; i0 < a.nl; i0 += 64) {
      const int leaf = i0 + lane < a.nl ? lfr[i0 + lane] : -1;
      const u64 bal = __ballot(leaf >= 0);
      if (leaf >= 0) ol[base + mbcnt64(bal)] = leaf;
      base += (uint32_t)__popcll(bal);
    }
    for (int i = (int)base + lane; i < a.s.nl_cap; i += 64) ol[i] = -1;
  }
  if (!valid_p) {
    write_invalid_row<BLOCK>(a.s.width, k, orow, srow);
    return;
  }
  const u64* src = a.s.part_keys + (size_t)row * a.cap;
  u64 pre[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int i = threadIdx.x + j * BLOCK;
    pre[j] = i < n_in ? src[i] : 0ull;
  }
  const bool done = write_top_k_row<BLOCK, M, true>(buf, n_in, k, 0, p, a.s.sink, a.s.window, orow, srow, &rs, ss,
                                                    nullptr, pre);
  if (!done && threadIdx.x == 0) a.fb_rows[atomicAdd(a.fb_n, 1u)] = (uint32_t)row;   // an uneven index spread
}

// ---------------------------------------------------------------------------
// row-tiled full scan (lsa_flat_select for large query batches)
// ---------------------------------------------------------------------------

constexpr int kFsBlock = 256;                              // 4 waves
constexpr int kFsWaveRows = 64;                            // two 32-row B tiles per wave
constexpr int kFsRows = (kFsBlock / 64) * kFsWaveRows;     // rows per workgroup
constexpr int kFsStage = 1024;                             // staged appends per wave (16 x 64)
constexpr int kFsSampleR = 32;                             // order statistic kept per lane
constexpr int64_t kFsSplitKeys = 16384;                     // keys per split of the scan
constexpr int kFsDepth = 2;                                // key tiles in flight per wave

// Rows of a KV head in scan order: i = token * G + group member.
__device__ __forceinline__ int fs_row(const PfArgs& a, int h, int64_t i) {
  return (int)((i / a.s.G) * a.s.Hq + (int64_t)h * a.s.G + i % a.s.G);
}

// Per-row threshold of the full scan.  ns keys evenly spaced over the CSR
// latent (a stratified sample: every bucket contributes in proportion to its
// size) are scored on the matrix cores against 32 rows per wave.  Each lane
// keeps the 32 best candidate scores of its half of the samples in a sorted
// register list (one v_med3 per entry and insertion), and the threshold is
// the smaller of the two halves' 32nd best, so at least 64 samples reach it
// and about 64 N / ns keys are expected at or above it.  Rows with an invalid
// position get +inf (nothing is appended); a row whose samples hold fewer
// than 32 candidates per half gets -inf (every candidate is appended).
template <int DL>
__global__ __launch_bounds__(kFsBlock) void fs_tau_kernel(PfArgs a) {
  constexpr int KS = DL / 16;
  if (*a.s.status != LSA_OK) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t tiles = (a.TG + 31) / 32;          // row tiles per KV head
  const int64_t gw = (int64_t)blockIdx.x * (kFsBlock / 64) + w;
  if (gw >= tiles * a.s.Hkv) return;
  const int h = (int)(gw / tiles);
  const int64_t i = (gw % tiles) * 32 + l32;
  int row = -1, chi = -1;
  bool pv = false;
  if (i < a.TG) {
    row = fs_row(a, h, i);
    const int p = a.s.q_pos[row / a.s.Hq];
    pv = p >= 0 && (int64_t)p < a.s.N;
    chi = pv ? p - a.s.window : -1;
  }
  v8s Bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (row >= 0) u = *(const uint4*)(a.qlat16 + (size_t)row * DL + 16 * s + 8 * half);
    Bq[s] = as_v8s(u);
  }
  const bf16_t* latb = (const bf16_t*)a.s.lat + (size_t)h * a.s.N * DL;
  const int* permb = a.s.perm + (size_t)h * a.s.N;
  const int64_t N = a.s.N, ns = a.ns;
  // sample tile: key l32 of the tile is sample tile * 32 + l32
  // (a lane past the last sample reads the last one and is masked where its
  // position is tested; nothing here uses the loaded values, so the next
  // tile's loads stay in flight while this one is scored)
  auto load = [&](int64_t tile, v8s* A, int* jl) {
    const int64_t key = min(tile * 32 + l32, ns - 1) * N / ns;
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = as_v8s(*(const uint4*)(latb + (size_t)key * DL + 16 * s + 8 * half));
    *jl = permb[key];
  };
  float t[kFsSampleR];
#pragma unroll
  for (int q = 0; q < kFsSampleR; ++q) t[q] = -__builtin_huge_valf();
  const int64_t ntile = (ns + 31) / 32;
  v8s A[KS], An[KS];
  int jl = INT_MAX, jn = INT_MAX;
  load(0, A, &jl);
  for (int64_t tile = 0; tile < ntile; ++tile) {
    if (tile + 1 < ntile) load(tile + 1, An, &jn);
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bq[s], acc, 0, 0, 0);
    const int jc = (tile * 32 + l32 < ns && jl >= a.s.sink) ? jl : INT_MAX;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * half + (r & 3);
      const int jm = __shfl(jc, m, 64);
      const float v = jm <= chi ? acc[r] : -__builtin_huge_valf();
      if (__ballot(v > t[kFsSampleR - 1]) != 0ull) {
#pragma unroll
        for (int q = kFsSampleR - 1; q > 0; --q) t[q] = __builtin_amdgcn_fmed3f(t[q - 1], t[q], v);
        t[0] = fmaxf(t[0], v);
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = An[s];
    jl = jn;
  }
  const float mine = t[kFsSampleR - 1];
  const float other = __shfl_xor(mine, 32, 64);
  if (half == 0 && row >= 0) a.tauf[row] = pv ? fminf(mine, other) : __builtin_huge_valf();
}

// The scan.  A workgroup takes 256 rows of one KV head (64 per wave, as two
// 32-row B operands held in registers) and one split of keys.  Every wave
// streams the split's 32-key tiles on its own, with no workgroup barrier (the
// four waves read the same keys, so all but the first read hit the caches):
// a tile is loaded coalesced two tiles ahead, passed through the wave's LDS
// tile to become the MFMA operand, and scored while the next tile's loads
// are in flight.  A tile whose keys all lie in every row's candidate range
// (one ballot) skips the per-key range test.  Scores at or above the row's
// threshold are staged in LDS per wave and flushed to the rows' append lists
// with one global atomic per row and flush.
template <int DL>
__global__ __launch_bounds__(kFsBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void fs_scan_kernel(PfArgs a) {
  constexpr int KS = DL / 16;
  if (*a.s.status != LSA_OK) return;
  constexpr int NW = kFsBlock / 64;
  constexpr int SE = kFsStage / 64;
  constexpr int TB = 32 * DL * 2;                  // bytes of a 32-key tile
  constexpr int RP = DL * 2 / 16;                  // 16-byte parts per key row
  constexpr int PL = TB / 16 / 64;                 // 16-byte parts per lane and tile
  __shared__ u64 skey[NW][kFsStage];
  __shared__ uint8_t srl[NW][kFsStage];
  __shared__ uint32_t scnt[NW][64];
  __shared__ int srid[NW][64];
  __shared__ __align__(16) unsigned char ktile[NW][2][TB];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // workgroup -> (KV head, key split, row block); with the KV heads a
  // multiple of 8, all workgroups of a head run on one XCD, so its keys are
  // shared through that XCD's L2
  const int64_t per_head = (int64_t)a.fs_rb * a.fs_split;
  int64_t logical = blockIdx.x;
  if (a.s.Hkv % 8 == 0) {
    const int64_t x = logical % 8, q = logical / 8;
    logical = (x + 8 * (q / per_head)) * per_head + q % per_head;
  }
  const int h = (int)(logical / per_head);
  const int sp = (int)((logical % per_head) / a.fs_rb);
  const int rb = (int)(logical % a.fs_rb);
  // this lane's rows: row tile u holds rows i0 + 32 u + l32
  const int64_t i0 = (int64_t)rb * kFsRows + w * kFsWaveRows;
  int rowu[2], chi[2];
  float tau[2];
  v8s B[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t i = i0 + 32 * u + l32;
    rowu[u] = -1;
    chi[u] = -1;
    tau[u] = __builtin_huge_valf();
    if (i < a.TG) {
      const int row = fs_row(a, h, i);
      const int p = a.s.q_pos[row / a.s.Hq];
      if (p >= 0 && (int64_t)p < a.s.N) {
        tau[u] = a.tauf[row];
        chi[u] = p - a.s.window;
      }
      rowu[u] = row;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (rowu[u] >= 0) v = *(const uint4*)(a.qlat16 + (size_t)rowu[u] * DL + 16 * s + 8 * half);
      B[u][s] = as_v8s(v);
    }
  }
  srid[w][lane] = rowu[half];                      // staged row index 32 u + l32 -> row
  // the smallest causal limit of the rows that can take keys
  int chimin = INT_MAX;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (tau[u] < __builtin_huge_valf()) chimin = min(chimin, chi[u]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) chimin = min(chimin, __shfl_xor(chimin, o, 64));

  const bf16_t* latb = (const bf16_t*)a.s.lat + (size_t)h * a.s.N * DL;
  const int* permb = a.s.perm + (size_t)h * a.s.N;
  const int64_t k0 = (int64_t)sp * a.fs_keys;
  const int64_t k1 = min(a.s.N, k0 + a.fs_keys);
  const int64_t ntile = k1 > k0 ? (k1 - k0 + 31) / 32 : 0;
  // tile i: A operand (key l32's dims) and the key's position.  A lane past
  // the range loads the range's last key instead (its scores are masked by
  // position), so the loads are unconditional and nothing here uses the
  // loaded values: they stay in flight until the tile is scored.
  auto tile_key = [&](int64_t i) { return min(k0 + i * 32 + l32, k1 - 1); };
  // A tile is loaded coalesced (eight lanes per 128-byte key row), written to
  // the wave's LDS tile with the 16-byte parts of row r XOR-swizzled by r % 8,
  // and read back as the MFMA operand (lane l32 takes key l32's parts) with
  // no bank conflicts: an operand load straight from global memory would
  // touch 32 cache lines per instruction.
  auto load_tile = [&](int64_t i, u32x4* P) {
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int c = lane + 64 * q;                 // part c: row c / RP, part c % RP
      const int64_t key = min(k0 + i * 32 + c / RP, k1 - 1);
      P[q] = *(const u32x4*)(latb + (size_t)key * DL + (c % RP) * 8);
    }
  };
  auto put_tile = [&](const u32x4* P, int buf) {
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      const int c = lane + 64 * q, r = c / RP, pt = c % RP;
      *(u32x4*)(&ktile[w][buf][r * RP * 16 + ((pt ^ (r & 7)) % RP) * 16]) = P[q];
    }
  };
  auto get_tile = [&](int buf, v8s* A) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int pt = 2 * s + half;
      A[s] = as_v8s(*(const uint4*)(&ktile[w][buf][l32 * RP * 16 + ((pt ^ (l32 & 7)) % RP) * 16]));
    }
  };
  auto mfma_tile = [&](const v8s* A, v16f& c0, v16f& c1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      c0[r] = 0.f;
      c1[r] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B[0][s], c0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B[1][s], c1, 0, 0, 0);
  };
  // staged entries -> the rows' append lists
  auto flush = [&](int n) {
    scnt[w][lane] = 0u;
    wave_lds_sync();
    uint32_t lp[SE];
#pragma unroll
    for (int q = 0; q < SE; ++q) {
      const int e = lane + 64 * q;
      lp[q] = e < n ? atomicAdd(&scnt[w][srl[w][e]], 1u) : 0u;
    }
    wave_lds_sync();
    const uint32_t c = scnt[w][lane];
    uint32_t base = 0u;
    if (c != 0u) base = atomicAdd(pf_count_of(a, srid[w][lane]), c);
    wave_lds_sync();
    scnt[w][lane] = base;
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < SE; ++q) {
      const int e = lane + 64 * q;
      if (e < n) {
        const int rl = srl[w][e];
        const uint32_t pos = scnt[w][rl] + lp[q];
        if (pos < (uint32_t)a.cap) a.s.part_keys[(size_t)srid[w][rl] * a.cap + pos] = skey[w][e];
      }
    }
    // loads and stores share one counter here: with the flush's stores
    // drained, the key loads in flight stay countable across the flush
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
    wave_lds_sync();
  };
  int cnt = 0;                                     // staged entries of this wave (wave-uniform)
  // results: lane holds its rows against keys m = 8 (r / 4) + 4 half + r % 4
  auto epilogue = [&](v16f& acc0, v16f& acc1, int jraw, int64_t i) {
    // a sink key, or a lane past the range, is no candidate
    const int jl = (jraw >= a.s.sink && k0 + i * 32 + l32 < k1) ? jraw : INT_MAX;
    int js[16];
    auto positions = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) js[r] = __shfl(jl, 8 * (r >> 2) + 4 * half + (r & 3), 64);
    };
    const bool dirty = __ballot(jl > chimin) != 0ull;
    if (dirty) {
      // some key lies outside some row's range: those scores become NaN,
      // which no comparison passes and fmaxf ignores
      positions();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (js[r] > chi[0]) acc0[r] = __builtin_nanf("");
        if (js[r] > chi[1]) acc1[r] = __builtin_nanf("");
      }
    }
    float m0 = acc0[0], m1 = acc1[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      m0 = fmaxf(m0, acc0[r]);
      m1 = fmaxf(m1, acc1[r]);
    }
    if (__ballot(m0 >= tau[0] || m1 >= tau[1]) == 0ull) return;
    if (!dirty) positions();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // one row tile adds at most 16 x 64 = kFsStage entries
      u64 bal[16];
      int tot = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bal[r] = __ballot((u ? acc1[r] : acc0[r]) >= tau[u]);
        tot += __popcll(bal[r]);
      }
      if (tot == 0) continue;
      if (cnt + tot > kFsStage) {
        flush(cnt);
        cnt = 0;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (bal[r] == 0ull) continue;
        const float v = u ? acc1[r] : acc0[r];
        if (v >= tau[u]) {
          const int e = cnt + (int)mbcnt64(bal[r]);
          skey[w][e] = rank_key(v, js[r]);
          srl[w][e] = (uint8_t)(32 * u + l32);
        }
        cnt += __popcll(bal[r]);
      }
    }
  };

  // kFsDepth tiles in flight: tile i is scored while the loads of tiles
  // i + 1 .. i + kFsDepth - 1 are outstanding; right after tile i's MFMAs
  // are issued its registers take tile i + kFsDepth's loads
  // Every load is unconditional (tiles past the range read its last key and
  // are masked), so the number of loads issued after any of them is fixed and
  // each wait covers only its own tile; a tile's registers are reloaded only
  // after they have been written to LDS, its position after its scores are
  // filtered.  Tile i + 1 goes to LDS before tile i is filtered.
  if (ntile > 0) {
    u32x4 P[kFsDepth][PL];
    int jt[kFsDepth];
#pragma unroll
    for (int d = 0; d < kFsDepth; ++d) {
      load_tile(d, P[d]);
      jt[d] = permb[tile_key(d)];
    }
    put_tile(P[0], 0);
    load_tile(kFsDepth, P[0]);
    // one tile step, with its ring slot d a compile-time constant
    auto step = [&](int64_t g, auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      constexpr int dn = (d + 1) % kFsDepth;
      const int64_t i = g * kFsDepth + d;
      // a wave's LDS accesses execute in order; these only keep the
      // compiler from moving them across each other
      __builtin_amdgcn_wave_barrier();
      v8s A[KS];
      get_tile((int)(i & 1), A);
      v16f c0, c1;
      mfma_tile(A, c0, c1);
      __builtin_amdgcn_wave_barrier();
      put_tile(P[dn], (int)((i + 1) & 1));
      load_tile(i + 1 + kFsDepth, P[dn]);
      epilogue(c0, c1, jt[d], i);
      jt[d] = permb[tile_key(i + kFsDepth)];
    };
    static_assert(kFsDepth == 2, "the step calls below");
    const int64_t ngrp = (ntile + kFsDepth - 1) / kFsDepth;
    for (int64_t g = 0; g < ngrp; ++g) {
      step(g, std::integral_constant<int, 0>{});
      step(g, std::integral_constant<int, 1>{});
    }
  }
  if (cnt > 0) flush(cnt);
}

__global__ void pf_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct PfWs {
  int* status;
  float* qlat;
  uint16_t* qlat16;
  int2* E[kMaxLevels];
  uint32_t* ccnt[kMaxLevels];
  uint32_t* cfill[kMaxLevels];
  uint32_t* cstart[kMaxLevels];
  u64* mask;
  int32_t* lf;
  uint16_t* smp;
  float* tauf;
  u64* part_keys;
  uint32_t* part_n;
  uint32_t* fb_rows;
  uint32_t* fb_n;
};

size_t carve_prefill(const lsa_index_desc& d, const PfPlan& pl, int64_t R, void* base, PfWs* out) {
  const Layout L = compute_layout(d);
  Carver c(base);
  PfWs w;
  memset(&w, 0, sizeof(w));
  const int DL = d.d_latent;
  w.status = c.take<int>(64);                 // byte 0 of the workspace (lsa.h)
  w.qlat = c.take<float>((size_t)(R * DL));
  w.qlat16 = c.take<uint16_t>((size_t)(R * DL));
  for (int e = 0; e < d.n_levels; ++e) {
    w.E[e] = c.take<int2>((size_t)(R * pl.nl[e + 1]));
    const size_t nodes = (size_t)(d.n_kv_heads * L.nodes[e + 1]);
    w.ccnt[e] = c.take<uint32_t>(nodes);
    w.cfill[e] = c.take<uint32_t>(nodes);
    w.cstart[e] = c.take<uint32_t>(nodes);
  }
  w.mask = c.take<u64>((size_t)(R * pl.nl[d.n_levels - 1]));
  w.lf = c.take<int32_t>((size_t)(R * pl.nl[d.n_levels]));
  w.smp = c.take<uint16_t>((size_t)(R * pl.nl[d.n_levels] * ((pl.spl + 3) / 4 * 4)));
  w.tauf = c.take<float>((size_t)R);
  w.part_keys = c.take<u64>((size_t)(R * pl.cap));
  w.part_n = c.take<uint32_t>((size_t)R);
  w.fb_rows = c.take<uint32_t>((size_t)R);
  w.fb_n = c.take<uint32_t>(64);
  if (out) *out = w;
  return align_up(c.used);
}

int clampi(int64_t x, int lo, int hi) { return (int)(x < lo ? lo : (x > hi ? hi : x)); }

template <int DL, int NT>
void launch_count_b(const PfArgs& a, int64_t grid, int be, hipStream_t st) {
  if (be <= 4) hipLaunchKernelGGL((pf_level_count<DL, NT, 4>), dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
  else if (be <= 8) hipLaunchKernelGGL((pf_level_count<DL, NT, 8>), dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
  else hipLaunchKernelGGL((pf_level_count<DL, NT, 16>), dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
}

// The merge of the usual rows, then the block merge over the rows it left.
// The usual-row merge holds M keys per thread for the tree (the block
// merge's buffer; rows past it are rare) and 2M for the full scan, whose
// threshold aims at 2k appended keys: 2M per thread hold 4k keys or more.
template <int DL, int M>
void launch_pf_merge(const PfArgs& a, hipStream_t st) {
  if (a.R <= 0) return;
  if (a.flat) {
    constexpr int MF = 2 * M;
    hipLaunchKernelGGL(pf_merge_fast<MF>, dim3((unsigned)a.R), dim3(kPfMergeBlock), ((size_t)a.s.k + 4) * 8, st, a);
  } else {
    hipLaunchKernelGGL(pf_merge_fast<M>, dim3((unsigned)a.R), dim3(kPfMergeBlock), ((size_t)a.s.k + 4) * 8, st, a);
  }
  auto mk = pf_merge_kernel<DL, M>;
  const size_t lists = ((size_t)a.nl * 2 + 2) * 4;
  const size_t lds = (size_t)M * kPfMergeBlock * 8 + (lists > sizeof(SortScratch) ? lists : sizeof(SortScratch));
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)mk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  // a grid-stride loop over the list; its length is known only on the device
  const int64_t grid = a.R < kPfMergeFbGrid ? a.R : kPfMergeFbGrid;
  hipLaunchKernelGGL(mk, dim3((unsigned)grid), dim3(kPfMergeBlock), lds, st, a);
}

template <typename KT, int DL>
int run_prefill(const lsa_index_desc& d, const lsa_select_params& p, const PfPlan& pl, const void* index,
                const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, char* err, size_t errlen) {
  const Layout L = compute_layout(d);
  const char* blob = (const char*)index;
  const int64_t R = (int64_t)T * Hq;
  PfWs w;
  carve_prefill(d, pl, R, ws, &w);
  PfArgs a;
  memset(&a, 0, sizeof(a));
  SelArgs& s = a.s;
  s.lat = blob + L.latent;
  s.perm = (const int*)(blob + L.perm);
  s.N = d.n_keys;
  s.Hkv = d.n_kv_heads;
  s.G = Hq / d.n_kv_heads;
  s.Hq = Hq;
  s.T = T;
  s.d_head = d.d_head;
  s.queries = queries;
  s.W = (const float*)(blob + L.W);
  s.qlat = w.qlat;
  s.q_pos = q_pos;
  s.sink = p.sink;
  s.window = p.window;
  s.k = p.k;
  s.width = p.sink + p.k + p.window;
  s.L = d.n_levels;
  for (int l = 0; l < d.n_levels; ++l) {
    s.cscore[l] = blob + L.cscore[l];
    s.off[l] = (const int*)(blob + L.offsets[l]);
    s.F[l] = d.fanout[l];
    s.P[l] = L.nodes[l + 1];
  }
  s.b = p.b;
  s.beam = p.beam;
  s.nl_cap = pl.nl_out;
  s.out_leaves = out_leaves;
  s.part_keys = w.part_keys;
  s.part_n = w.part_n;
  s.part_cap = pl.cap;
  s.out_idx = out_idx;
  s.out_scores = out_scores;
  a.qlat16 = w.qlat16;
  a.R = R;
  a.TG = T * s.G;
  a.mask = w.mask;
  a.lf = w.lf;
  a.nl = pl.nl[d.n_levels];
  a.spl = pl.spl;
  a.spl4 = (pl.spl + 3) / 4 * 4;
  a.shalf = pl.shalf;
  set_header_check(s, d, L, index, w.status);
  a.smp = w.smp;
  a.tauf = w.tauf;
  a.cap = pl.cap;
  a.fb_rows = w.fb_rows;
  a.fb_n = w.fb_n;

#define PF_CHECK(what)                                                               \
  do {                                                                               \
    hipError_t e_ = hipGetLastError();                                               \
    if (e_ != hipSuccess) {                                                          \
      snprintf(err, errlen, "%s launch failed: %s", what, hipGetErrorString(e_));    \
      return LSA_ERR_HIP;                                                            \
    }                                                                                \
  } while (0)

  prof_begin(LSA_STAGE_DESCEND, st);
  hipLaunchKernelGGL((pf_qproj_kernel<KT, DL>), dim3((unsigned)R), dim3(256), 0, st, a);
  PF_CHECK("query projection");
  for (int lev = 0; lev < d.n_levels; ++lev) {
    const int64_t nodes = (int64_t)d.n_kv_heads * L.nodes[lev + 1];
    hipLaunchKernelGGL(pf_fill_u32, dim3(clampi((nodes + 255) / 256, 1, 4096)), dim3(256), 0, st, w.ccnt[lev], nodes, 0u);
    hipLaunchKernelGGL(pf_fill_u32, dim3(clampi((nodes + 255) / 256, 1, 4096)), dim3(256), 0, st, w.cfill[lev], nodes, 0u);
    a.lev = lev;
    a.be = pl.be[lev];
    a.sub = pl.nl[d.n_levels] / pl.nl[lev + 1];
    a.CH = pl.ch[lev];
    a.P_par = L.nodes[lev];
    a.pstart = lev ? w.cstart[lev - 1] : nullptr;
    a.pcnt = lev ? w.ccnt[lev - 1] : nullptr;
    a.Eprev = lev ? w.E[lev - 1] : nullptr;
    a.Enext = w.E[lev];
    a.ccnt = w.ccnt[lev];
    a.cfill = w.cfill[lev];
    a.cstart = w.cstart[lev];
    const int64_t grid = (int64_t)d.n_kv_heads * L.nodes[lev] * a.CH;
    if (d.fanout[lev] <= 32) launch_count_b<DL, 1>(a, grid, a.be, st);
    else launch_count_b<DL, 2>(a, grid, a.be, st);
    PF_CHECK("level scoring");
    if (a.be <= 4) hipLaunchKernelGGL(pf_level_scatter<4>, dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
    else if (a.be <= 8) hipLaunchKernelGGL(pf_level_scatter<8>, dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
    else hipLaunchKernelGGL(pf_level_scatter<16>, dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
    PF_CHECK("level lists");
  }
  prof_end(LSA_STAGE_DESCEND, st);
  {
    const int lev = d.n_levels - 1;
    a.lev = lev;
    a.CH = pl.chg;
    a.P_par = L.nodes[lev];
    a.Enext = w.E[lev];
    a.ccnt = w.ccnt[lev];
    a.cstart = w.cstart[lev];
    const int64_t grid = (int64_t)d.n_kv_heads * L.nodes[lev] * a.CH;
    const unsigned rgrid = (unsigned)((R + kPfNW - 1) / kPfNW);
    prof_begin(LSA_STAGE_SAMPLE, st);
    hipLaunchKernelGGL((pf_sample<DL>), dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
    PF_CHECK("sample pass");
    // rows whose slots fit one chunk and whose samples fit the registers
    // keep them there for both histogram passes
    if (a.nl >= 512) {
      if (a.nl <= 64 * 8 && a.spl <= 4) hipLaunchKernelGGL((pf_tau_kernel<8, 1>), dim3(rgrid), dim3(kPfBlock), 0, st, a);
      else hipLaunchKernelGGL((pf_tau_kernel<8, 0>), dim3(rgrid), dim3(kPfBlock), 0, st, a);
    } else {
      // (three groups of samples kept in registers would cost half the waves)
      hipLaunchKernelGGL((pf_tau_kernel<4, 0>), dim3(rgrid), dim3(kPfBlock), 0, st, a);
    }
    PF_CHECK("thresholds");
    prof_end(LSA_STAGE_SAMPLE, st);
    prof_begin(LSA_STAGE_GATHER, st);
    hipLaunchKernelGGL((pf_gather<DL>), dim3((unsigned)grid), dim3(kPfBlock), 0, st, a);
    PF_CHECK("gather");
    prof_end(LSA_STAGE_GATHER, st);
  }
  prof_begin(LSA_STAGE_MERGE, st);
  switch (pl.merge_m) {
    case 1: launch_pf_merge<DL, 1>(a, st); break;
    case 2: launch_pf_merge<DL, 2>(a, st); break;
    case 4: launch_pf_merge<DL, 4>(a, st); break;
    case 8: launch_pf_merge<DL, 8>(a, st); break;
    default: launch_pf_merge<DL, 16>(a, st); break;
  }
  prof_end(LSA_STAGE_MERGE, st);
  PF_CHECK("merge");
#undef PF_CHECK
  return LSA_OK;
}

struct FsWs {
  int* status;
  float* qlat;
  uint16_t* qlat16;
  float* tauf;
  u64* part_keys;
  uint32_t* part_n;
  uint32_t* fb_rows;
  uint32_t* fb_n;
};

size_t carve_flat_tiled(const lsa_index_desc& d, const FsPlan& pl, int64_t R, void* base, FsWs* out) {
  Carver c(base);
  FsWs w;
  w.status = c.take<int>(64);                 // byte 0 of the workspace (lsa.h)
  w.qlat = c.take<float>((size_t)(R * d.d_latent));
  w.qlat16 = c.take<uint16_t>((size_t)(R * d.d_latent));
  w.tauf = c.take<float>((size_t)R);
  w.part_keys = c.take<u64>((size_t)(R * pl.cap));
  w.part_n = c.take<uint32_t>((size_t)R);
  w.fb_rows = c.take<uint32_t>((size_t)R);
  w.fb_n = c.take<uint32_t>(64);
  if (out) *out = w;
  return align_up(c.used);
}

template <typename KT, int DL>
int run_flat_tiled(const lsa_index_desc& d, const lsa_select_params& p, const FsPlan& pl, const void* index,
                   const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                   float* out_scores, void* ws, hipStream_t st, char* err, size_t errlen) {
  const Layout L = compute_layout(d);
  const char* blob = (const char*)index;
  const int64_t R = (int64_t)T * Hq;
  FsWs w;
  carve_flat_tiled(d, pl, R, ws, &w);
  PfArgs a;
  memset(&a, 0, sizeof(a));
  SelArgs& s = a.s;
  s.lat = blob + L.latent;
  s.perm = (const int*)(blob + L.perm);
  s.N = d.n_keys;
  s.Hkv = d.n_kv_heads;
  s.G = Hq / d.n_kv_heads;
  s.Hq = Hq;
  s.T = T;
  s.d_head = d.d_head;
  s.queries = queries;
  s.W = (const float*)(blob + L.W);
  s.qlat = w.qlat;
  s.q_pos = q_pos;
  s.sink = p.sink;
  s.window = p.window;
  s.k = p.k;
  s.width = p.sink + p.k + p.window;
  s.L = d.n_levels;
  s.part_keys = w.part_keys;
  s.part_n = w.part_n;
  s.part_cap = pl.cap;
  s.out_idx = out_idx;
  s.out_scores = out_scores;
  a.qlat16 = w.qlat16;
  a.R = R;
  a.TG = T * s.G;
  a.nl = 1;
  a.tauf = w.tauf;
  a.cap = pl.cap;
  a.flat = true;
  a.ns = pl.ns;
  a.fs_keys = pl.keys;
  a.fs_split = pl.split;
  a.fs_rb = pl.rb;
  a.fb_rows = w.fb_rows;
  a.fb_n = w.fb_n;
  set_header_check(s, d, L, index, w.status);

#define FS_CHECK(what)                                                               \
  do {                                                                               \
    hipError_t e_ = hipGetLastError();                                               \
    if (e_ != hipSuccess) {                                                          \
      snprintf(err, errlen, "%s launch failed: %s", what, hipGetErrorString(e_));    \
      return LSA_ERR_HIP;                                                            \
    }                                                                                \
  } while (0)

  prof_begin(LSA_STAGE_PROJECT, st);
  hipLaunchKernelGGL((pf_qproj_kernel<KT, DL>), dim3((unsigned)R), dim3(256), 0, st, a);
  prof_end(LSA_STAGE_PROJECT, st);
  FS_CHECK("query projection");
  prof_begin(LSA_STAGE_SAMPLE, st);
  {
    const int64_t waves = (int64_t)d.n_kv_heads * ((a.TG + 31) / 32);
    const int64_t blocks = (waves + kFsBlock / 64 - 1) / (kFsBlock / 64);
    hipLaunchKernelGGL((fs_tau_kernel<DL>), dim3((unsigned)blocks), dim3(kFsBlock), 0, st, a);
  }
  prof_end(LSA_STAGE_SAMPLE, st);
  FS_CHECK("thresholds");
  prof_begin(LSA_STAGE_FLAT, st);
  {
    const int64_t blocks = (int64_t)d.n_kv_heads * pl.rb * pl.split;
    hipLaunchKernelGGL((fs_scan_kernel<DL>), dim3((unsigned)blocks), dim3(kFsBlock), 0, st, a);
  }
  prof_end(LSA_STAGE_FLAT, st);
  FS_CHECK("full scan");
  prof_begin(LSA_STAGE_MERGE, st);
  switch (pl.merge_m) {
    case 1: launch_pf_merge<DL, 1>(a, st); break;
    case 2: launch_pf_merge<DL, 2>(a, st); break;
    case 4: launch_pf_merge<DL, 4>(a, st); break;
    case 8: launch_pf_merge<DL, 8>(a, st); break;
    default: launch_pf_merge<DL, 16>(a, st); break;
  }
  prof_end(LSA_STAGE_MERGE, st);
  FS_CHECK("merge");
#undef FS_CHECK
  return LSA_OK;
}

}  // namespace

PfPlan plan_prefill(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq) {
  PfPlan pl;
  memset(&pl, 0, sizeof(pl));
  pl.ok = false;
  if (d.latent_dtype != LSA_BF16 || (d.d_latent != 32 && d.d_latent != 64)) return pl;
  if (p.beam != LSA_BEAM_PER_PARENT || p.k > 2048 || p.k < 1) return pl;
  const int G = Hq / d.n_kv_heads;
  if ((int64_t)T * G < kPfMinRows) return pl;
  const Layout L = compute_layout(d);
  const int64_t R = (int64_t)T * Hq;
  pl.nl[0] = 1;
  for (int e = 0; e < d.n_levels; ++e) {
    const int F = d.fanout[e];
    if (F > kPfMaxF) return pl;
    pl.be[e] = p.b < F ? p.b : F;
    if (pl.be[e] > kPfMaxB || pl.be[e] < 1) return pl;
    pl.nl[e + 1] = pl.nl[e] * pl.be[e];
  }
  const int nl = pl.nl[d.n_levels];
  if (R * nl >= ((int64_t)1 << 31)) return pl;
  pl.nl_out = 1;
  for (int e = 0; e < d.n_levels; ++e) pl.nl_out *= p.b;
  pl.cap = 3 * (int64_t)p.k;
  int capl = 512;
  while (capl < 2 * p.k) capl <<= 1;
  pl.merge_m = capl / kPfMergeBlock;
  if (pl.merge_m > 16) return pl;
  const double avg_leaf = (double)d.n_keys / (double)L.nodes[d.n_levels];
  // with many small leaves per row, only the leaves with an even child index
  // are sampled (half the sample items), each with twice the samples; with
  // large leaves a row's best keys sit in few leaves and skipping half of
  // them would misplace the threshold
  pl.shalf = (nl >= 64 && avg_leaf <= 64.0) ? 1 : 0;
  pl.spl = clampi((int64_t)ceil(kPfSampleR * avg_leaf / (kPfTarget * p.k)) * (pl.shalf ? 2 : 1), 1, 32);
  for (int e = 0; e < d.n_levels; ++e) {
    const double parents = (double)d.n_kv_heads * (double)L.nodes[e];
    const double tiles = (double)R * pl.nl[e] / parents / 32.0;
    pl.ch[e] = clampi((int64_t)ceil(tiles / (4.0 * kPfNW)), 1, 4096);
  }
  {
    const int lev = d.n_levels - 1;
    const double rows_per_leaf = (double)R * nl / ((double)d.n_kv_heads * (double)L.nodes[lev + 1]);
    const double items = (double)d.fanout[lev] * ceil(rows_per_leaf / 32.0);
    // several items per wave: a short workgroup costs more to dispatch than
    // its items take
    pl.chg = clampi((int64_t)ceil(items / (4.0 * kPfNW)), 1, 4096);
  }
  pl.bytes = carve_prefill(d, pl, R, nullptr, nullptr);
  pl.ok = true;
  return pl;
}

int launch_prefill(const lsa_index_desc& d, const lsa_select_params& p, const PfPlan& pl, const void* index,
                   const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                   float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, char* err, size_t errlen) {
  const bool kb = d.key_dtype == LSA_BF16;
  if (d.d_latent == 64) {
    if (kb) return run_prefill<bf16_t, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, err, errlen);
    return run_prefill<float, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, err, errlen);
  }
  if (kb) return run_prefill<bf16_t, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, err, errlen);
  return run_prefill<float, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, out_leaves, ws, st, err, errlen);
}


FsPlan plan_flat_tiled(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq) {
  FsPlan pl;
  memset(&pl, 0, sizeof(pl));
  pl.ok = false;
  if (d.latent_dtype != LSA_BF16 || (d.d_latent != 32 && d.d_latent != 64)) return pl;
  if (p.k > 2048 || p.k < 1) return pl;
  const int G = Hq / d.n_kv_heads;
  const int64_t TG = (int64_t)T * G, R = (int64_t)T * Hq, N = d.n_keys;
  if (TG < kPfMinRows || R >= ((int64_t)1 << 31)) return pl;
  // about 64 N / ns keys are expected at or above the sampled threshold:
  // aim at 2k, and keep 5k places per row (each half's 32nd best sample
  // sits within a factor 2.5 of its mean far beyond one row in a billion)
  int64_t ns = (32 * N + p.k - 1) / p.k;
  ns = (ns + 31) / 32 * 32;
  if (ns >= N) ns = N;
  pl.ns = ns;
  pl.cap = 5 * (int64_t)p.k < N ? 5 * (int64_t)p.k : N;
  int capl = 512;
  while (capl < 2 * p.k) capl <<= 1;
  pl.merge_m = capl / kPfMergeBlock;
  pl.rb = (int)((TG + kFsRows - 1) / kFsRows);
  // key splits of 16384 keys (2 MiB of bf16 latent): the workgroups of one
  // split are dispatched together and share its keys through L2
  pl.keys = kFsSplitKeys;
  pl.split = (int)((N + pl.keys - 1) / pl.keys);
  pl.bytes = carve_flat_tiled(d, pl, R, nullptr, nullptr);
  pl.ok = true;
  return pl;
}

int launch_flat_tiled(const lsa_index_desc& d, const lsa_select_params& p, const FsPlan& pl, const void* index,
                      const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                      float* out_scores, void* ws, hipStream_t st, char* err, size_t errlen) {
  const bool kb = d.key_dtype == LSA_BF16;
  if (d.d_latent == 64) {
    if (kb) return run_flat_tiled<bf16_t, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, ws, st, err, errlen);
    return run_flat_tiled<float, 64>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, ws, st, err, errlen);
  }
  if (kb) return run_flat_tiled<bf16_t, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, ws, st, err, errlen);
  return run_flat_tiled<float, 32>(d, p, pl, index, queries, q_pos, T, Hq, out_idx, out_scores, ws, st, err, errlen);
}

}  // namespace lsa
