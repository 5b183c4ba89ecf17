// Device-side building blocks of the LSA indexer for gfx950 (wave64).
//
//  * number formats: bf16 <-> fp32 (round to nearest even), order-preserving
//    uint32 image of an fp32 score;
//  * rank keys: a 64-bit key (order(score) << 32 | ~index) whose unsigned
//    order is "higher score first, then lower index first", so the best-k
//    set is unique and a radix select over the keys reproduces the tie rule
//    (score descending, index ascending);
//  * block primitives (exclusive scan, the radix-select compaction of an LDS
//    buffer to its k largest keys, bitonic sort);
//  * the streaming top-k buffer used by the gather, merge and flat kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef uint16_t bf16_t;
typedef unsigned long long u64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float round_to_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// Unsigned image of an fp32 value that preserves order; -0 is folded into +0.
__device__ __forceinline__ uint32_t order_u32(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_u32_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Valid rank keys are never 0 (order_u32 of any non-NaN float is > 0x007FFFFF),
// so 0 marks an absent entry.
__device__ __forceinline__ u64 rank_key(float s, int32_t idx) {
  return ((u64)order_u32(s) << 32) | (u64)(~(uint32_t)idx);
}
__device__ __forceinline__ int32_t rank_key_index(u64 k) { return (int32_t)(~(uint32_t)k); }
__device__ __forceinline__ float rank_key_score(u64 k) { return order_u32_to_f32((uint32_t)(k >> 32)); }

// ---------------------------------------------------------------------------
// latent rows: loads of 16 bytes and their dot product with a query slice
// ---------------------------------------------------------------------------

template <typename LT> struct Lat;
template <> struct Lat<float> {
  static constexpr int PER16 = 4;     // elements per 16 bytes
  __device__ static __forceinline__ float dot16(const uint4& v, const float* q) {
    float acc = __uint_as_float(v.x) * q[0];
    acc = fmaf(__uint_as_float(v.y), q[1], acc);
    acc = fmaf(__uint_as_float(v.z), q[2], acc);
    acc = fmaf(__uint_as_float(v.w), q[3], acc);
    return acc;
  }
  __device__ static __forceinline__ float get(const float* row, int i) { return row[i]; }
};
typedef short v2s16 __attribute__((ext_vector_type(2)));

// 8 bf16 latents . 8 bf16 query values (two per dword), fp32 accumulation with
// the packed dot2 instruction (bf16 x bf16 products are exact in fp32).
__device__ __forceinline__ float dot16_bf16x2(const uint4& v, const uint4& q) {
  float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s16, v.x), __builtin_bit_cast(v2s16, q.x), 0.f, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s16, v.y), __builtin_bit_cast(v2s16, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s16, v.z), __builtin_bit_cast(v2s16, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s16, v.w), __builtin_bit_cast(v2s16, q.w), acc, false);
  return acc;
}

// Query slice held as the operand the row dot products want: packed bf16
// pairs for a bf16 latent store (the query latent is bf16-valued there), fp32
// values for an fp32 store.
template <typename LT> struct QSlice;
template <> struct QSlice<bf16_t> {
  uint4 q;
  __device__ __forceinline__ void load(const float* src) {   // 8 bf16-valued floats
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (__float_as_uint(src[2 * i]) >> 16) | (__float_as_uint(src[2 * i + 1]) & 0xFFFF0000u);
    q = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ __forceinline__ float dot(const uint4& v) const { return dot16_bf16x2(v, q); }
};

template <> struct Lat<bf16_t> {
  static constexpr int PER16 = 8;
  __device__ static __forceinline__ float dot16(const uint4& v, const float* q) {
    float acc = __uint_as_float(v.x << 16) * q[0];
    acc = fmaf(__uint_as_float(v.x & 0xFFFF0000u), q[1], acc);
    acc = fmaf(__uint_as_float(v.y << 16), q[2], acc);
    acc = fmaf(__uint_as_float(v.y & 0xFFFF0000u), q[3], acc);
    acc = fmaf(__uint_as_float(v.z << 16), q[4], acc);
    acc = fmaf(__uint_as_float(v.z & 0xFFFF0000u), q[5], acc);
    acc = fmaf(__uint_as_float(v.w << 16), q[6], acc);
    acc = fmaf(__uint_as_float(v.w & 0xFFFF0000u), q[7], acc);
    return acc;
  }
  __device__ static __forceinline__ float get(const bf16_t* row, int i) { return bf16_to_f32(row[i]); }
};

// Keys / queries in their storage format, widened to fp32.
template <typename KT> struct KeyLoad;
template <> struct KeyLoad<float> {
  __device__ static __forceinline__ float get(const float* p, int i) { return p[i]; }
};
template <> struct KeyLoad<bf16_t> {
  __device__ static __forceinline__ float get(const bf16_t* p, int i) { return bf16_to_f32(p[i]); }
};

template <> struct QSlice<float> {
  float q[4];
  __device__ __forceinline__ void load(const float* src) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = src[i];
  }
  __device__ __forceinline__ float dot(const uint4& v) const { return Lat<float>::dot16(v, q); }
};

// Sum over aligned groups of G lanes (G in {1,2,4,8,16}) with DPP moves; the
// first lane of every group (lane % G == 0) receives the group's sum (other
// lanes hold partial sums).  xor-1 and xor-2 quad permutations, then row
// shifts left by 4 and by 8 (lane i reads lane i+4 / i+8 of its 16-lane row).
template <int G>
__device__ __forceinline__ float group_sum_lead(float v) {
  if (G >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  if (G >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  if (G >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xF, 0xF, true));
  if (G >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108, 0xF, 0xF, true));
  static_assert(G <= 16, "groups wider than a DPP row");
  return v;
}

// ---------------------------------------------------------------------------
// wave / block primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ u64 wave_max_u64(u64 v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    u64 o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t mbcnt64(u64 mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive prefix sum of one int per thread over the block; *total gets the
// block sum.  `wsum` is LDS scratch of BLOCK/64 ints.  Contains barriers.
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_scan(int x, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) {
    int s = wsum[i];
    base += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// Exclusive prefix sum in reversed thread order: thread t gets the sum of x
// over threads t+1 .. BLOCK-1.  Contains barriers.
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_scan_rev(int x, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;   // sum over lanes >= lane within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_down(incl, off, 64);
    if (lane + off < 64) incl += o;
  }
  if (lane == 0) wsum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) {
    int s = wsum[i];
    base += (i > w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// LDS scratch of the radix select.
struct RadixScratch {
  uint32_t hist[256];
  int wsum[16];
  u64 wmin[16], wmax[16];
  int digit;
  uint32_t above;
  uint32_t hd;
  uint32_t sel[2][4];          // digit, keys above it, keys in it: two passes in flight
};

__device__ __forceinline__ u64 wave_min_u64(u64 v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    u64 o = __shfl_xor(v, m, 64);
    v = o < v ? o : v;
  }
  return v;
}

// Keep the k largest nonzero keys of buf[0..n) (n <= BLOCK*M, k < n, keys
// unique) in buf[0..k), in no particular order.  Returns a value t such that
// every kept key is >= t and every dropped key is < t (so a future key can
// only belong to the best k if it is > t).  MSB-first radix select on keys
// held in registers: the bits the smallest and largest key share are common
// to all keys and skipped, then 8-bit digits from the highest bit where they
// differ (so the first histogram is spread, not piled into one bin).  All
// threads of the block must call.
template <int BLOCK, int M>
__device__ u64 topk_compact(u64* buf, int n, int k, RadixScratch* sc) {
  constexpr int NW = BLOCK / 64;
  u64 v[M];
  u64 lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int i = threadIdx.x + j * BLOCK;
    v[j] = (i < n) ? buf[i] : 0ull;
    if (v[j] != 0ull) {
      lo = v[j] < lo ? v[j] : lo;
      hi = v[j] > hi ? v[j] : hi;
    }
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if ((threadIdx.x & 63) == 0) {
    sc->wmin[threadIdx.x >> 6] = lo;
    sc->wmax[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  lo = sc->wmin[0];
  hi = sc->wmax[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    lo = sc->wmin[i] < lo ? sc->wmin[i] : lo;
    hi = sc->wmax[i] > hi ? sc->wmax[i] : hi;
  }
  const int top = (lo == hi) ? 0 : 64 - __clzll(lo ^ hi);     // bits [0, top) vary
  u64 mask = top >= 64 ? 0ull : (~0ull << top);
  u64 prefix = lo & mask;
  uint32_t need = (uint32_t)k;
  for (int hb = top; hb > 0;) {
    const int lb = hb > 8 ? hb - 8 : 0;
    const u64 dmask = ((1ull << (hb - lb)) - 1ull);
    for (int i = threadIdx.x; i < 256; i += BLOCK) sc->hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (v[j] != 0ull && (v[j] & mask) == prefix) atomicAdd(&sc->hist[(uint32_t)((v[j] >> lb) & dmask)], 1u);
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      const uint32_t h0 = sc->hist[4 * l], h1 = sc->hist[4 * l + 1], h2 = sc->hist[4 * l + 2],
                     h3 = sc->hist[4 * l + 3];
      const uint32_t s = h0 + h1 + h2 + h3;
      uint32_t incl = s;  // sum over lanes >= l
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = __shfl_down(incl, off, 64);
        if (l + off < 64) incl += o;
      }
      const uint32_t above = incl - s;
      if (above < need && need <= incl) {
        uint32_t acc = above;
        int d;
        uint32_t hd;
        if (acc + h3 >= need) { d = 4 * l + 3; hd = h3; }
        else if ((acc += h3) + h2 >= need) { d = 4 * l + 2; hd = h2; }
        else if ((acc += h2) + h1 >= need) { d = 4 * l + 1; hd = h1; }
        else { acc += h1; d = 4 * l; hd = h0; }
        sc->digit = d;
        sc->above = acc;
        sc->hd = hd;
      }
    }
    __syncthreads();
    const int d = sc->digit;
    need -= sc->above;
    const uint32_t hdv = sc->hd;
    prefix |= (u64)d << lb;
    mask |= dmask << lb;
    __syncthreads();
    if (hdv == need) break;
    hb = lb;
  }
  int mine = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) mine += (v[j] != 0ull && (v[j] & mask) >= prefix) ? 1 : 0;
  int total;
  int pos = block_exclusive_scan<BLOCK>(mine, sc->wsum, &total);
#pragma unroll
  for (int j = 0; j < M; ++j)
    if (v[j] != 0ull && (v[j] & mask) >= prefix) buf[pos++] = v[j];
  __syncthreads();
  return prefix;
}

// Sort buf[0..n) ascending (n <= cap, cap a power of two); slots n..cap-1 are
// filled with ~0.  Block-wide bitonic sort in LDS.
template <int BLOCK>
__device__ void bitonic_sort_asc(u64* buf, int n, int cap) {
  int p = 1;
  while (p < n) p <<= 1;
  if (p > cap) p = cap;
  for (int i = n + threadIdx.x; i < p; i += BLOCK) buf[i] = ~0ull;
  __syncthreads();
  for (int size = 2; size <= p; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (p >> 1); t += BLOCK) {
        const int i = 2 * stride * (t / stride) + (t % stride);
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const u64 a = buf[i], b = buf[j];
        if ((a > b) == up) {
          buf[i] = b;
          buf[j] = a;
        }
      }
      __syncthreads();
    }
  }
}

// LDS scratch of the bucket sort by key index.
constexpr int kSortBuckets = 1024;
struct SortScratch {
  uint32_t cnt[kSortBuckets];
  int wsum[16];
  int big;
};

// One output row from the n unique nonzero rank keys in buf[0..n) (or in
// global src[0..n) when src is given; n <= BLOCK*M): the sink positions, the
// best k keys in ascending index order with their scores (-1 / -inf past the
// last), the window positions.  The keys stay in registers throughout.  The
// k-th key is found by an MSB-first radix select as in topk_compact (with two
// histograms, so a pass takes two barriers).  The kept keys are re-keyed as
// (index << 32 | order(score)), bucketed by index over [0, p] (1024 buckets;
// a bucket is a 32-bit multiply-high of the index, monotone in it, clamped to
// the last) and scattered into buf in bucket order; every key then counts the
// smaller keys of its own bucket, which gives its position in the sorted
// row.  A bucket of more than 64 keys (a very uneven index spread) sends the
// kept set to the bitonic sort instead.  buf[0..cap) is scratch (cap >= n,
// cap >= 2k, a power of two).  The caller's writes to buf must be visible (a barrier before the
// call); all threads of the block call.  DIRECT: the keys are put in order
// in buf itself once every key knows its place, so buf needs only k + 4
// entries (cap is not used); a bucket of more than 64 keys then writes
// nothing of the row and returns false (block-uniform) for the caller to
// take the row another way.  Returns true once the row is written.
template <int BLOCK, int M, bool DIRECT = false>
__device__ bool write_top_k_row(u64* buf, int n, int k, int cap, int p, int sink, int window, int32_t* row,
                                float* scores_row, RadixScratch* sc, SortScratch& ss,
                                const u64* src = nullptr, const u64* pre = nullptr) {
  constexpr int NW = BLOCK / 64;
  constexpr int NB = kSortBuckets;
  static_assert(NB >= 256, "the second radix histogram lives in the bucket counts");
  u64 v[M];
  u64 lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int i = threadIdx.x + j * BLOCK;
    v[j] = (i < n) ? (pre ? pre[j] : src ? src[i] : buf[i]) : 0ull;
    if (v[j] != 0ull) {
      lo = v[j] < lo ? v[j] : lo;
      hi = v[j] > hi ? v[j] : hi;
    }
  }
  u64 mask = 0ull, prefix = 0ull;                 // keep v with (v & mask) >= prefix
  if (n > k) {
    for (int i = threadIdx.x; i < 256; i += BLOCK) {
      sc->hist[i] = 0u;
      ss.cnt[i] = 0u;
    }
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    if ((threadIdx.x & 63) == 0) {
      sc->wmin[threadIdx.x >> 6] = lo;
      sc->wmax[threadIdx.x >> 6] = hi;
    }
    __syncthreads();
    lo = sc->wmin[0];
    hi = sc->wmax[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      lo = sc->wmin[i] < lo ? sc->wmin[i] : lo;
      hi = sc->wmax[i] > hi ? sc->wmax[i] : hi;
    }
    const int top = (lo == hi) ? 0 : 64 - __clzll(lo ^ hi);
    mask = top >= 64 ? 0ull : (~0ull << top);
    prefix = lo & mask;
    uint32_t need = (uint32_t)k;
    // pass i counts into sc->hist (even i) or ss.cnt[0, 256) (odd i) and
    // posts its result in sel[i & 1];
    // wave 0 clears the histogram it has read, ready for pass i + 2, and
    // every thread reads sel[i & 1] before it reaches the next pass's barrier
    int par = 0;
    for (int hb = top; hb > 0; par ^= 1) {
      const int lb = hb > 8 ? hb - 8 : 0;
      const u64 dmask = ((1ull << (hb - lb)) - 1ull);
      uint32_t* h = par ? ss.cnt : sc->hist;
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (v[j] != 0ull && (v[j] & mask) == prefix) atomicAdd(&h[(uint32_t)((v[j] >> lb) & dmask)], 1u);
      __syncthreads();
      if (threadIdx.x < 64) {
        const int l = threadIdx.x;
        const uint32_t h0 = h[4 * l], h1 = h[4 * l + 1], h2 = h[4 * l + 2], h3 = h[4 * l + 3];
        h[4 * l] = 0u;
        h[4 * l + 1] = 0u;
        h[4 * l + 2] = 0u;
        h[4 * l + 3] = 0u;
        const uint32_t s4 = h0 + h1 + h2 + h3;
        uint32_t incl = s4;  // sum over lanes >= l
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          uint32_t o = __shfl_down(incl, off, 64);
          if (l + off < 64) incl += o;
        }
        const uint32_t above = incl - s4;
        if (above < need && need <= incl) {
          uint32_t acc = above;
          int d;
          uint32_t hd;
          if (acc + h3 >= need) { d = 4 * l + 3; hd = h3; }
          else if ((acc += h3) + h2 >= need) { d = 4 * l + 2; hd = h2; }
          else if ((acc += h2) + h1 >= need) { d = 4 * l + 1; hd = h1; }
          else { acc += h1; d = 4 * l; hd = h0; }
          sc->sel[par][0] = (uint32_t)d;
          sc->sel[par][1] = acc;
          sc->sel[par][2] = hd;
        }
      }
      __syncthreads();
      const uint32_t d = sc->sel[par][0];
      need -= sc->sel[par][1];
      const uint32_t hdv = sc->sel[par][2];
      prefix |= (u64)d << lb;
      mask |= dmask << lb;
      if (hdv == need) break;
      hb = lb;
    }
  }
  // re-key the kept keys so an ascending sort orders by index, and count
  // the buckets (every thread has passed the last histogram read)
  const uint64_t span = (uint64_t)(p > 0 ? p : 0) + 1;
  const uint32_t scale = span <= (uint64_t)NB ? 0u : (uint32_t)(((uint64_t)NB << 32) / span);
  auto bucket = [&](u64 key) {
    const uint32_t d = (uint32_t)(key >> 32);
    return (int)min(scale == 0u ? d : __umulhi(d, scale), (uint32_t)(NB - 1));
  };
  for (int b = threadIdx.x; b < NB; b += BLOCK) ss.cnt[b] = 0u;
  if (threadIdx.x == 0) ss.big = 0;
  __syncthreads();
  // a dropped key becomes 0 (a re-keyed key never is: its low word is an
  // order image, > 0x007FFFFF), so v[j] != 0 marks the kept keys from here on
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const bool keep = v[j] != 0ull && (v[j] & mask) >= prefix;
    v[j] = keep ? (((u64)(uint32_t)rank_key_index(v[j]) << 32) | (v[j] >> 32)) : 0ull;
    if (keep) atomicAdd(&ss.cnt[bucket(v[j])], 1u);
  }
  __syncthreads();
  constexpr int PER = NB / BLOCK > 0 ? NB / BLOCK : 1;
  int mine = 0, mx = 0;
  if ((int)threadIdx.x * PER < NB)
    for (int j = 0; j < PER; ++j) {
      const int c = (int)ss.cnt[threadIdx.x * PER + j];
      mine += c;
      mx = c > mx ? c : mx;
    }
  if (mx > 64) ss.big = 1;
  int nk;
  int run = block_exclusive_scan<BLOCK>(mine, ss.wsum, &nk);   // (its barriers publish big)
  if (DIRECT && ss.big) return false;
  if ((int)threadIdx.x * PER < NB)
    for (int j = 0; j < PER; ++j) {
      const int c = (int)ss.cnt[threadIdx.x * PER + j];
      ss.cnt[threadIdx.x * PER + j] = (uint32_t)run;
      run += c;
    }
  __syncthreads();
  // buf is free: every key is in registers
#pragma unroll
  for (int j = 0; j < M; ++j)
    if (v[j] != 0ull) buf[atomicAdd(&ss.cnt[bucket(v[j])], 1u)] = v[j];
  __syncthreads();
  if constexpr (DIRECT) {
    // a key's place is its bucket's start plus the smaller keys in it (as
    // below; entries past the bucket's end are masked, buf holds k + 4);
    // once every place is known, the keys are put in order in buf itself and
    // the row is written from there with coalesced stores
    const uint32_t* hw = (const uint32_t*)buf + 1;
    int rr[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      rr[j] = -1;
      if (v[j] != 0ull) {
        const int b = bucket(v[j]);
        const int st = b == 0 ? 0 : (int)ss.cnt[b - 1], e = (int)ss.cnt[b];
        const uint32_t xi = (uint32_t)(v[j] >> 32);
        int r = st;
        for (int i = st; i < e; i += 4) {
          const uint32_t y0 = hw[2 * i], y1 = hw[2 * i + 2], y2 = hw[2 * i + 4], y3 = hw[2 * i + 6];
          r += (y0 < xi ? 1 : 0) + (i + 1 < e && y1 < xi ? 1 : 0) + (i + 2 < e && y2 < xi ? 1 : 0) +
               (i + 3 < e && y3 < xi ? 1 : 0);
        }
        rr[j] = r;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (rr[j] >= 0) buf[rr[j]] = v[j];
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += BLOCK) {
      if (i < nk) {
        const u64 key = buf[i];
        row[sink + i] = (int32_t)(key >> 32);
        if (scores_row) scores_row[i] = order_u32_to_f32((uint32_t)key);
      } else {
        row[sink + i] = -1;
        if (scores_row) scores_row[i] = -__builtin_huge_valf();
      }
    }
  } else {
    const u64* sorted = buf;
    if (ss.big) {
      bitonic_sort_asc<BLOCK>(buf, nk, cap);
    } else {
      // cnt[b] is now the end of bucket b and its start is the end of b - 1;
      // a key's position is its bucket's start plus the smaller keys in it.
      // The keys land in buf[cap/2, cap/2 + nk) in order, so the row is
      // written with coalesced stores
      u64* out = buf + cap / 2;
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (v[j] != 0ull) {
          const int b = bucket(v[j]);
          const int st = b == 0 ? 0 : (int)ss.cnt[b - 1], e = (int)ss.cnt[b];
          // indices are unique, so the high words alone order the keys; four
          // independent reads per step (entries past e, still inside buf since
          // nk + 3 < cap, are masked)
          const uint32_t xi = (uint32_t)(v[j] >> 32);
          const uint32_t* hw = (const uint32_t*)buf + 1;
          int r = st;
          for (int i = st; i < e; i += 4) {
            const uint32_t y0 = hw[2 * i], y1 = hw[2 * i + 2], y2 = hw[2 * i + 4], y3 = hw[2 * i + 6];
            r += (y0 < xi ? 1 : 0) + (i + 1 < e && y1 < xi ? 1 : 0) + (i + 2 < e && y2 < xi ? 1 : 0) +
                 (i + 3 < e && y3 < xi ? 1 : 0);
          }
          out[r] = v[j];
        }
      __syncthreads();
      sorted = out;
    }
    for (int i = threadIdx.x; i < k; i += BLOCK) {
      if (i < nk) {
        const u64 key = sorted[i];
        row[sink + i] = (int32_t)(key >> 32);
        if (scores_row) scores_row[i] = order_u32_to_f32((uint32_t)key);
      } else {
        row[sink + i] = -1;
        if (scores_row) scores_row[i] = -__builtin_huge_valf();
      }
    }
  }
  const int ns = min(sink, p + 1);
  for (int i = threadIdx.x; i < sink; i += BLOCK) row[i] = i < ns ? i : -1;
  const int w0 = max(sink, p - window + 1);
  const int nw = p - w0 + 1;
  for (int i = threadIdx.x; i < window; i += BLOCK) row[sink + k + i] = i < nw ? w0 + i : -1;
  return true;
}

// The same, with the sort scratch in a static LDS block of its own.  The
// keys come from buf, from src, or (pre) from the M keys each thread already
// holds, key threadIdx.x + j BLOCK in pre[j].
template <int BLOCK, int M>
__device__ void write_top_k_row(u64* buf, int n, int k, int cap, int p, int sink, int window, int32_t* row,
                                float* scores_row, RadixScratch* sc, const u64* src = nullptr,
                                const u64* pre = nullptr) {
  __shared__ SortScratch ss;
  write_top_k_row<BLOCK, M>(buf, n, k, cap, p, sink, window, row, scores_row, sc, ss, src, pre);
}

// A row for a query whose position is outside [0, N): all -1.
template <int BLOCK>
__device__ void write_invalid_row(int width, int k, int32_t* row, float* scores_row) {
  for (int i = threadIdx.x; i < width; i += BLOCK) row[i] = -1;
  if (scores_row)
    for (int i = threadIdx.x; i < k; i += BLOCK) scores_row[i] = -__builtin_huge_valf();
}

}  // namespace lsa
