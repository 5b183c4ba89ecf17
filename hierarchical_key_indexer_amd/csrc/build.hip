// Index build for gfx950: latent projection, top-down Lloyd k-means per tree
// node, CSR bucket layout.
//
// Step 1 of "How does LSA work?" (page "Latent Sparse Attention (LSA): The
// 72.4x and 22.7x Speedups, and What They Compare Against"): keys are
// clustered into buckets in a latent space, organised as a hierarchy.  The
// clustering algorithm (Lloyd k-means, seeded init, 10 rounds) and the CSR
// layout are the readings this library takes; they are spelled out in
// include/lsa.h.
//
// Kernels, in launch order for every level l = 1..L:
//   project_kernel          K . W_h -> latent (fp32 accumulate, RNE)       HBM
//   kmeans_init_kernel      seeded Forgy draws per parent (splitmix64)
//   init_centroids_kernel   copy the drawn members' latents
//   kmeans_assign_kernel    nearest centroid per member (+ fixed-point sums) fp32 ALU
//   kmeans_update_kernel    centroid = sum / count (empty keeps its value)
//   csr_count/scan/scatter  stable counting sort of every parent's members
// All reductions are integer (fixed-point sums, counts), so the build is
// deterministic: the same inputs give the same bytes.
#include <string.h>

#include "lsa_device.h"
#include "lsa_internal.h"
#include "select_device.h"

namespace lsa {

// ---------------------------------------------------------------------------
// projection: out = round(X . W) for 64 rows x one head per workgroup
// ---------------------------------------------------------------------------

// X [nrows][nheads][dh]; W [heads/group][dh][DL]; the output row of (row, head)
// is out + ((head_major ? head * nrows + row : row * nheads + head) * DL).
// OUT_BF16: store bf16 bits (uint16) of the RNE rounding; otherwise store
// fp32.  maxabs (if set) receives, by an atomic max over the bit patterns,
// the largest magnitude of the stored values (a NaN orders above +inf).
template <typename KT, int DL, bool OUT_BF16>
__global__ __launch_bounds__(256) void project_kernel(const KT* __restrict__ X, int64_t nrows, int nheads,
                                                      int dh, int group, const float* __restrict__ W,
                                                      void* __restrict__ out, int head_major,
                                                      unsigned int* __restrict__ maxabs) {
  constexpr int TR = 64, TK = 64, CPT = DL / 16;
  __shared__ float xs[TR][TK + 1];
  __shared__ float ws[TK][DL];
  const int head = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * TR;
  const float* Wh = W + (size_t)(head / group) * dh * DL;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][CPT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[r][c] = 0.f;

  for (int k0 = 0; k0 < dh; k0 += TK) {
    for (int i = threadIdx.x; i < TR * TK; i += 256) {
      const int r = i / TK, kk = i % TK;
      const int64_t row = row0 + r;
      xs[r][kk] = row < nrows ? KeyLoad<KT>::get(X + (row * nheads + head) * dh + k0, kk) : 0.f;
    }
    for (int i = threadIdx.x; i < TK * DL; i += 256) ws[i / DL][i % DL] = Wh[(size_t)(k0 + i / DL) * DL + i % DL];
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[CPT];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = xs[ty * 4 + r][kk];
#pragma unroll
      for (int c = 0; c < CPT; ++c) b[c] = ws[kk][tx * CPT + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
    }
    __syncthreads();
  }
  unsigned int mx = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + ty * 4 + r;
    if (row >= nrows) continue;
    const int64_t o = (head_major ? (int64_t)head * nrows + row : row * nheads + head) * DL + tx * CPT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const float v = OUT_BF16 ? round_to_bf16(acc[r][c]) : acc[r][c];
      if (OUT_BF16) {
        ((bf16_t*)out)[o + c] = (bf16_t)(__float_as_uint(v) >> 16);
      } else {
        ((float*)out)[o + c] = v;
      }
      mx = max(mx, __float_as_uint(v) & 0x7FFFFFFFu);
    }
  }
  if (maxabs) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (unsigned int)__shfl_xor((int)mx, o, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(maxabs, mx);
  }
}

// ---------------------------------------------------------------------------
// k-means initial centroids: seeded Forgy draws (splitmix64)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

struct LevelArgs {
  int64_t N;
  int Hkv;
  int64_t Pprev;          // parents (nodes of level l-1)
  int F;                  // children per parent
  int level;              // l (1-based)
  const int* off_prev;    // [Hkv][Pprev+1] or null (level 1: one parent covering [0, N))
  const int* perm_prev;   // [Hkv][N] key index by position, or null (identity)
};

__device__ __forceinline__ void parent_range(const LevelArgs& a, int h, int64_t p, int64_t& start, int64_t& m) {
  if (a.off_prev) {
    const int* o = a.off_prev + (size_t)h * (a.Pprev + 1);
    start = o[p];
    m = (int64_t)o[p + 1] - o[p];
  } else {
    start = 0;
    m = a.N;
  }
}

__device__ __forceinline__ int key_at(const LevelArgs& a, int h, int64_t pos) {
  return a.perm_prev ? a.perm_prev[(size_t)h * a.N + pos] : (int)pos;
}

// One thread per (head, parent): init_key[h][p][c] = key index of child c's
// initial centroid, -1 for a void child.
__global__ void kmeans_init_kernel(LevelArgs a, uint64_t seed, int* __restrict__ init_key) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)a.Hkv * a.Pprev) return;
  const int h = (int)(gid / a.Pprev);
  const int64_t p = gid % a.Pprev;
  int64_t start, m;
  parent_range(a, h, p, start, m);
  int* out = init_key + (size_t)gid * a.F;
  if (m <= a.F) {
    for (int c = 0; c < a.F; ++c) out[c] = c < m ? key_at(a, h, start + c) : -1;
    return;
  }
  const uint64_t tag = ((uint64_t)(h * 16 + a.level) << 32) + (uint64_t)p;
  uint64_t state = seed ^ splitmix_mix(tag + kGamma);
  int chosen = 0;
  // ordinals are kept in `out` until all are drawn, then mapped to key indices
  while (chosen < a.F) {
    state += kGamma;
    const int u = (int)(splitmix_mix(state) % (uint64_t)m);
    bool dup = false;
    for (int i = 0; i < chosen; ++i) dup |= (out[i] == u);
    if (!dup) out[chosen++] = u;
  }
  for (int c = 0; c < a.F; ++c) out[c] = key_at(a, h, start + out[c]);
}

template <typename LT>
__global__ void init_centroids_kernel(LevelArgs a, int DL, const int* __restrict__ init_key,
                                      const LT* __restrict__ lat, float* __restrict__ cent) {
  const int64_t total = (int64_t)a.Hkv * a.Pprev * a.F * DL;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t node = i / DL;            // flattened (h, p*F + c)
    const int j = (int)(i % DL);
    const int h = (int)(node / (a.Pprev * a.F));
    const int key = init_key[node];
    cent[i] = key >= 0 ? Lat<LT>::get(lat + ((size_t)h * a.N + key) * DL, j) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// fixed-point scale of the k-means member sums
// ---------------------------------------------------------------------------

// A member's latent x enters its centroid's sum as round(x * 2^shift), a
// 64-bit integer, so the sums are exact and independent of the order of
// addition (the build is deterministic).  With every |x| < 2^e and at most
// 2^c members (N <= 2^c), shift = 61 - c - e keeps every sum below 2^61 in
// magnitude, whatever the data's scale, and each value is quantised to a step
// of 2^-(61-c) of the largest magnitude (2^-37 at 10M keys).  A non-finite
// latent leaves the sums meaningless; the header then marks the index bad.
struct FixedPoint {
  unsigned int maxabs;    // largest |latent| (fp32 bits), atomic max target
  int shift;
  int nonfinite;          // 1 if some latent value is inf or NaN
  float scale;            // 2^shift
  double inv_scale;       // 2^-shift
};

__global__ void fixed_point_kernel(FixedPoint* fx, int c) {
  if (threadIdx.x != 0) return;
  const unsigned int b = fx->maxabs;
  const int nonfinite = b >= 0x7F800000u;
  // |x| < 2^e: e = biased exponent - 126 (subnormals and zero: -126)
  const int e = (b >> 23) == 0u ? -126 : (int)(b >> 23) - 126;
  int shift = nonfinite ? 0 : 61 - c - e;
  shift = shift > 100 ? 100 : (shift < -100 ? -100 : shift);
  fx->shift = shift;
  fx->nonfinite = nonfinite;
  fx->scale = ldexpf(1.f, shift);
  fx->inv_scale = ldexp(1.0, -shift);
}

// ---------------------------------------------------------------------------
// k-means assignment (+ fixed-point accumulation of the member sums)
// ---------------------------------------------------------------------------

struct AssignArgs {
  LevelArgs lv;
  int S;                            // workgroups per parent
  const void* lat;                  // [Hkv][N][DL] latent (unsorted)
  const float* cent;                // [Hkv][Pprev*F][DL]
  uint8_t* child;                   // [Hkv][N] child id by position
  unsigned long long* gsum;         // [Hkv][Pprev*F][DL] fixed point
  unsigned int* gcnt;               // [Hkv][Pprev*F]
  const FixedPoint* fx;             // scale of the member sums
};

// |mu|^2, summed in index order (one fma per element).
template <int DL>
__device__ __forceinline__ float centroid_norm(const float* mu) {
  float acc = 0.f;
  for (int j = 0; j < DL; ++j) acc = fmaf(mu[j], mu[j], acc);
  return acc;
}

// |mu|^2 - 2 x.mu: the squared distance up to |x|^2, which is common to every
// centroid.  The assignment of the build and the routing of appended keys
// both use exactly this arithmetic, so they agree bit for bit.
template <int DL>
__device__ __forceinline__ float centroid_dist(const float* x, const float* mu, float mm) {
  const float4* cr = (const float4*)mu;
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int j = 0; j < DL / 4; j += 2) {
    const float4 u = cr[j], w = cr[j + 1];
    d0 = fmaf(x[4 * j + 0], u.x, d0); d0 = fmaf(x[4 * j + 1], u.y, d0);
    d0 = fmaf(x[4 * j + 2], u.z, d0); d0 = fmaf(x[4 * j + 3], u.w, d0);
    d1 = fmaf(x[4 * j + 4], w.x, d1); d1 = fmaf(x[4 * j + 5], w.y, d1);
    d1 = fmaf(x[4 * j + 6], w.z, d1); d1 = fmaf(x[4 * j + 7], w.w, d1);
  }
  return fmaf(-2.f, d0 + d1, mm);
}

template <typename LT, int DL, bool ACC, bool LDS_ACC>
__global__ __launch_bounds__(256) void kmeans_assign_kernel(AssignArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int F = a.lv.F;
  float* cs = (float*)smem;                                   // [F][DL]
  float* cn = cs + F * DL;                                    // [F]
  const size_t acc_off = ((size_t)F * DL * 4 + (size_t)F * 4 + 15) / 16 * 16;
  unsigned long long* lsum = (unsigned long long*)(smem + acc_off);   // [F][DL]
  unsigned int* lcnt = (unsigned int*)(lsum + (LDS_ACC ? F * DL : 0));

  const int h = blockIdx.z;
  const int64_t p = blockIdx.y;
  const int s = blockIdx.x;
  int64_t start, m;
  parent_range(a.lv, h, p, start, m);
  if (m == 0) return;
  const int nv = m < F ? (int)m : F;
  const int64_t lo = start + m * s / a.S, hi = start + m * (s + 1) / a.S;
  if (lo >= hi) return;

  const size_t node0 = ((size_t)h * a.lv.Pprev + p) * F;
  const float* cg = a.cent + node0 * DL;
  for (int i = threadIdx.x; i < nv * DL; i += 256) cs[i] = cg[i];
  if (ACC && LDS_ACC) {
    for (int i = threadIdx.x; i < nv * DL; i += 256) lsum[i] = 0ull;
    for (int i = threadIdx.x; i < nv; i += 256) lcnt[i] = 0u;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nv; c += 256) cn[c] = centroid_norm<DL>(cs + c * DL);
  __syncthreads();

  const LT* lat = (const LT*)a.lat + (size_t)h * a.lv.N * DL;
  const float fx_scale = ACC ? a.fx->scale : 0.f;
  for (int64_t pos = lo + threadIdx.x; pos < hi; pos += 256) {
    const int key = key_at(a.lv, h, pos);
    float x[DL];
    const uint4* row = (const uint4*)(lat + (size_t)key * DL);
#pragma unroll
    for (int i = 0; i < DL / Lat<LT>::PER16; ++i) {
      const uint4 v = row[i];
      if (Lat<LT>::PER16 == 8) {
        x[8 * i + 0] = __uint_as_float(v.x << 16); x[8 * i + 1] = __uint_as_float(v.x & 0xFFFF0000u);
        x[8 * i + 2] = __uint_as_float(v.y << 16); x[8 * i + 3] = __uint_as_float(v.y & 0xFFFF0000u);
        x[8 * i + 4] = __uint_as_float(v.z << 16); x[8 * i + 5] = __uint_as_float(v.z & 0xFFFF0000u);
        x[8 * i + 6] = __uint_as_float(v.w << 16); x[8 * i + 7] = __uint_as_float(v.w & 0xFFFF0000u);
      } else {
        x[4 * i + 0] = __uint_as_float(v.x); x[4 * i + 1] = __uint_as_float(v.y);
        x[4 * i + 2] = __uint_as_float(v.z); x[4 * i + 3] = __uint_as_float(v.w);
      }
    }
    // nearest centroid by |mu|^2 - 2 x.mu (|x|^2 is common to all); ties -> lowest c
    float best = __builtin_huge_valf();
    int bc = 0;
    for (int c = 0; c < nv; ++c) {
      const float d = centroid_dist<DL>(x, cs + c * DL, cn[c]);
      if (d < best) { best = d; bc = c; }
    }
    a.child[(size_t)h * a.lv.N + pos] = (uint8_t)bc;
    if (ACC) {
      if (LDS_ACC) {
#pragma unroll
        for (int j = 0; j < DL; ++j)
          atomicAdd(&lsum[bc * DL + j], (unsigned long long)__float2ll_rn(x[j] * fx_scale));
        atomicAdd(&lcnt[bc], 1u);
      } else {
        unsigned long long* gs = a.gsum + (node0 + bc) * DL;
#pragma unroll
        for (int j = 0; j < DL; ++j) atomicAdd(&gs[j], (unsigned long long)__float2ll_rn(x[j] * fx_scale));
        atomicAdd(&a.gcnt[node0 + bc], 1u);
      }
    }
  }
  if (ACC && LDS_ACC) {
    __syncthreads();
    for (int i = threadIdx.x; i < nv * DL; i += 256)
      if (lcnt[i / DL] != 0u) atomicAdd(&a.gsum[node0 * DL + i], lsum[i]);
    for (int i = threadIdx.x; i < nv; i += 256)
      if (lcnt[i] != 0u) atomicAdd(&a.gcnt[node0 + i], lcnt[i]);
  }
}

// One wave per child node: centroid = sum / count when count > 0; then the
// accumulators are cleared for the next round.
__global__ __launch_bounds__(256) void kmeans_update_kernel(int64_t nodes, int DL, float* __restrict__ cent,
                                                            unsigned long long* __restrict__ gsum,
                                                            unsigned int* __restrict__ gcnt,
                                                            const FixedPoint* __restrict__ fx) {
  const int64_t node = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (node >= nodes) return;
  const double inv_scale = fx->inv_scale;
  const unsigned int cnt = gcnt[node];
  __builtin_amdgcn_wave_barrier();
  if (cnt != 0u) {
    for (int j = lane; j < DL; j += 64) {
      const long long s = (long long)gsum[node * DL + j];
      cent[node * DL + j] = (float)(((double)s * inv_scale) / (double)cnt);
      gsum[node * DL + j] = 0ull;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) gcnt[node] = 0u;
}

// ---------------------------------------------------------------------------
// CSR: stable counting sort of each parent's members by child id
// ---------------------------------------------------------------------------

struct CsrArgs {
  LevelArgs lv;
  int S;                       // workgroups per parent
  const uint8_t* child;        // [Hkv][N] by position
  int* cnt;                    // [Hkv][Pprev][S][F] counts, then (after scan) bases
  int* off_out;                // [Hkv][Pprev*F + 1] offsets of level l
  int* perm_out;               // [Hkv][N]
  const void* lat;             // unsorted latent (final level only)
  void* lat_out;               // CSR latent (final level only), or null
  int row_bytes;               // DL * latent element bytes
};

__global__ __launch_bounds__(256) void csr_count_kernel(CsrArgs a) {
  __shared__ unsigned int hist[256];
  const int h = blockIdx.z;
  const int64_t p = blockIdx.y;
  const int s = blockIdx.x, F = a.lv.F;
  int64_t start, m;
  parent_range(a.lv, h, p, start, m);
  for (int i = threadIdx.x; i < F; i += 256) hist[i] = 0u;
  __syncthreads();
  const int64_t lo = start + m * s / a.S, hi = start + m * (s + 1) / a.S;
  const uint8_t* ch = a.child + (size_t)h * a.lv.N;
  for (int64_t pos = lo + threadIdx.x; pos < hi; pos += 256) atomicAdd(&hist[ch[pos]], 1u);
  __syncthreads();
  int* out = a.cnt + (((size_t)h * a.lv.Pprev + p) * a.S + s) * F;
  for (int i = threadIdx.x; i < F; i += 256) out[i] = (int)hist[i];
}

// One workgroup per parent: exclusive scan of the counts in (child, split)
// order -> the first row of every (split, child) run, and the level offsets.
__global__ __launch_bounds__(256) void csr_scan_kernel(CsrArgs a) {
  __shared__ int wsum[4];
  const int h = blockIdx.y;
  const int64_t p = blockIdx.x;
  const int F = a.lv.F, S = a.S;
  int64_t start, m;
  parent_range(a.lv, h, p, start, m);
  int* c = a.cnt + ((size_t)h * a.lv.Pprev + p) * S * F;
  const int items = F * S;                       // item i = (child i / S, split i % S)
  const int per = (items + 255) / 256;
  const int i0 = min(items, (int)threadIdx.x * per), i1 = min(items, i0 + per);
  int sum = 0;
  for (int i = i0; i < i1; ++i) sum += c[(i % S) * F + i / S];
  int total;
  int run = block_exclusive_scan<256>(sum, wsum, &total) + (int)start;
  for (int i = i0; i < i1; ++i) {
    const int idx = (i % S) * F + i / S;
    const int v = c[idx];
    if (i % S == 0) a.off_out[(size_t)h * (a.lv.Pprev * F + 1) + p * F + i / S] = run;
    c[idx] = run;
    run += v;
  }
  if (p == a.lv.Pprev - 1 && threadIdx.x == 0)
    a.off_out[(size_t)h * (a.lv.Pprev * F + 1) + a.lv.Pprev * F] = (int)(start + m);
}

// Scatter in member order: rank among same-child members = earlier chunks
// (running count) + earlier waves of this chunk + earlier lanes of this wave.
__global__ __launch_bounds__(256) void csr_scatter_kernel(CsrArgs a) {
  __shared__ int run[256];
  __shared__ int wc[4][256];
  const int h = blockIdx.z;
  const int64_t p = blockIdx.y;
  const int s = blockIdx.x, F = a.lv.F;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t start, m;
  parent_range(a.lv, h, p, start, m);
  const int* base = a.cnt + (((size_t)h * a.lv.Pprev + p) * a.S + s) * F;
  for (int i = threadIdx.x; i < F; i += 256) run[i] = base[i];
  for (int i = threadIdx.x; i < 4 * 256; i += 256) (&wc[0][0])[i] = 0;
  __syncthreads();
  const int64_t lo = start + m * s / a.S, hi = start + m * (s + 1) / a.S;
  const uint8_t* ch = a.child + (size_t)h * a.lv.N;
  int* perm_out = a.perm_out + (size_t)h * a.lv.N;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = lo; c0 < hi; c0 += 256) {
    const int64_t pos = c0 + threadIdx.x;
    const bool valid = pos < hi;
    const int c = valid ? ch[pos] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bb = __ballot(valid && ((c >> b) & 1));
      same &= ((c >> b) & 1) ? bb : ~bb;
    }
    const int rank_w = __popcll(same & lt_mask);
    if (valid && rank_w == 0) wc[w][c] = __popcll(same);
    __syncthreads();
    if (valid) {
      int r = run[c] + rank_w;
      for (int ww = 0; ww < w; ++ww) r += wc[ww][c];
      const int key = key_at(a.lv, h, pos);
      perm_out[r] = key;
      if (a.lat_out) {
        const uint4* src = (const uint4*)((const char*)a.lat + ((size_t)h * a.lv.N + key) * a.row_bytes);
        uint4* dst = (uint4*)((char*)a.lat_out + ((size_t)h * a.lv.N + r) * a.row_bytes);
        for (int q = 0; q < a.row_bytes / 16; ++q) dst[q] = src[q];
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < F; i += 256) {
      run[i] += wc[0][i] + wc[1][i] + wc[2][i] + wc[3][i];
      wc[0][i] = wc[1][i] = wc[2][i] = wc[3][i] = 0;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// incremental upkeep: keys appended after the build
// ---------------------------------------------------------------------------

struct AppendArgs {
  const void* keys;                // [n_new][Hkv][d_head] key dtype
  int first;                       // pool slot of keys[0]
  int d_head;
  const float* W;                  // [Hkv][d_head][DL] (the blob's latent map)
  const float* cent[kMaxLevels];   // [Hkv][P_l][DL] stored centroids
  const int* off[kMaxLevels];      // [Hkv][P_l + 1] CSR ranges (non-empty children)
  int F[kMaxLevels];
  int64_t P[kMaxLevels];
  int L;
  int* pool_leaf;                  // [Hkv][cap]
  void* pool_lat;                  // [Hkv][cap][DL]
  int64_t cap;
  const uint32_t* hdr;             // the blob's header and the words it must hold
  uint32_t hx[kHeaderCheckWords];
};

// One workgroup per (appended key, KV head).  The key's latent is computed
// as the build computes every key's (fp32 fma over d_head in index order,
// one rounding to the latent dtype), then it descends from the root: at each
// level the child of the current node with the smallest |mu|^2 - 2 x.mu
// (the build's own assignment arithmetic) among the children that hold keys,
// ties to the lowest child.  The pool slot gets the leaf and the latent; a
// blob whose header does not match leaves the slot's leaf at -1 (never a
// member of anything).
template <typename KT, typename LT, int DL>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ float xk[256];
  __shared__ __align__(16) float x[DL];
  __shared__ u64 wmin[4];
  const int i = blockIdx.x, h = blockIdx.y, Hkv = gridDim.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t slot = (size_t)h * a.cap + a.first + i;
  if (!header_words_match(a.hdr, a.hx)) {      // block-uniform
    if (threadIdx.x == 0) a.pool_leaf[slot] = -1;
    return;
  }
  const KT* key = (const KT*)a.keys + ((size_t)i * Hkv + h) * a.d_head;
  for (int k = threadIdx.x; k < a.d_head; k += 256) xk[k] = KeyLoad<KT>::get(key, k);
  __syncthreads();
  if (threadIdx.x < DL) {
    const float* Wh = a.W + (size_t)h * a.d_head * DL + threadIdx.x;
    float acc = 0.f;
    for (int k = 0; k < a.d_head; ++k) acc = fmaf(xk[k], Wh[(size_t)k * DL], acc);
    const float v = Lat<LT>::PER16 == 8 ? round_to_bf16(acc) : acc;
    x[threadIdx.x] = v;
    if (Lat<LT>::PER16 == 8) ((bf16_t*)a.pool_lat)[slot * DL + threadIdx.x] = (bf16_t)(__float_as_uint(v) >> 16);
    else ((float*)a.pool_lat)[slot * DL + threadIdx.x] = v;
  }
  __syncthreads();
  int64_t node = 0;
  for (int l = 0; l < a.L; ++l) {
    const int F = a.F[l];
    const int64_t kid = node * F + threadIdx.x;
    u64 key = ~0ull;
    if ((int)threadIdx.x < F) {
      const int* off = a.off[l] + (size_t)h * (a.P[l] + 1);
      if (off[kid + 1] > off[kid]) {
        const float* mu = a.cent[l] + ((size_t)h * a.P[l] + kid) * DL;
        const float d = centroid_dist<DL>(x, mu, centroid_norm<DL>(mu));
        key = ((u64)order_u32(d) << 32) | (u64)threadIdx.x;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const u64 y = ((u64)(uint32_t)__shfl_xor((int)(key >> 32), o, 64) << 32) |
                    (uint32_t)__shfl_xor((int)(uint32_t)key, o, 64);
      key = y < key ? y : key;
    }
    if (lane == 0) wmin[w] = key;
    __syncthreads();
    u64 m = wmin[0];
    for (int ww = 1; ww < 4; ++ww) m = wmin[ww] < m ? wmin[ww] : m;
    __syncthreads();
    if (m == ~0ull) {                          // no child holds keys (not for a node that holds some)
      node = -1;
      break;
    }
    node = node * F + (int64_t)(uint32_t)m;
  }
  if (threadIdx.x == 0) a.pool_leaf[slot] = (int)node;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void copy_u32_kernel(uint32_t* dst, const uint32_t* src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) dst[i] = src[i];
}

__global__ void cscore_kernel(const float* cent, void* out, int64_t n, int bf16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (bf16) ((bf16_t*)out)[i] = (bf16_t)f32_to_bf16_bits(cent[i]);
    else ((float*)out)[i] = cent[i];
  }
}

// Word 15 of the header is the build status: 0, or 1 when a latent value was
// not finite (select then refuses the index).
__global__ void header_kernel(BlobHeader hdr, const FixedPoint* fx, uint32_t* out) {
  if (threadIdx.x < 64) out[threadIdx.x] = threadIdx.x == 15 ? (uint32_t)fx->nonfinite : hdr.w[threadIdx.x];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

int grid_for(int64_t n, int block = 256, int cap = 65536) {
  int64_t g = (n + block - 1) / block;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

int ceil_log2(int64_t n) {
  int b = 0;
  while ((int64_t(1) << b) < n) ++b;
  return b;
}

int splits_for(int64_t n, int64_t parents, int64_t per_wg) {
  int64_t s = (n + parents * per_wg - 1) / (parents * per_wg);
  return (int)(s < 1 ? 1 : (s > 4096 ? 4096 : s));
}

struct BuildWsPtrs {
  void* lat;
  int* perm[2];
  uint8_t* child;
  int* init_key;
  unsigned long long* gsum;
  unsigned int* gcnt;
  int* csr_cnt;
  FixedPoint* fx;
};

size_t carve_build(const lsa_index_desc& d, void* base, BuildWsPtrs* w) {
  const Layout L = compute_layout(d);
  const int64_t hk = d.n_kv_heads, n = d.n_keys, dl = d.d_latent;
  int64_t csr_items = 0;
  for (int l = 1; l <= d.n_levels; ++l) {
    const int64_t pp = L.nodes[l - 1];
    const int S = splits_for(n, pp, 8192);
    csr_items = csr_items > pp * S * d.fanout[l - 1] ? csr_items : pp * S * d.fanout[l - 1];
  }
  Carver c(base);
  BuildWsPtrs t;
  t.lat = c.take<char>((size_t)(hk * n * dl * latent_elem_bytes(d)));
  t.perm[0] = c.take<int>((size_t)(hk * n));
  t.perm[1] = c.take<int>((size_t)(hk * n));
  t.child = c.take<uint8_t>((size_t)(hk * n));
  t.init_key = c.take<int>((size_t)(hk * L.nodes[d.n_levels]));
  t.gsum = c.take<unsigned long long>((size_t)(hk * L.nodes[d.n_levels] * dl));
  t.gcnt = c.take<unsigned int>((size_t)(hk * L.nodes[d.n_levels]));
  t.csr_cnt = c.take<int>((size_t)(hk * csr_items));
  t.fx = c.take<FixedPoint>(1);
  if (w) *w = t;
  return align_up(c.used);
}

#define LSA_LAUNCH_CHECK()                                                        \
  do {                                                                            \
    hipError_t e_ = hipGetLastError();                                            \
    if (e_ != hipSuccess) {                                                       \
      snprintf(err, errlen, "HIP launch failed: %s", hipGetErrorString(e_));      \
      return LSA_ERR_HIP;                                                         \
    }                                                                             \
  } while (0)

template <typename KT, typename LT>
int run_build(const lsa_index_desc& d, const void* keys, const float* W, void* index, void* ws,
              hipStream_t st, char* err, size_t errlen) {
  const Layout L = compute_layout(d);
  BuildWsPtrs w;
  carve_build(d, ws, &w);
  char* blob = (char*)index;
  const int64_t N = d.n_keys, hk = d.n_kv_heads;
  const int DL = d.d_latent;
  const bool lat_bf16 = d.latent_dtype == LSA_BF16;

  // every byte of the blob is defined (section padding included)
  {
    const int64_t nb = (int64_t)(L.total / 4);
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(nb)), dim3(256), 0, st, (uint32_t*)blob, 0u, nb);
    LSA_LAUNCH_CHECK();
  }
  // latent keys [Hkv][N][DL], their largest magnitude, the fixed-point scale
  {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, st, (uint32_t*)w.fx, 0u, (int64_t)1);
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)hk);
    unsigned int* mx = &w.fx->maxabs;
    if (DL == 64) {
      if (lat_bf16) hipLaunchKernelGGL((project_kernel<KT, 64, true>), grid, dim3(256), 0, st, (const KT*)keys, N, (int)hk, d.d_head, 1, W, w.lat, 1, mx);
      else hipLaunchKernelGGL((project_kernel<KT, 64, false>), grid, dim3(256), 0, st, (const KT*)keys, N, (int)hk, d.d_head, 1, W, w.lat, 1, mx);
    } else {
      if (lat_bf16) hipLaunchKernelGGL((project_kernel<KT, 32, true>), grid, dim3(256), 0, st, (const KT*)keys, N, (int)hk, d.d_head, 1, W, w.lat, 1, mx);
      else hipLaunchKernelGGL((project_kernel<KT, 32, false>), grid, dim3(256), 0, st, (const KT*)keys, N, (int)hk, d.d_head, 1, W, w.lat, 1, mx);
    }
    hipLaunchKernelGGL(fixed_point_kernel, dim3(1), dim3(64), 0, st, w.fx, ceil_log2(N));
    LSA_LAUNCH_CHECK();
  }
  // the latent map travels with the index
  {
    const int64_t nw = hk * d.d_head * DL;
    hipLaunchKernelGGL(copy_u32_kernel, dim3(grid_for(nw)), dim3(256), 0, st, (uint32_t*)(blob + L.W), (const uint32_t*)W, nw);
    LSA_LAUNCH_CHECK();
  }
  {
    const int64_t ng = hk * L.nodes[d.n_levels] * DL * 2;
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(ng)), dim3(256), 0, st, (uint32_t*)w.gsum, 0u, ng);
    const int64_t nc = hk * L.nodes[d.n_levels];
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(nc)), dim3(256), 0, st, (uint32_t*)w.gcnt, 0u, nc);
    LSA_LAUNCH_CHECK();
  }
  for (int l = 1; l <= d.n_levels; ++l) {
    LevelArgs lv;
    lv.N = N;
    lv.Hkv = (int)hk;
    lv.Pprev = L.nodes[l - 1];
    lv.F = d.fanout[l - 1];
    lv.level = l;
    lv.off_prev = l == 1 ? nullptr : (const int*)(blob + L.offsets[l - 2]);
    lv.perm_prev = l == 1 ? nullptr : w.perm[l % 2];
    int* perm_out = l == d.n_levels ? (int*)(blob + L.perm) : w.perm[(l + 1) % 2];
    float* cent = (float*)(blob + L.cent[l - 1]);
    const int64_t nchild = lv.Pprev * lv.F;

    hipLaunchKernelGGL(kmeans_init_kernel, dim3(grid_for(hk * lv.Pprev, 64)), dim3(64), 0, st, lv, d.seed, w.init_key);
    hipLaunchKernelGGL((init_centroids_kernel<LT>), dim3(grid_for(hk * nchild * DL)), dim3(256), 0, st, lv, DL,
                       (const int*)w.init_key, (const LT*)w.lat, cent);
    LSA_LAUNCH_CHECK();

    AssignArgs aa;
    aa.lv = lv;
    aa.S = splits_for(N, lv.Pprev, 4096);
    aa.lat = w.lat;
    aa.cent = cent;
    aa.child = w.child;
    aa.gsum = w.gsum;
    aa.gcnt = w.gcnt;
    aa.fx = w.fx;
    const size_t base_lds = align_up((size_t)lv.F * DL * 4 + lv.F * 4, 16);
    const size_t lds_acc = base_lds + (size_t)lv.F * DL * 8 + lv.F * 4;
    const bool use_lds_acc = lds_acc <= 64 * 1024;
    dim3 agrid((unsigned)aa.S, (unsigned)lv.Pprev, (unsigned)hk);
    for (int it = 0; it <= d.kmeans_iters; ++it) {
      const bool acc = it < d.kmeans_iters;
#define LSA_ASSIGN(DLV)                                                                                           \
  if (acc && use_lds_acc)                                                                                         \
    hipLaunchKernelGGL((kmeans_assign_kernel<LT, DLV, true, true>), agrid, dim3(256), lds_acc, st, aa);           \
  else if (acc)                                                                                                   \
    hipLaunchKernelGGL((kmeans_assign_kernel<LT, DLV, true, false>), agrid, dim3(256), base_lds, st, aa);         \
  else                                                                                                            \
    hipLaunchKernelGGL((kmeans_assign_kernel<LT, DLV, false, false>), agrid, dim3(256), base_lds, st, aa);
      if (DL == 64) { LSA_ASSIGN(64) } else { LSA_ASSIGN(32) }
#undef LSA_ASSIGN
      LSA_LAUNCH_CHECK();
      if (acc) {
        const int64_t nodes = hk * nchild;
        hipLaunchKernelGGL(kmeans_update_kernel, dim3((unsigned)((nodes + 3) / 4)), dim3(256), 0, st, nodes, DL, cent,
                           w.gsum, w.gcnt, (const FixedPoint*)w.fx);
        LSA_LAUNCH_CHECK();
      }
    }

    CsrArgs ca;
    ca.lv = lv;
    ca.S = splits_for(N, lv.Pprev, 8192);
    ca.child = w.child;
    ca.cnt = w.csr_cnt;
    ca.off_out = (int*)(blob + L.offsets[l - 1]);
    ca.perm_out = perm_out;
    ca.lat = w.lat;
    ca.lat_out = l == d.n_levels ? (void*)(blob + L.latent) : nullptr;
    ca.row_bytes = DL * latent_elem_bytes(d);
    hipLaunchKernelGGL(csr_count_kernel, dim3((unsigned)ca.S, (unsigned)lv.Pprev, (unsigned)hk), dim3(256), 0, st, ca);
    hipLaunchKernelGGL(csr_scan_kernel, dim3((unsigned)lv.Pprev, (unsigned)hk), dim3(256), 0, st, ca);
    hipLaunchKernelGGL(csr_scatter_kernel, dim3((unsigned)ca.S, (unsigned)lv.Pprev, (unsigned)hk), dim3(256), 0, st, ca);
    LSA_LAUNCH_CHECK();
  }
  for (int l = 1; l <= d.n_levels; ++l) {
    const int64_t n = hk * L.nodes[l] * DL;
    hipLaunchKernelGGL(cscore_kernel, dim3(grid_for(n)), dim3(256), 0, st, (const float*)(blob + L.cent[l - 1]),
                       (void*)(blob + L.cscore[l - 1]), n, lat_bf16 ? 1 : 0);
  }
  LSA_LAUNCH_CHECK();

  const BlobHeader hdr = make_header(d, L);
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, st, hdr, (const FixedPoint*)w.fx, (uint32_t*)blob);
  LSA_LAUNCH_CHECK();
  return LSA_OK;
}

}  // namespace

size_t build_workspace_bytes(const lsa_index_desc& d) { return carve_build(d, nullptr, nullptr); }

int launch_append(const lsa_index_desc& d, const void* index, const void* keys, int32_t n_new, int32_t first,
                  void* pool, int32_t cap, hipStream_t st, char* err, size_t errlen) {
  if (n_new == 0) return LSA_OK;
  const Layout L = compute_layout(d);
  const PoolLayout PL = pool_layout(d, cap);
  const char* blob = (const char*)index;
  AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.keys = keys;
  a.first = first;
  a.d_head = d.d_head;
  a.W = (const float*)(blob + L.W);
  for (int l = 0; l < d.n_levels; ++l) {
    a.cent[l] = (const float*)(blob + L.cent[l]);
    a.off[l] = (const int*)(blob + L.offsets[l]);
    a.F[l] = d.fanout[l];
    a.P[l] = L.nodes[l + 1];
  }
  a.L = d.n_levels;
  a.pool_leaf = (int*)((char*)pool + PL.leaf);
  a.pool_lat = (char*)pool + PL.latent;
  a.cap = cap;
  const BlobHeader want = make_header(d, L);
  a.hdr = (const uint32_t*)index;
  for (int i = 0; i < kHeaderCheckWords; ++i) a.hx[i] = want.w[i];
  const dim3 grid((unsigned)n_new, (unsigned)d.n_kv_heads);
  const bool kb = d.key_dtype == LSA_BF16, lb = d.latent_dtype == LSA_BF16;
#define LSA_APPEND(KT, LT, DLV) hipLaunchKernelGGL((append_kernel<KT, LT, DLV>), grid, dim3(256), 0, st, a)
  if (d.d_latent == 64) {
    if (kb && lb) LSA_APPEND(bf16_t, bf16_t, 64);
    else if (kb) LSA_APPEND(bf16_t, float, 64);
    else if (lb) LSA_APPEND(float, bf16_t, 64);
    else LSA_APPEND(float, float, 64);
  } else {
    if (kb && lb) LSA_APPEND(bf16_t, bf16_t, 32);
    else if (kb) LSA_APPEND(bf16_t, float, 32);
    else if (lb) LSA_APPEND(float, bf16_t, 32);
    else LSA_APPEND(float, float, 32);
  }
#undef LSA_APPEND
  LSA_LAUNCH_CHECK();
  return LSA_OK;
}

int launch_build(const lsa_index_desc& d, const void* keys, const float* W, void* index, void* ws,
                 hipStream_t stream, char* err, size_t errlen) {
  const bool kb = d.key_dtype == LSA_BF16, lb = d.latent_dtype == LSA_BF16;
  if (kb && lb) return run_build<bf16_t, bf16_t>(d, keys, W, index, ws, stream, err, errlen);
  if (kb && !lb) return run_build<bf16_t, float>(d, keys, W, index, ws, stream, err, errlen);
  if (!kb && lb) return run_build<float, bf16_t>(d, keys, W, index, ws, stream, err, errlen);
  return run_build<float, float>(d, keys, W, index, ws, stream, err, errlen);
}

}  // namespace lsa
