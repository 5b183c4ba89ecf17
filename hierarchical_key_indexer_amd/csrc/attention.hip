// Exact sparse attention over the selected keys.  The page "Latent Sparse
// Attention (LSA): The 72.4x and 22.7x Speedups, and What They Compare
// Against" (section "How does LSA work?", step 3): what a query reads is the
// indexer's far keys, the sink positions and the recent window, and the
// attention computation stays the ordinary one: softmax attention restricted to the keys
// that an lsa_select row lists,
//   out = sum_j softmax_j(scale * q . k_j) v_j   over the entries j >= 0,
// an entry listed twice counting twice, an entry outside [0, N) counting as
// padding and a row with no key giving zeros.
//
// One workgroup per (token, query head).  Pass 1 scores the listed keys: LPK
// lanes read a key row with 16-byte loads (a load instruction covers KPW whole
// rows, four instructions in flight per lane) and reduce their partial dots;
// the scores go to LDS.  The row's maximum and the exponentials follow in LDS.
// Pass 2 reads the value rows the same way: a group of lanes owns one value
// row at a time and accumulates p_j v_j for its slice of the dims; the groups'
// partial outputs are added in LDS.  Everything is fp32 (keys, queries and
// values widened from their stored format).
//
// Few rows (decode) would leave most of the chip idle, so a row's entries are
// then split over S workgroups.  Each writes its partial result (maximum
// score m_s, sum of exp(s_j - m_s), and the unnormalised weighted sum of
// values) to the workspace, and attention_combine_kernel rescales the parts to
// the common maximum M: out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) z_s.
#include <math.h>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kAttBlock = 256;
constexpr int kAttNW = kAttBlock / 64;
constexpr int kAttU = 4;                     // key rows in flight per lane in pass 1

template <typename KT>
struct Row16;
template <>
struct Row16<float> {
  static constexpr int E = 4;                 // elements per 16 bytes
  __device__ static __forceinline__ void widen(const uint4& u, float* x) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
};
template <>
struct Row16<bf16_t> {
  static constexpr int E = 8;
  __device__ static __forceinline__ void widen(const uint4& u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

template <int G>
__device__ __forceinline__ float group_sum_all(float v) {   // every lane of the aligned group of G
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kAttNW; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAttNW; ++i) s += red[i];
  __syncthreads();
  return s;
}

template <typename KT, int D>
__global__ __launch_bounds__(kAttBlock) void sparse_attention_kernel(const KT* queries, const KT* keys,
                                                                     const KT* values, const int32_t* idx,
                                                                     int64_t N, int width, int Hq, int Hkv,
                                                                     float scale, float* out, int split,
                                                                     float* part) {
  constexpr int E = Row16<KT>::E;
  constexpr int LPK = D / E;                  // lanes per row
  constexpr int KPW = 64 / LPK;               // rows per wave and load instruction
  constexpr int NG = kAttBlock / LPK;         // row groups of the block in pass 2
  extern __shared__ __align__(16) float sm[];
  __shared__ float red[kAttNW];
  const int64_t row = blockIdx.x;
  const int sp = blockIdx.y;                  // this workgroup's share of the row
  const int hq = (int)(row % Hq), h = hq / (Hq / Hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lig = lane % LPK, g = lane / LPK;
  const int jlo = (int)((int64_t)width * sp / split), jhi = (int)((int64_t)width * (sp + 1) / split);
  const int32_t* ir = idx + row * width + jlo;
  width = jhi - jlo;                          // from here on: this share of the row
  float* s = sm;                              // [width] scores, then weights
  float* po = sm + ((width + 3) & ~3);        // [NG][D] partial outputs
  // this lane's slice of the query
  float qv[E];
  Row16<KT>::widen(*(const uint4*)(queries + row * D + lig * E), qv);
  const size_t rstride = (size_t)Hkv * D;
  const KT* kb = keys + (size_t)h * D + lig * E;
  const KT* vb = values + (size_t)h * D;
  // pass 1: scores (-inf for a padding entry)
  for (int j0 = w * KPW; j0 < width; j0 += kAttNW * KPW * kAttU) {
    int id[kAttU];
    uint4 kr[kAttU];
#pragma unroll
    for (int u = 0; u < kAttU; ++u) {
      const int j = j0 + u * kAttNW * KPW + g;
      const int x = j < width ? ir[j] : -1;
      id[u] = (x >= 0 && (int64_t)x < N) ? x : -1;   // outside [0, N): padding
    }
#pragma unroll
    for (int u = 0; u < kAttU; ++u)     // a padding entry reads row 0 (dropped)
      kr[u] = *(const uint4*)(kb + (size_t)(id[u] >= 0 ? id[u] : 0) * rstride);
#pragma unroll
    for (int u = 0; u < kAttU; ++u) {
      float x[E];
      Row16<KT>::widen(kr[u], x);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) p = fmaf(qv[e], x[e], p);
      p = group_sum_all<LPK>(p);
      const int j = j0 + u * kAttNW * KPW + g;
      if (lig == 0 && j < width) s[j] = id[u] >= 0 ? scale * p : -__builtin_huge_valf();
    }
  }
  __syncthreads();
  float m = -__builtin_huge_valf();
  for (int j = threadIdx.x; j < width; j += kAttBlock) m = fmaxf(m, s[j]);
  m = block_max(m, red);
  float z = 0.f;
  for (int j = threadIdx.x; j < width; j += kAttBlock) {
    const float p = s[j] == -__builtin_huge_valf() ? 0.f : expf(s[j] - m);
    s[j] = p;
    z += p;
  }
  z = block_sum(z, red);                      // its barriers publish s
  // pass 2: group gr of LPK lanes owns rows gr, gr + NG, ...; lane lig owns
  // dims [lig * E, lig * E + E)
  const int gr = threadIdx.x / LPK;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int j = gr; j < width; j += NG) {
    const float p = s[j];
    if (p == 0.f) continue;
    float x[E];
    Row16<KT>::widen(*(const uint4*)(vb + (size_t)ir[j] * rstride + lig * E), x);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(p, x[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) po[gr * D + lig * E + e] = acc[e];
  __syncthreads();
  if (split == 1) {
    float* o = out + row * D;
    for (int i = threadIdx.x; i < D; i += kAttBlock) {
      float t = 0.f;
      for (int q = 0; q < NG; ++q) t += po[q * D + i];
      o[i] = z > 0.f ? t / z : 0.f;
    }
    return;
  }
  float* pp = part + ((size_t)row * split + sp) * (D + 2);
  for (int i = threadIdx.x; i < D; i += kAttBlock) {
    float t = 0.f;
    for (int q = 0; q < NG; ++q) t += po[q * D + i];
    pp[i] = t;
  }
  if (threadIdx.x == 0) {
    pp[D] = m;                                // -inf for a share with no key
    pp[D + 1] = z;
  }
}

// Parts of a row -> its output (see the file comment).  Wave 0 reads every
// part's maximum and sum once (split <= 64: one lane each) and leaves the
// rescale factors in LDS; every thread then sums its dims over the parts.
template <int D>
__global__ __launch_bounds__(kAttBlock) void attention_combine_kernel(const float* part, int split, float* out) {
  __shared__ float f[64];
  __shared__ float zsum;
  const int64_t row = blockIdx.x;
  const float* pr = part + (size_t)row * split * (D + 2);
  if (threadIdx.x < 64) {
    const int sp = threadIdx.x;
    const float ms = sp < split ? pr[(size_t)sp * (D + 2) + D] : -__builtin_huge_valf();
    const float zs = sp < split ? pr[(size_t)sp * (D + 2) + D + 1] : 0.f;
    float M = ms;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float fs = ms == -__builtin_huge_valf() ? 0.f : expf(ms - M);
    float Z = fs * zs;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) Z += __shfl_xor(Z, o, 64);
    f[sp] = fs;
    if (sp == 0) zsum = Z;
  }
  __syncthreads();
  const float Z = zsum;
  for (int i = threadIdx.x; i < D; i += kAttBlock) {
    float t = 0.f;
#pragma unroll 8
    for (int sp = 0; sp < split; ++sp) t += f[sp] * pr[(size_t)sp * (D + 2) + i];
    out[row * D + i] = Z > 0.f ? t / Z : 0.f;
  }
}

template <typename KT, int D>
int launch_att(const void* q, const void* k, const void* v, const int32_t* idx, int64_t N, int width, int64_t rows,
               int Hq, int Hkv, float scale, float* out, int split, float* part, hipStream_t st, char* err,
               size_t errlen) {
  constexpr int E = Row16<KT>::E;
  constexpr int NG = kAttBlock / (D / E);
  const int wmax = (width + split - 1) / split;
  const size_t lds = (size_t)((wmax + 3) & ~3) * 4 + (size_t)NG * D * 4;
  auto kern = sparse_attention_kernel<KT, D>;
  if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  // rows <= 2^30 (validated), split workgroups per row
  hipLaunchKernelGGL(kern, dim3((unsigned)rows, (unsigned)split), dim3(kAttBlock), lds, st, (const KT*)q,
                     (const KT*)k, (const KT*)v, idx, N, width, Hq, Hkv, scale, out, split, part);
  if (split > 1)
    hipLaunchKernelGGL(attention_combine_kernel<D>, dim3((unsigned)rows), dim3(kAttBlock), 0, st, (const float*)part,
                       split, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "sparse attention launch failed: %s", hipGetErrorString(e));
    return LSA_ERR_HIP;
  }
  return LSA_OK;
}

}  // namespace

int attention_split(int64_t rows, int width) {
  if (rows >= 768) return 1;
  int64_t sp = (768 + rows - 1) / rows;               // one round of workgroups
  const int64_t by_work = width / 64 > 1 ? width / 64 : 1;   // at least 64 entries each
  sp = sp < by_work ? sp : by_work;
  return (int)(sp < 1 ? 1 : (sp > 64 ? 64 : sp));
}

size_t attention_workspace_bytes(const lsa_index_desc& d, int32_t width, int32_t T, int32_t Hq) {
  const int64_t rows = (int64_t)T * Hq;
  const int sp = attention_split(rows, width);
  return sp > 1 ? align_up((size_t)rows * sp * (d.d_head + 2) * 4) : 0;
}

int launch_sparse_attention(const lsa_index_desc& d, const void* q, const void* k, const void* v,
                            const int32_t* idx, int32_t width, int32_t T, int32_t Hq, float scale, float* out,
                            void* ws, hipStream_t st, char* err, size_t errlen) {
  const int64_t rows = (int64_t)T * Hq;
  if (rows == 0) return LSA_OK;
  const int sp = attention_split(rows, width);
  float* part = (float*)ws;
  const bool bf = d.key_dtype == LSA_BF16;
#define LSA_ATT(KT, D) \
  launch_att<KT, D>(q, k, v, idx, d.n_keys, width, rows, Hq, d.n_kv_heads, scale, out, sp, part, st, err, errlen)
  switch (d.d_head) {
    case 64: return bf ? LSA_ATT(bf16_t, 64) : LSA_ATT(float, 64);
    case 128: return bf ? LSA_ATT(bf16_t, 128) : LSA_ATT(float, 128);
    default: return bf ? LSA_ATT(bf16_t, 256) : LSA_ATT(float, 256);
  }
#undef LSA_ATT
}

}  // namespace lsa
