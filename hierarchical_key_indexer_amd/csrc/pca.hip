// Training-free latent map.  The page "Latent Sparse Attention (LSA): The
// 72.4x and 22.7x Speedups, and What They Compare Against" (section "How does
// LSA work?") lists a PCA map as the option that needs no training.  Reading
// taken: per KV head, the d_latent leading eigenvectors of the keys'
// mean-centred covariance are the columns of W_h (the layout lsa_build_index
// takes), eigenvalues descending, each column signed so that its entry of
// largest magnitude (lowest row on a tie) is positive.
//
// GPU part (lsa_pca_covariance): pca_gram_kernel sums, per chunk of one
// head's keys, the outer products of the keys shifted by the head's first key
// (the shift keeps the centred result free of cancellation when the mean is
// large) and their sum, in fp32; pca_reduce_kernel adds the chunks in fp64 and
// centres.  Host part (lsa_pca_map): a cyclic Jacobi eigensolver in fp64.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "lsa_device.h"
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kPcaBlock = 256;
constexpr int kPcaTile = 32;          // keys per LDS tile
constexpr int kPcaMaxChunks = 256;    // chunks per head
constexpr int kPcaMinRows = 4096;     // rows per chunk, at least

// Chunk ch of head h: rows [r0, r1).  Thread t of pass z owns the 8 x 8 block
// z * 256 + t of the d x d sum (row block / (d / 8), column block % (d / 8)).
template <typename KT>
__global__ __launch_bounds__(kPcaBlock) void pca_gram_kernel(const KT* keys, int64_t N, int Hkv, int d,
                                                             int64_t rows, float* part, float* psum) {
  extern __shared__ __align__(16) float xs[];     // [kPcaTile][d], then the shift [d]
  float* shift = xs + kPcaTile * d;
  const int ch = blockIdx.x, h = blockIdx.y, z = blockIdx.z;
  const int nch = gridDim.x;
  const int64_t r0 = (int64_t)ch * rows, r1 = min(N, r0 + rows);
  const int t = threadIdx.x;
  const int d8 = d / 8;
  const int bi = z * kPcaBlock + t;
  const bool owner = bi < d8 * d8;
  const int br = owner ? bi / d8 : 0, bc = owner ? bi % d8 : 0;
  for (int i = t; i < d; i += kPcaBlock) shift[i] = KeyLoad<KT>::get(keys + (size_t)h * d, i);
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  float sum = 0.f;                                // column t of the shifted sum (pass 0)
  __syncthreads();
  for (int64_t k0 = r0; k0 < r1; k0 += kPcaTile) {
    const int nk = (int)min((int64_t)kPcaTile, r1 - k0);
    for (int e = t; e < kPcaTile * d; e += kPcaBlock) {
      const int kr = e / d, dim = e % d;
      xs[e] = kr < nk ? KeyLoad<KT>::get(keys + ((size_t)(k0 + kr) * Hkv + h) * d, dim) - shift[dim] : 0.f;
    }
    __syncthreads();
    if (owner) {
      for (int kr = 0; kr < kPcaTile; ++kr) {
        const float* x = xs + kr * d;
        float a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[i] = x[8 * br + i];
          b[i] = x[8 * bc + i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
    if (z == 0 && t < d)
      for (int kr = 0; kr < kPcaTile; ++kr) sum += xs[kr * d + t];
    __syncthreads();
  }
  if (owner) {
    float* out = part + ((size_t)h * nch + ch) * d * d;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) out[(size_t)(8 * br + i) * d + 8 * bc + j] = acc[i][j];
  }
  if (z == 0 && t < d) psum[((size_t)h * nch + ch) * d + t] = sum;
}

// cov[h][i][j] = S_ij / N - m_i m_j, with S the shifted outer-product sum and
// m the shifted mean, every sum over chunks in fp64.
__global__ __launch_bounds__(kPcaBlock) void pca_reduce_kernel(const float* part, const float* psum, int64_t N,
                                                               int d, int nch, double* cov) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * kPcaBlock + threadIdx.x;
  if (e >= d * d) return;
  const int i = e / d, j = e % d;
  double g = 0.0, si = 0.0, sj = 0.0;
  for (int c = 0; c < nch; ++c) {
    const size_t hc = (size_t)h * nch + c;
    g += (double)part[hc * d * d + e];
    si += (double)psum[hc * d + i];
    sj += (double)psum[hc * d + j];
  }
  const double n = (double)N;
  cov[(size_t)h * d * d + e] = g / n - (si / n) * (sj / n);
}

struct PcaPlan {
  int nch;
  int64_t rows;
  size_t bytes;
};

PcaPlan plan_pca(const lsa_index_desc& dsc) {
  PcaPlan p;
  const int64_t N = dsc.n_keys;
  int64_t nch = (N + kPcaMinRows - 1) / kPcaMinRows;
  nch = nch < 1 ? 1 : (nch > kPcaMaxChunks ? kPcaMaxChunks : nch);
  p.rows = (N + nch - 1) / nch;
  p.nch = (int)((N + p.rows - 1) / p.rows);
  const size_t d = (size_t)dsc.d_head;
  p.bytes = align_up((size_t)dsc.n_kv_heads * p.nch * d * d * 4) + align_up((size_t)dsc.n_kv_heads * p.nch * d * 4);
  return p;
}

// Symmetric eigenproblem of a (n x n, row-major, overwritten) by cyclic Jacobi
// rotations: on return the diagonal of a holds the eigenvalues and column c
// of v the eigenvector of a[c][c].  Each rotation zeroes one off-diagonal pair
// (p, q): with theta = (a_qq - a_pp) / (2 a_pq), t = sign(theta) / (|theta| +
// sqrt(theta^2 + 1)) is the smaller root of t^2 + 2 theta t - 1 = 0, and
// c = 1 / sqrt(1 + t^2), s = t c.  Sweeps run until the off-diagonal mass is
// below 1e-30 of the total (or 100 sweeps).
void jacobi_eigen(std::vector<double>& a, std::vector<double>& v, int n) {
  v.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
  auto A = [&](int r, int c) -> double& { return a[(size_t)r * n + c]; };
  auto V = [&](int r, int c) -> double& { return v[(size_t)r * n + c]; };
  double total = 0.0;
  for (size_t i = 0; i < a.size(); ++i) total += a[i] * a[i];
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += 2.0 * A(p, q) * A(p, q);
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < n - 1; ++p)
      for (int q = p + 1; q < n; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double theta = (A(q, q) - A(p, p)) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(1.0 + t * t), s = t * c;
        // A <- J^T A J on rows and columns p, q
        for (int k = 0; k < n; ++k) {
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        for (int k = 0; k < n; ++k) {
          const double vkp = V(k, p), vkq = V(k, q);
          V(k, p) = c * vkp - s * vkq;
          V(k, q) = s * vkp + c * vkq;
        }
      }
  }
}

}  // namespace

size_t pca_workspace_bytes(const lsa_index_desc& d) { return plan_pca(d).bytes; }

int launch_pca_covariance(const lsa_index_desc& dsc, const void* keys, double* cov, void* ws, hipStream_t st,
                          char* err, size_t errlen) {
  const PcaPlan pl = plan_pca(dsc);
  const int d = dsc.d_head, Hkv = dsc.n_kv_heads;
  Carver c(ws);
  float* part = c.take<float>((size_t)Hkv * pl.nch * d * d);
  float* psum = c.take<float>((size_t)Hkv * pl.nch * d);
  const int nb = (d / 8) * (d / 8);
  const dim3 grid((unsigned)pl.nch, (unsigned)Hkv, (unsigned)((nb + kPcaBlock - 1) / kPcaBlock));
  const size_t lds = ((size_t)kPcaTile * d + d) * sizeof(float);
  if (dsc.key_dtype == LSA_BF16)
    hipLaunchKernelGGL(pca_gram_kernel<bf16_t>, grid, dim3(kPcaBlock), lds, st, (const bf16_t*)keys, dsc.n_keys,
                       Hkv, d, pl.rows, part, psum);
  else
    hipLaunchKernelGGL(pca_gram_kernel<float>, grid, dim3(kPcaBlock), lds, st, (const float*)keys, dsc.n_keys, Hkv,
                       d, pl.rows, part, psum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "pca_gram_kernel launch failed: %s", hipGetErrorString(e));
    return LSA_ERR_HIP;
  }
  hipLaunchKernelGGL(pca_reduce_kernel, dim3((unsigned)((d * d + kPcaBlock - 1) / kPcaBlock), (unsigned)Hkv),
                     dim3(kPcaBlock), 0, st, part, psum, dsc.n_keys, d, pl.nch, cov);
  e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(err, errlen, "pca_reduce_kernel launch failed: %s", hipGetErrorString(e));
    return LSA_ERR_HIP;
  }
  return LSA_OK;
}

void pca_map_host(const lsa_index_desc& dsc, const double* cov, float* W, double* eig) {
  const int d = dsc.d_head, dl = dsc.d_latent;
  std::vector<double> a, v;
  std::vector<int> order(d);
  for (int h = 0; h < dsc.n_kv_heads; ++h) {
    a.assign(cov + (size_t)h * d * d, cov + (size_t)(h + 1) * d * d);
    // symmetrise (the two halves of a computed covariance agree to rounding)
    for (int i = 0; i < d; ++i)
      for (int j = i + 1; j < d; ++j) {
        const double m = 0.5 * (a[(size_t)i * d + j] + a[(size_t)j * d + i]);
        a[(size_t)i * d + j] = m;
        a[(size_t)j * d + i] = m;
      }
    jacobi_eigen(a, v, d);
    for (int i = 0; i < d; ++i) order[i] = i;
    // descending eigenvalue; equal values keep the lower index first
    for (int i = 1; i < d; ++i) {
      const int x = order[i];
      int j = i - 1;
      while (j >= 0 && a[(size_t)order[j] * d + order[j]] < a[(size_t)x * d + x]) {
        order[j + 1] = order[j];
        --j;
      }
      order[j + 1] = x;
    }
    for (int c2 = 0; c2 < dl; ++c2) {
      const int col = order[c2];
      int rmax = 0;
      for (int r = 1; r < d; ++r)
        if (fabs(v[(size_t)r * d + col]) > fabs(v[(size_t)rmax * d + col])) rmax = r;
      const double sg = v[(size_t)rmax * d + col] < 0.0 ? -1.0 : 1.0;
      for (int r = 0; r < d; ++r) W[((size_t)h * d + r) * dl + c2] = (float)(sg * v[(size_t)r * d + col]);
      if (eig) eig[(size_t)h * dl + c2] = a[(size_t)col * d + col];
    }
  }
}

}  // namespace lsa
