// Host-side internals shared by the ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdio.h>
#include <string.h>
#include <math.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

constexpr int kMaxLevels = 4;
constexpr size_t kAlign = 256;
constexpr int kMaxLeaves = 4096;   // b^L (or b) cap of a query's leaf list
constexpr int kMaxK = 4096;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Byte offsets of the index blob sections (the layout lsa.h specifies).
struct Layout {
  size_t W = 0, perm = 0, latent = 0, total = 0;
  size_t cent[kMaxLevels] = {0, 0, 0, 0};
  size_t cscore[kMaxLevels] = {0, 0, 0, 0};
  size_t offsets[kMaxLevels] = {0, 0, 0, 0};
  int64_t nodes[kMaxLevels + 1] = {1, 0, 0, 0, 0};   // nodes[l] = P_l, nodes[0] = 1
};

inline int latent_elem_bytes(const lsa_index_desc& d) { return d.latent_dtype == LSA_BF16 ? 2 : 4; }
inline int key_elem_bytes(const lsa_index_desc& d) { return d.key_dtype == LSA_BF16 ? 2 : 4; }

inline Layout compute_layout(const lsa_index_desc& d) {
  Layout L;
  const int64_t hk = d.n_kv_heads, n = d.n_keys, dl = d.d_latent, dh = d.d_head;
  const int ls = latent_elem_bytes(d);
  for (int l = 1; l <= d.n_levels; ++l) L.nodes[l] = L.nodes[l - 1] * d.fanout[l - 1];
  size_t cur = 256;
  auto put = [&](size_t& off, size_t bytes) {
    off = cur;
    cur = align_up(cur + bytes);
  };
  put(L.W, (size_t)(hk * dh * dl * 4));
  for (int l = 1; l <= d.n_levels; ++l) put(L.cent[l - 1], (size_t)(hk * L.nodes[l] * dl * 4));
  for (int l = 1; l <= d.n_levels; ++l) put(L.cscore[l - 1], (size_t)(hk * L.nodes[l] * dl * ls));
  for (int l = 1; l <= d.n_levels; ++l) put(L.offsets[l - 1], (size_t)(hk * (L.nodes[l] + 1) * 4));
  put(L.perm, (size_t)(hk * n * 4));
  put(L.latent, (size_t)(hk * n * dl * ls));
  L.total = cur;
  return L;
}

// The 256-byte header, passed by value to the kernel that writes it.
struct BlobHeader {
  uint32_t w[64];
};

// The header lsa.h specifies for a descriptor (build status word 15 = 0).
inline BlobHeader make_header(const lsa_index_desc& d, const Layout& L) {
  BlobHeader hdr;
  memset(&hdr, 0, sizeof(hdr));
  char* hb = (char*)hdr.w;
  memcpy(hb, "LSA1", 4);
  const uint32_t version = 1;
  memcpy(hb + 4, &version, 4);
  memcpy(hb + 8, &d.n_keys, 8);
  const int32_t i32[12] = {d.n_kv_heads, d.d_head, d.d_latent, d.key_dtype, d.latent_dtype, d.n_levels,
                           d.n_levels > 0 ? d.fanout[0] : 0, d.n_levels > 1 ? d.fanout[1] : 0,
                           d.n_levels > 2 ? d.fanout[2] : 0, d.n_levels > 3 ? d.fanout[3] : 0,
                           d.kmeans_iters, 0};
  memcpy(hb + 16, i32, sizeof(i32));
  uint64_t u64[17] = {d.seed, L.total, L.W, L.perm, L.latent};
  for (int l = 0; l < 4; ++l) {
    u64[5 + l] = l < d.n_levels ? L.cent[l] : 0;
    u64[9 + l] = l < d.n_levels ? L.cscore[l] : 0;
    u64[13 + l] = l < d.n_levels ? L.offsets[l] : 0;
  }
  memcpy(hb + 64, u64, sizeof(u64));
  return hdr;
}

// What a select call compares before it reads anything else of a blob: the
// first kHeaderCheckWords header words, except kmeans_iters (word 14) and the
// seed (words 16-17), which select does not depend on.  Word 15, the build
// status, must be 0.
constexpr int kHeaderCheckWords = 20;
constexpr uint32_t kHeaderCheckMask = 0xFFFFFu & ~((1u << 14) | (1u << 16) | (1u << 17));

// Byte offsets of an append pool of `cap` keys per KV head (lsa.h): the leaf
// each appended key joined, then its latent row.
struct PoolLayout {
  size_t leaf = 0, latent = 0, total = 0;
};
inline PoolLayout pool_layout(const lsa_index_desc& d, int64_t cap) {
  PoolLayout P;
  P.leaf = 0;
  P.latent = align_up((size_t)(d.n_kv_heads * cap * 4));
  P.total = align_up(P.latent + (size_t)(d.n_kv_heads * cap * d.d_latent * latent_elem_bytes(d)));
  return P;
}

// Bump allocator over a caller workspace; with base == nullptr it only sizes.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    size_t off = align_up(used);
    used = off + count * sizeof(T);
    return base ? (T*)(base + off) : nullptr;
  }
};

// ---- build -----------------------------------------------------------------
size_t build_workspace_bytes(const lsa_index_desc& d);
int launch_build(const lsa_index_desc& d, const void* keys, const float* W, void* index, void* ws,
                 hipStream_t stream, char* err, size_t errlen);

// ---- incremental upkeep (build.hip) ---------------------------------------------
int launch_append(const lsa_index_desc& d, const void* index, const void* keys, int32_t n_new, int32_t first,
                  void* pool, int32_t cap, hipStream_t stream, char* err, size_t errlen);

// ---- training-free latent map (pca.hip) ---------------------------------------
size_t pca_workspace_bytes(const lsa_index_desc& d);
int launch_pca_covariance(const lsa_index_desc& d, const void* keys, double* cov, void* ws, hipStream_t stream,
                          char* err, size_t errlen);
void pca_map_host(const lsa_index_desc& d, const double* cov, float* W, double* eig);

// ---- exact sparse attention over the selected keys (attention.hip) --------------
constexpr int kMaxAttWidth = 32768;
size_t attention_workspace_bytes(const lsa_index_desc& d, int32_t width, int32_t T, int32_t Hq);
int launch_sparse_attention(const lsa_index_desc& d, const void* q, const void* k, const void* v,
                            const int32_t* idx, int32_t width, int32_t T, int32_t Hq, float scale, float* out,
                            void* ws, hipStream_t stream, char* err, size_t errlen);

// ---- instrumentation ---------------------------------------------------------
void prof_begin(int stage, hipStream_t st);
void prof_end(int stage, hipStream_t st);

// ---- select ------------------------------------------------------------------

// Node-major prefill path (prefill.hip): taken for large query batches when
// the latent is bf16, the beam is per parent and the tree shape fits.
struct PfPlan {
  bool ok;                     // the path applies
  int be[kMaxLevels];          // children kept per parent at each level
  int nl[kMaxLevels + 1];      // slots per query head at each depth (nl[0] = 1)
  int nl_out;                  // out_leaves row width, b^L
  int spl;                     // samples per (query head, leaf)
  int shalf;                   // 1: only leaves with an even child index are sampled
  int64_t cap;                 // appended keys per query head
  int merge_m;                 // merge buffer entries per thread
  int ch[kMaxLevels];          // workgroups per parent at each level
  int chg;                     // workgroups per parent in the gather
  size_t bytes;                // workspace bytes
};
PfPlan plan_prefill(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq);
int launch_prefill(const lsa_index_desc& d, const lsa_select_params& p, const PfPlan& pl, const void* index,
                   const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                   float* out_scores, int32_t* out_leaves, void* ws, hipStream_t st, char* err, size_t errlen);

// Row-tiled full scan (prefill.hip): lsa_flat_select for large query batches
// on a bf16 latent.
struct FsPlan {
  bool ok;                     // the path applies
  int64_t ns;                  // sampled keys per KV head
  int64_t cap;                 // appended keys per query head
  int merge_m;                 // merge buffer entries per thread
  int rb;                      // row blocks (256 query heads) per KV head
  int split;                   // key splits per (KV head, row block)
  int64_t keys;                // keys per split
  size_t bytes;                // workspace bytes
};
FsPlan plan_flat_tiled(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq);
int launch_flat_tiled(const lsa_index_desc& d, const lsa_select_params& p, const FsPlan& pl, const void* index,
                      const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq, int32_t* out_idx,
                      float* out_scores, void* ws, hipStream_t st, char* err, size_t errlen);

struct SelectPlan {
  int64_t qh;          // T * Hq
  int nl_cap;          // leaf-list capacity per query head
  int splits;          // workgroups per query head in the gather (1 = direct)
  int flat_splits;     // workgroups per (token, KV head) in the flat scan
  bool appended;       // appended mode (sorted leaf ids kept for the pool's membership test)
  int g1;              // > 0: split descent with g1 workgroups per query head
  size_t bytes;        // workspace bytes
  PfPlan pf;           // node-major prefill path (pf.ok)
  FsPlan fs;           // row-tiled full scan (fs.ok)
};
// Keys appended after the build (lsa_select_appended): a pool of `cap` keys
// per KV head, the first `n` of them in use.
struct AppendView {
  const void* pool = nullptr;
  int64_t cap = 0;
  int n = 0;
  bool on = false;             // appended mode: the per-query-head path, with the pool's keys
};

SelectPlan plan_select(const lsa_index_desc& d, const lsa_select_params& p, int32_t T, int32_t Hq, bool flat,
                       bool appended = false);
int launch_select(const lsa_index_desc& d, const lsa_select_params& p, const SelectPlan& plan,
                  const void* index, const void* queries, const int32_t* q_pos, int32_t T, int32_t Hq,
                  int32_t* out_idx, float* out_scores, int32_t* out_leaves, void* ws, hipStream_t stream,
                  bool flat, char* err, size_t errlen, const AppendView& app = AppendView());

}  // namespace lsa
