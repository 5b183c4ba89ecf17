// The C ABI of include/lsa.h: argument validation (always before any HIP
// call), workspace sizing and dispatch to the build / select launchers.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "lsa_internal.h"

// Device scratch of lsa_select_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in); it uses the device address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[LSA_NOALLOC_SCRATCH_BYTES];

namespace lsa {
size_t build_workspace_bytes(const lsa_index_desc& d);

namespace {
struct StageEvents {
  void* start = nullptr;
  void* stop = nullptr;
};
thread_local StageEvents g_stage[8];
}  // namespace

void prof_begin(int stage, hipStream_t st) {
  if (g_stage[stage].start) (void)hipEventRecord((hipEvent_t)g_stage[stage].start, st);
}
void prof_end(int stage, hipStream_t st) {
  if (g_stage[stage].stop) (void)hipEventRecord((hipEvent_t)g_stage[stage].stop, st);
}
}  // namespace lsa

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_err() { g_err[0] = 0; }

int check_desc(const lsa_index_desc* d) {
  if (!d) return fail(LSA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->n_keys < 1 || d->n_keys >= (int64_t(1) << 31))
    return fail(LSA_ERR_UNSUPPORTED, "n_keys = %lld outside [1, 2^31)", (long long)d->n_keys);
  if (d->n_kv_heads < 1 || d->n_kv_heads > 1024)
    return fail(LSA_ERR_UNSUPPORTED, "n_kv_heads = %d outside [1, 1024]", d->n_kv_heads);
  if (d->d_head != 64 && d->d_head != 128 && d->d_head != 256)
    return fail(LSA_ERR_UNSUPPORTED, "d_head = %d not in {64, 128, 256}", d->d_head);
  if (d->d_latent != 32 && d->d_latent != 64)
    return fail(LSA_ERR_UNSUPPORTED, "d_latent = %d not in {32, 64}", d->d_latent);
  if ((d->key_dtype != LSA_F32 && d->key_dtype != LSA_BF16) ||
      (d->latent_dtype != LSA_F32 && d->latent_dtype != LSA_BF16))
    return fail(LSA_ERR_UNSUPPORTED, "dtype codes must be LSA_F32 or LSA_BF16");
  if (d->n_levels < 1 || d->n_levels > 4) return fail(LSA_ERR_UNSUPPORTED, "n_levels = %d outside [1, 4]", d->n_levels);
  int64_t prod = 1;
  for (int l = 0; l < d->n_levels; ++l) {
    if (d->fanout[l] < 2 || d->fanout[l] > 256)
      return fail(LSA_ERR_UNSUPPORTED, "fanout[%d] = %d outside [2, 256]", l, d->fanout[l]);
    if (l == d->n_levels - 1 && prod > 65535)
      return fail(LSA_ERR_UNSUPPORTED, "more than 65535 nodes above the leaf level");
    prod *= d->fanout[l];
    if (prod > (int64_t(1) << 22)) return fail(LSA_ERR_UNSUPPORTED, "product of fanouts exceeds 2^22");
  }
  if (d->kmeans_iters < 0 || d->kmeans_iters > 1000)
    return fail(LSA_ERR_UNSUPPORTED, "kmeans_iters = %d outside [0, 1000]", d->kmeans_iters);
  const double bytes = (double)d->n_keys * d->n_kv_heads * d->d_head * 4.0;
  if (bytes > 4.0e12) return fail(LSA_ERR_UNSUPPORTED, "index too large");
  return LSA_OK;
}

int check_params(const lsa_index_desc* d, const lsa_select_params* p, bool flat) {
  if (!p) return fail(LSA_ERR_INVALID_ARG, "params is NULL");
  if (p->k < 1 || p->k > lsa::kMaxK) return fail(LSA_ERR_UNSUPPORTED, "k = %d outside [1, %d]", p->k, lsa::kMaxK);
  if (p->sink < 0 || p->window < 0) return fail(LSA_ERR_INVALID_ARG, "sink and window must be >= 0");
  if ((int64_t)p->sink + p->k + p->window > (int64_t(1) << 30)) return fail(LSA_ERR_UNSUPPORTED, "row width too large");
  if (flat) return LSA_OK;
  if (p->beam != LSA_BEAM_PER_PARENT && p->beam != LSA_BEAM_GLOBAL)
    return fail(LSA_ERR_INVALID_ARG, "beam = %d is not an lsa_beam", p->beam);
  if (p->b < 1) return fail(LSA_ERR_INVALID_ARG, "b = %d must be >= 1", p->b);
  if (p->beam == LSA_BEAM_PER_PARENT) {
    int64_t cap = 1;
    for (int l = 0; l < d->n_levels; ++l) {
      if (p->b > d->fanout[l]) return fail(LSA_ERR_UNSUPPORTED, "b = %d exceeds fanout[%d] = %d", p->b, l, d->fanout[l]);
      cap *= p->b;
    }
    if (cap > lsa::kMaxLeaves) return fail(LSA_ERR_UNSUPPORTED, "b^n_levels = %lld exceeds %d", (long long)cap, lsa::kMaxLeaves);
  } else if (p->b > 64) {
    return fail(LSA_ERR_UNSUPPORTED, "global beam supports b <= 64");
  }
  return LSA_OK;
}

int check_shape(const lsa_index_desc* d, int32_t T, int32_t Hq, bool flat) {
  if (T < 0) return fail(LSA_ERR_INVALID_ARG, "n_tokens = %d < 0", T);
  if (Hq < 1 || Hq % d->n_kv_heads != 0)
    return fail(LSA_ERR_INVALID_ARG, "n_q_heads = %d is not a positive multiple of n_kv_heads = %d", Hq, d->n_kv_heads);
  const int G = Hq / d->n_kv_heads;
  if (flat && G != 1 && G != 2 && G != 4)
    return fail(LSA_ERR_UNSUPPORTED, "flat scan supports 1, 2 or 4 query heads per KV head (got %d)", G);
  if (Hq > 65535) return fail(LSA_ERR_UNSUPPORTED, "n_q_heads = %d exceeds 65535", Hq);
  if ((int64_t)T * Hq > (int64_t(1) << 30)) return fail(LSA_ERR_UNSUPPORTED, "too many query heads");
  return LSA_OK;
}

}  // namespace

extern "C" {

const char* lsa_last_error(void) { return g_err; }

int32_t lsa_abi_version(void) { return 1; }

int lsa_set_profile_events(int32_t stage, void* start, void* stop) {
  clear_err();
  if (stage < LSA_STAGE_PROJECT || stage > LSA_STAGE_SAMPLE) return fail(LSA_ERR_INVALID_ARG, "unknown stage %d", stage);
  if ((start == nullptr) != (stop == nullptr)) return fail(LSA_ERR_INVALID_ARG, "start and stop must both be set or both NULL");
  lsa::g_stage[stage].start = start;
  lsa::g_stage[stage].stop = stop;
  return LSA_OK;
}

size_t lsa_index_bytes(const lsa_index_desc* desc) {
  clear_err();
  if (check_desc(desc) != LSA_OK) return 0;
  return lsa::compute_layout(*desc).total;
}

size_t lsa_build_workspace_bytes(const lsa_index_desc* desc) {
  clear_err();
  if (check_desc(desc) != LSA_OK) return 0;
  return lsa::build_workspace_bytes(*desc);
}

int lsa_build_index(const lsa_index_desc* desc, const void* keys, const float* W, void* index, size_t index_bytes,
                    void* workspace, size_t workspace_bytes, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc != LSA_OK) return rc;
  if (!keys || !W || !index || !workspace) return fail(LSA_ERR_INVALID_ARG, "keys, W, index and workspace must be non-NULL");
  const size_t need_i = lsa::compute_layout(*desc).total;
  if (index_bytes < need_i)
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "index buffer has %zu bytes, %zu needed", index_bytes, need_i);
  const size_t need_w = lsa::build_workspace_bytes(*desc);
  if (workspace_bytes < need_w)
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, need_w);
  char err[256] = {0};
  rc = lsa::launch_build(*desc, keys, W, index, workspace, (hipStream_t)stream, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

int32_t lsa_select_out_width(const lsa_select_params* params) {
  clear_err();
  if (!params) return fail(LSA_ERR_INVALID_ARG, "params is NULL"), -1;
  return params->sink + params->k + params->window;
}

size_t lsa_select_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                                  int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) || check_params(desc, params, false) || check_shape(desc, n_tokens, n_q_heads, false)) return 0;
  return lsa::plan_select(*desc, *params, n_tokens, n_q_heads, false).bytes;
}

int32_t lsa_select_path(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                        int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) || check_params(desc, params, false) || check_shape(desc, n_tokens, n_q_heads, false)) return -1;
  return lsa::plan_select(*desc, *params, n_tokens, n_q_heads, false).pf.ok ? LSA_PATH_NODE_MAJOR
                                                                           : LSA_PATH_PER_QUERY_HEAD;
}

int32_t lsa_flat_select_path(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                             int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) || check_params(desc, params, true) || check_shape(desc, n_tokens, n_q_heads, true)) return -1;
  return lsa::plan_select(*desc, *params, n_tokens, n_q_heads, true).fs.ok ? LSA_PATH_ROW_TILED
                                                                          : LSA_PATH_PER_QUERY_HEAD;
}

size_t lsa_flat_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                                int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) || check_params(desc, params, true) || check_shape(desc, n_tokens, n_q_heads, true)) return 0;
  return lsa::plan_select(*desc, *params, n_tokens, n_q_heads, true).bytes;
}

static int select_common(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
                         int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
                         float* out_scores, int32_t* out_leaves, void* workspace, size_t workspace_bytes,
                         void* stream, bool flat) {
  clear_err();
  int rc = check_desc(desc);
  if (rc == LSA_OK) rc = check_params(desc, params, flat);
  if (rc == LSA_OK) rc = check_shape(desc, n_tokens, n_q_heads, flat);
  if (rc != LSA_OK) return rc;
  if (n_tokens == 0) return LSA_OK;
  if (!index || !queries || !q_pos || !out_idx || !workspace)
    return fail(LSA_ERR_INVALID_ARG, "index, queries, q_pos, out_idx and workspace must be non-NULL");
  const lsa::SelectPlan plan = lsa::plan_select(*desc, *params, n_tokens, n_q_heads, flat);
  if (workspace_bytes < plan.bytes)
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.bytes);
  char err[256] = {0};
  rc = lsa::launch_select(*desc, *params, plan, index, queries, q_pos, n_tokens, n_q_heads, out_idx, out_scores,
                          out_leaves, workspace, (hipStream_t)stream, flat, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

int lsa_select(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
               int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
               float* out_scores, int32_t* out_leaves, void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(desc, index, queries, q_pos, n_tokens, n_q_heads, params, out_idx, out_scores, out_leaves,
                       workspace, workspace_bytes, stream, false);
}

// Device address of `scratch` on the current device, found once per device.
static int scratch_on_current_device(void** out, char* err, size_t errlen) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(err, errlen, "hipGetDevice failed: %s", hipGetErrorString(e));
    return LSA_ERR_HIP;
  }
  if (dev < 0 || dev >= 64) {
    snprintf(err, errlen, "device %d outside the 64 devices the static scratch supports", dev);
    return LSA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      snprintf(err, errlen, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return LSA_ERR_HIP;
    }
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return LSA_OK;
}

int lsa_select_noalloc(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
                       int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
                       float* out_scores, int32_t* out_leaves, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc == LSA_OK) rc = check_params(desc, params, false);
  if (rc == LSA_OK) rc = check_shape(desc, n_tokens, n_q_heads, false);
  if (rc != LSA_OK) return rc;
  if (n_tokens == 0) return LSA_OK;
  if (!index || !queries || !q_pos || !out_idx)
    return fail(LSA_ERR_INVALID_ARG, "index, queries, q_pos and out_idx must be non-NULL");
  const lsa::SelectPlan plan = lsa::plan_select(*desc, *params, n_tokens, n_q_heads, false);
  if (plan.bytes > (size_t)LSA_NOALLOC_SCRATCH_BYTES)
    return fail(LSA_ERR_UNSUPPORTED,
                "this batch needs %zu bytes of workspace; the static scratch holds %u (call lsa_select with a "
                "workspace)", plan.bytes, (unsigned)LSA_NOALLOC_SCRATCH_BYTES);
  char err[256] = {0};
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  rc = lsa::launch_select(*desc, *params, plan, index, queries, q_pos, n_tokens, n_q_heads, out_idx, out_scores,
                          out_leaves, ws, (hipStream_t)stream, false, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

int lsa_flat_select(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
                    int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
                    float* out_scores, void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(desc, index, queries, q_pos, n_tokens, n_q_heads, params, out_idx, out_scores, nullptr,
                       workspace, workspace_bytes, stream, true);
}

// ---- incremental upkeep ---------------------------------------------------------

static int check_pool(const lsa_index_desc* d, int32_t capacity) {
  if (capacity < 1) return fail(LSA_ERR_INVALID_ARG, "capacity = %d must be >= 1", capacity);
  if (d->n_keys + (int64_t)capacity >= (int64_t(1) << 31))
    return fail(LSA_ERR_UNSUPPORTED, "n_keys + capacity must stay below 2^31");
  return LSA_OK;
}

size_t lsa_append_pool_bytes(const lsa_index_desc* desc, int32_t capacity) {
  clear_err();
  if (check_desc(desc) != LSA_OK || check_pool(desc, capacity) != LSA_OK) return 0;
  return lsa::pool_layout(*desc, capacity).total;
}

int lsa_append_keys(const lsa_index_desc* desc, const void* index, const void* keys, int32_t n_new, int32_t first,
                    void* pool, int32_t capacity, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc == LSA_OK) rc = check_pool(desc, capacity);
  if (rc != LSA_OK) return rc;
  if (n_new < 0 || first < 0 || (int64_t)first + n_new > capacity)
    return fail(LSA_ERR_INVALID_ARG, "slots [%d, %lld) do not fit a pool of %d", first, (long long)first + n_new,
                capacity);
  if (n_new == 0) return LSA_OK;
  if (!index || !keys || !pool) return fail(LSA_ERR_INVALID_ARG, "index, keys and pool must be non-NULL");
  char err[256] = {0};
  rc = lsa::launch_append(*desc, index, keys, n_new, first, pool, capacity, (hipStream_t)stream, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

size_t lsa_select_appended_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params,
                                           int32_t n_tokens, int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) || check_params(desc, params, false) || check_shape(desc, n_tokens, n_q_heads, false)) return 0;
  return lsa::plan_select(*desc, *params, n_tokens, n_q_heads, false, true).bytes;
}

int lsa_select_appended(const lsa_index_desc* desc, const void* index, const void* pool, int32_t capacity,
                        int32_t n_appended, const void* queries, const int32_t* q_pos, int32_t n_tokens,
                        int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx, float* out_scores,
                        int32_t* out_leaves, void* workspace, size_t workspace_bytes, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc == LSA_OK) rc = check_params(desc, params, false);
  if (rc == LSA_OK) rc = check_shape(desc, n_tokens, n_q_heads, false);
  if (rc == LSA_OK) rc = check_pool(desc, capacity);
  if (rc != LSA_OK) return rc;
  if (n_appended < 0 || n_appended > capacity)
    return fail(LSA_ERR_INVALID_ARG, "n_appended = %d outside [0, capacity = %d]", n_appended, capacity);
  if (n_tokens == 0) return LSA_OK;
  if (!index || !queries || !q_pos || !out_idx || !workspace || (n_appended > 0 && !pool))
    return fail(LSA_ERR_INVALID_ARG, "index, queries, q_pos, out_idx, workspace and pool must be non-NULL");
  const lsa::SelectPlan plan = lsa::plan_select(*desc, *params, n_tokens, n_q_heads, false, true);
  if (workspace_bytes < plan.bytes)
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.bytes);
  lsa::AppendView app;
  app.pool = pool;
  app.cap = capacity;
  app.n = n_appended;
  app.on = true;
  char err[256] = {0};
  rc = lsa::launch_select(*desc, *params, plan, index, queries, q_pos, n_tokens, n_q_heads, out_idx, out_scores,
                          out_leaves, workspace, (hipStream_t)stream, false, err, sizeof(err), app);
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

size_t lsa_pca_workspace_bytes(const lsa_index_desc* desc) {
  clear_err();
  if (check_desc(desc) != LSA_OK) return 0;
  return lsa::pca_workspace_bytes(*desc);
}

int lsa_pca_covariance(const lsa_index_desc* desc, const void* keys, double* cov, void* workspace,
                       size_t workspace_bytes, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc != LSA_OK) return rc;
  if (!keys || !cov || !workspace) return fail(LSA_ERR_INVALID_ARG, "keys, cov and workspace must be non-NULL");
  const size_t need = lsa::pca_workspace_bytes(*desc);
  if (workspace_bytes < need)
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  char err[256] = {0};
  rc = lsa::launch_pca_covariance(*desc, keys, cov, workspace, (hipStream_t)stream, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

int lsa_pca_map(const lsa_index_desc* desc, const double* cov, float* W, double* eigenvalues) {
  clear_err();
  int rc = check_desc(desc);
  if (rc != LSA_OK) return rc;
  if (!cov || !W) return fail(LSA_ERR_INVALID_ARG, "cov and W must be non-NULL");
  lsa::pca_map_host(*desc, cov, W, eigenvalues);
  return LSA_OK;
}

size_t lsa_sparse_attention_workspace_bytes(const lsa_index_desc* desc, int32_t width, int32_t n_tokens,
                                            int32_t n_q_heads) {
  clear_err();
  if (check_desc(desc) != LSA_OK || check_shape(desc, n_tokens, n_q_heads, false) != LSA_OK) return 0;
  if (width < 1 || width > lsa::kMaxAttWidth) return 0;
  return lsa::attention_workspace_bytes(*desc, width, n_tokens, n_q_heads);
}

int lsa_sparse_attention(const lsa_index_desc* desc, const void* queries, const void* keys, const void* values,
                         const int32_t* idx, int32_t width, int32_t n_tokens, int32_t n_q_heads, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream) {
  clear_err();
  int rc = check_desc(desc);
  if (rc != LSA_OK) return rc;
  rc = check_shape(desc, n_tokens, n_q_heads, false);
  if (rc != LSA_OK) return rc;
  if (!queries || !keys || !values || !idx || !out)
    return fail(LSA_ERR_INVALID_ARG, "queries, keys, values, idx and out must be non-NULL");
  if (width < 1 || width > lsa::kMaxAttWidth)
    return fail(LSA_ERR_UNSUPPORTED, "width = %d outside [1, %d]", width, lsa::kMaxAttWidth);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return fail(LSA_ERR_INVALID_ARG, "scale is not finite");
  const size_t need = lsa::attention_workspace_bytes(*desc, width, n_tokens, n_q_heads);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_BUFFER_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace ? workspace_bytes : 0, need);
  char err[256] = {0};
  rc = lsa::launch_sparse_attention(*desc, queries, keys, values, idx, width, n_tokens, n_q_heads, scale, out,
                                    workspace, (hipStream_t)stream, err, sizeof(err));
  if (rc != LSA_OK) return fail(rc, "%s", err);
  return LSA_OK;
}

}  // extern "C"
