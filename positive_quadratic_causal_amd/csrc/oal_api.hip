// Host side of the liboal C ABI: argument validation, dispatch to the kernels,
// ownership of prefix states and error reporting.  See include/oal.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "oal_common.h"

namespace oal {

static thread_local char g_last_error[512] = "";

oal_status set_error(oal_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

oal_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(OAL_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return OAL_OK;
}

// ---- per-kernel event timing -------------------------------------------------

namespace {
struct ProfEntry {
  std::string kernel;
  hipEvent_t start, stop;
};
struct ProfTotals {
  double ms = 0.0;
  int64_t launches = 0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;   // when not empty: the one kernel that gets events
std::vector<ProfEntry> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;
std::map<std::string, ProfTotals> g_prof_totals;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Resolve every pending entry (waits for its stop event).
oal_status prof_drain() {
  oal_status st = OAL_OK;
  for (auto& p : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
      st = set_error(OAL_ERR_HIP, "profiling events for %s failed", p.kernel.c_str());
    ProfTotals& t = g_prof_totals[p.kernel];
    t.ms += ms;
    t.launches += 1;
    g_prof_pool.push_back(p.start);
    g_prof_pool.push_back(p.stop);
  }
  g_prof_pending.clear();
  return st;
}
}  // namespace

int prof_begin(const char* kernel, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return -1;
  if (!g_prof_only.empty() && g_prof_only != kernel) return -1;
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return -1;
  if (hipEventRecord(a, stream) != hipSuccess) return -1;
  g_prof_pending.push_back(ProfEntry{kernel, a, b});
  return (int)g_prof_pending.size() - 1;
}

void prof_end(int slot, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (slot < 0 || slot >= (int)g_prof_pending.size()) return;
  (void)hipEventRecord(g_prof_pending[slot].stop, stream);
}

// kernels' launchers (one per source file)
oal_status launch_contrib(int n_q_heads, int n_kv_heads, int n_prompts, int total,
                          oal_dtype in_dtype, const void* q, const void* k, const int32_t* offsets,
                          float* chi_prompt, float* chi, hipStream_t stream);
oal_status launch_grouping(int n_q_heads, int n_prompts, const float* chi_prompt, int n_boot,
                           const int32_t* boot_idx, float alpha, float tau, float gamma, int g_min,
                           float eps, int32_t* group_map, int32_t* n_groups, float* support,
                           float* gap, hipStream_t stream);
int grouping_max_prompts();
size_t calib_workspace(int n_q_heads, int n_pos);
oal_status launch_embed_global(int n_q_heads, int g_max, int g_ld, const int32_t* n_groups,
                               const float* Lg, float* L, hipStream_t stream);
oal_status launch_calib_grad(int n_q_heads, int n_kv_heads, int seq_len, oal_dtype in_dtype,
                             const void* q, const void* k, const void* v, const float* y_ref,
                             const int32_t* positions, int n_pos, int g_max,
                             const int32_t* n_groups, const int32_t* group_map, const float* L,
                             float eps, float* dL, float* loss, void* ws, hipStream_t stream);
oal_status launch_adam(int n_q_heads, int g_max, const int32_t* n_groups, float* L, const float* dL,
                       float* m, float* v, int t, float lr, float beta1, float beta2, float eps,
                       float clip, hipStream_t stream);
oal_status launch_output_mse(int batch, int n_q_heads, int seq_len, int d_v, const float* y,
                             const float* y_ref, float* mse, hipStream_t stream);
size_t backward_workspace(int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk);
oal_status launch_backward(int batch, int n_q_heads, int n_kv_heads, int seq_len, int chunk,
                           oal_dtype in_dtype, const void* q, const void* k, const void* v,
                           const void* coeffs, const float* dy, float* dq, float* dk, float* dv,
                           float* da, float* db, float* dC, void* ws, hipStream_t stream);
oal_status launch_coeffs_backward(int n_q_heads, int g_max, const int32_t* n_groups,
                                  const int32_t* group_map, const float* L, const float* da,
                                  const float* db, const float* dC, float* dL, hipStream_t stream);
oal_status launch_dim_coeffs(int n_q_heads, const float* a, const float* b, const float* C,
                             void* coeffs, hipStream_t stream);
oal_status launch_expand(int n_q_heads, int g_max, const int32_t* n_groups,
                         const int32_t* group_map, const float* L, float eps, void* coeffs,
                         hipStream_t stream);
oal_status launch_fill_zero(float* p, size_t n_floats, hipStream_t stream);
oal_status launch_export(const oal_state* st, float* dst, hipStream_t stream);
oal_status launch_decode(int batch, int n_q_heads, int n_kv_heads, oal_dtype in_dtype,
                         const void* q, const void* k, const void* v, const void* coeffs,
                         float* state, void* y, oal_dtype out_dtype, hipStream_t stream);
size_t prefill_vec_workspace(int batch, int n_kv_heads, int seq_len, int chunk);
size_t state_mfma_workspace(int batch, int n_kv_heads, int seq_len, int chunk, bool with_tiles);
oal_status launch_softmax(int batch, int n_q_heads, int n_kv_heads, int seq_len, const void* q,
                          const void* k, const void* v, void* y, oal_dtype out_dtype,
                          hipStream_t stream);
oal_status launch_prefill_mfma(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                               const void* q, const void* k, const void* v, const void* coeffs,
                               int chunk, float* state, bool init_zero, void* y, oal_dtype out_dtype,
                               void* ws, hipStream_t stream);
oal_status launch_prefill_vec(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                              oal_dtype in_dtype, const void* q, const void* k, const void* v,
                              const void* coeffs, int chunk, float* state, void* y,
                              oal_dtype out_dtype, void* ws, bool dim, hipStream_t stream);

static bool valid_dtype(oal_dtype d) { return d == OAL_F32 || d == OAL_BF16; }

static oal_status check_heads(int batch, int n_q_heads, int n_kv_heads, int d_h, int d_v) {
  if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1)
    return set_error(OAL_ERR_INVALID_ARG, "batch (%d), n_q_heads (%d) and n_kv_heads (%d) must be >= 1",
                     batch, n_q_heads, n_kv_heads);
  if (n_q_heads % n_kv_heads != 0)
    return set_error(OAL_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                     n_q_heads, n_kv_heads);
  if (d_h != DH || d_v != DV)
    return set_error(OAL_ERR_UNSUPPORTED, "only d_h = d_v = 64 is supported (got %d, %d)", d_h, d_v);
  if ((long long)batch * n_kv_heads > 65535 || (long long)batch * n_q_heads > 65535 * 64LL)
    return set_error(OAL_ERR_UNSUPPORTED, "batch * heads too large for one launch");
  return OAL_OK;
}

static int resolve_chunk(int chunk) { return chunk == 0 ? 128 : chunk; }

}  // namespace oal

using namespace oal;

extern "C" {

const char* oal_status_string(oal_status s) {
  switch (s) {
    case OAL_OK: return "OAL_OK";
    case OAL_ERR_INVALID_ARG: return "OAL_ERR_INVALID_ARG";
    case OAL_ERR_UNSUPPORTED: return "OAL_ERR_UNSUPPORTED";
    case OAL_ERR_OUT_OF_MEMORY: return "OAL_ERR_OUT_OF_MEMORY";
    case OAL_ERR_HIP: return "OAL_ERR_HIP";
  }
  return "OAL_ERR_UNKNOWN";
}

const char* oal_last_error(void) { return g_last_error; }

oal_status oal_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  return OAL_OK;
}

oal_status oal_profile_filter(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = kernel ? kernel : "";
  return OAL_OK;
}

oal_status oal_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  oal_status st = prof_drain();
  g_prof_totals.clear();
  return st;
}

oal_status oal_profile_query(const char* kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return set_error(OAL_ERR_INVALID_ARG, "null output pointer");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  oal_status st = prof_drain();
  double ms = 0.0;
  int64_t n = 0;
  for (auto& kv : g_prof_totals) {
    if (kernel == nullptr || kv.first == kernel) {
      ms += kv.second.ms;
      n += kv.second.launches;
    }
  }
  *total_ms = ms;
  *launches = n;
  return st;
}

size_t oal_coeffs_bytes(int n_q_heads, int d_h, int g_max) {
  if (n_q_heads < 1 || d_h != DH || g_max < 1 || g_max > GMAX) return 0;
  return (size_t)n_q_heads * OAL_COEF_WORDS * sizeof(float);
}

oal_status oal_expand_coeffs(int n_q_heads, int d_h, int g_max, const int32_t* n_groups,
                             const int32_t* group_map, const float* L, float eps, void* coeffs,
                             hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (d_h != DH) return set_error(OAL_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
  if (g_max < 1 || g_max > GMAX)
    return set_error(OAL_ERR_UNSUPPORTED, "g_max must be in 1..%d (got %d)", GMAX, g_max);
  if (!n_groups || !group_map || !L || !coeffs)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  if (!(eps > 0.0f)) return set_error(OAL_ERR_INVALID_ARG, "eps must be > 0 (got %g)", (double)eps);
  return launch_expand(n_q_heads, g_max, n_groups, group_map, L, eps, coeffs, stream);
}

oal_status oal_dim_coeffs(int n_q_heads, int d_h, const float* a, const float* b, const float* C,
                          void* coeffs, hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (d_h != DH) return set_error(OAL_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
  if (!a || !b || !C || !coeffs) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_dim_coeffs(n_q_heads, a, b, C, coeffs, stream);
}

oal_status oal_state_alloc(int batch, int n_kv_heads, int d_h, int d_v, oal_state** out) {
  if (!out) return set_error(OAL_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  oal_status st = check_heads(batch, n_kv_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  oal_state* s = new (std::nothrow) oal_state();
  if (!s) return set_error(OAL_ERR_OUT_OF_MEMORY, "host allocation failed");
  s->batch = batch;
  s->n_kv_heads = n_kv_heads;
  s->tokens = 0;
  s->bytes = (size_t)batch * n_kv_heads * STATE_FLOATS * sizeof(float);
  if (hipGetDevice(&s->device) != hipSuccess) {
    delete s;
    return set_error(OAL_ERR_HIP, "hipGetDevice failed");
  }
  if (hipMalloc(reinterpret_cast<void**>(&s->data), s->bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete s;
    return set_error(OAL_ERR_OUT_OF_MEMORY, "hipMalloc of %zu bytes failed", (size_t)s->bytes);
  }
  st = launch_fill_zero(s->data, s->bytes / sizeof(float), nullptr);
  if (st == OAL_OK && hipDeviceSynchronize() != hipSuccess)
    st = set_error(OAL_ERR_HIP, "zeroing the state failed");
  if (st != OAL_OK) {
    (void)hipFree(s->data);
    delete s;
    return st;
  }
  *out = s;
  return OAL_OK;
}

oal_status oal_state_reset(oal_state* s, hipStream_t stream) {
  if (!s) return set_error(OAL_ERR_INVALID_ARG, "state is null");
  s->tokens = 0;
  return launch_fill_zero(s->data, s->bytes / sizeof(float), stream);
}

oal_status oal_state_free(oal_state* s) {
  if (!s) return OAL_OK;
  oal_status st = OAL_OK;
  if (hipDeviceSynchronize() != hipSuccess) st = set_error(OAL_ERR_HIP, "hipDeviceSynchronize failed");
  if (hipFree(s->data) != hipSuccess) st = set_error(OAL_ERR_HIP, "hipFree failed");
  delete s;
  return st;
}

oal_status oal_state_copy(oal_state* dst, const oal_state* src, hipStream_t stream) {
  if (!dst || !src) return set_error(OAL_ERR_INVALID_ARG, "state is null");
  if (dst->batch != src->batch || dst->n_kv_heads != src->n_kv_heads)
    return set_error(OAL_ERR_INVALID_ARG, "state shapes differ");
  if (hipMemcpyAsync(dst->data, src->data, src->bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return set_error(OAL_ERR_HIP, "hipMemcpyAsync failed");
  dst->tokens = src->tokens;
  return OAL_OK;
}

size_t oal_state_bytes(const oal_state* s) { return s ? s->bytes : 0; }

int64_t oal_state_tokens(const oal_state* s) { return s ? s->tokens : -1; }

oal_status oal_state_export(const oal_state* s, float* dst, hipStream_t stream) {
  if (!s || !dst) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_export(s, dst, stream);
}

size_t oal_prefill_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                   int d_v, int chunk, oal_dtype in_dtype, int with_output) {
  if (check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v) != OAL_OK) return 0;
  if (seq_len < 0 || !valid_dtype(in_dtype)) return 0;
  chunk = resolve_chunk(chunk);
  if (chunk != 64 && chunk != 128 && chunk != 256) return 0;
  if (seq_len == 0) return 0;
  if (in_dtype == OAL_BF16) return state_mfma_workspace(batch, n_kv_heads, seq_len, chunk, with_output != 0);
  return with_output ? prefill_vec_workspace(batch, n_kv_heads, seq_len, chunk) : 0;
}

// Argument checks shared by oal_prefill and oal_prefill_dim; need = the
// workspace size the chosen path requires.
static oal_status prefill_checks(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                 int d_v, oal_dtype in_dtype, const void* q, const void* k,
                                 const void* v, const void* coeffs, int chunk,
                                 const oal_state* state, const void* y, oal_dtype out_dtype,
                                 const void* workspace, size_t workspace_bytes, size_t need) {
  oal_status st = check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (seq_len < 0) return set_error(OAL_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", seq_len);
  if (chunk != 64 && chunk != 128 && chunk != 256)
    return set_error(OAL_ERR_INVALID_ARG, "chunk must be 0, 64, 128 or 256 (got %d)", chunk);
  if (state && (state->batch != batch || state->n_kv_heads != n_kv_heads))
    return set_error(OAL_ERR_INVALID_ARG, "state shape (%d, %d) does not match (%d, %d)",
                     state->batch, state->n_kv_heads, batch, n_kv_heads);
  if (!y && !state)
    return set_error(OAL_ERR_INVALID_ARG, "y and state are both null: nothing to compute");
  if (seq_len == 0) return OAL_OK;
  if (!k || !v) return set_error(OAL_ERR_INVALID_ARG, "k and v must not be null");
  if (y && (!q || !coeffs)) return set_error(OAL_ERR_INVALID_ARG, "q and coeffs must not be null");
  if ((long long)seq_len * 64 * (long long)batch * n_q_heads > (1LL << 40))
    return set_error(OAL_ERR_UNSUPPORTED, "problem too large");
  if (need > 0 && (!workspace || workspace_bytes < need))
    return set_error(OAL_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", need,
                     workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return set_error(OAL_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return OAL_OK;
}

oal_status oal_prefill(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                       oal_dtype in_dtype, const void* q, const void* k, const void* v,
                       const void* coeffs, int chunk, oal_state* state, void* y,
                       oal_dtype out_dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  chunk = resolve_chunk(chunk);
  const size_t need = oal_prefill_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v,
                                                  chunk, in_dtype, y != nullptr);
  oal_status st = prefill_checks(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v,
                                 coeffs, chunk, state, y, out_dtype, workspace, workspace_bytes, need);
  if (st != OAL_OK || seq_len == 0) return st;
  if (in_dtype == OAL_BF16)
    st = launch_prefill_mfma(batch, n_q_heads, n_kv_heads, seq_len, q, k, v, coeffs, chunk,
                             state ? state->data : nullptr, false, y, out_dtype, workspace, stream);
  else
    st = launch_prefill_vec(batch, n_q_heads, n_kv_heads, seq_len, in_dtype, q, k, v, coeffs, chunk,
                            state ? state->data : nullptr, y, out_dtype, workspace, false, stream);
  if (st == OAL_OK && state) state->tokens += seq_len;
  return st;
}

oal_status oal_prefill_fresh(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                             oal_dtype in_dtype, const void* q, const void* k, const void* v,
                             const void* coeffs, int chunk, oal_state* state, void* y,
                             oal_dtype out_dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!state) return set_error(OAL_ERR_INVALID_ARG, "oal_prefill_fresh needs a state (else use oal_prefill)");
  chunk = resolve_chunk(chunk);
  const size_t need = oal_prefill_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v,
                                                  chunk, in_dtype, y != nullptr);
  oal_status st = prefill_checks(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v,
                                 coeffs, chunk, state, y, out_dtype, workspace, workspace_bytes, need);
  if (st != OAL_OK) return st;
  if (seq_len == 0 || in_dtype != OAL_BF16) {
    // no tokens, or the fp32 path (which adds to the state it reads): clear, then append
    st = launch_fill_zero(state->data, state->bytes / sizeof(float), stream);
    if (st != OAL_OK) return st;
    state->tokens = 0;
    if (seq_len == 0) return OAL_OK;
    return oal_prefill(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v, coeffs,
                       chunk, state, y, out_dtype, workspace, workspace_bytes, stream);
  }
  // the builder starts from zero without reading the state and writes every entry
  // of it (the padding beyond the 2145 features is zero from the allocation on)
  st = launch_prefill_mfma(batch, n_q_heads, n_kv_heads, seq_len, q, k, v, coeffs, chunk, state->data,
                           true, y, out_dtype, workspace, stream);
  if (st == OAL_OK) state->tokens = seq_len;
  return st;
}

// ---- allocation-free prefill -------------------------------------------------
// The scratch of oal_prefill_noalloc: a file-scope device array (one copy on every
// GPU the library runs on, held until the process ends).  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept here.
namespace {
__device__ __align__(256) uint8_t scratch[OAL_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

oal_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(OAL_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(OAL_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(OAL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OAL_OK;
}
}  // namespace

size_t oal_prefill_noalloc_scratch_bytes(void) { return OAL_NOALLOC_SCRATCH_BYTES; }

oal_status oal_prefill_noalloc(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                               int d_v, oal_dtype in_dtype, const void* q, const void* k,
                               const void* v, const void* coeffs, int chunk, oal_state* state,
                               void* y, oal_dtype out_dtype, hipStream_t stream) {
  chunk = resolve_chunk(chunk);
  const size_t need = oal_prefill_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v,
                                                  chunk, in_dtype, y != nullptr);
  if (need > OAL_NOALLOC_SCRATCH_BYTES)
    return set_error(OAL_ERR_UNSUPPORTED,
                     "oal_prefill_noalloc: these sizes need %zu bytes of scratch, the static buffer "
                     "holds %zu (use oal_prefill with a workspace)", need,
                     (size_t)OAL_NOALLOC_SCRATCH_BYTES);
  // the same checks as oal_prefill (with a stand-in for the workspace) before any
  // HIP call, so that invalid arguments fail the same way
  oal_status st = prefill_checks(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v,
                                 coeffs, chunk, state, y, out_dtype,
                                 need > 0 ? reinterpret_cast<void*>(256) : nullptr,
                                 OAL_NOALLOC_SCRATCH_BYTES, need);
  if (st != OAL_OK || seq_len == 0) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_ptr(&ws);
    if (st != OAL_OK) return st;
  }
  return oal_prefill(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v, coeffs,
                     chunk, state, y, out_dtype, ws, need > 0 ? OAL_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t oal_prefill_dim_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                       int d_h, int d_v, int chunk, int with_output) {
  if (check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v) != OAL_OK) return 0;
  chunk = resolve_chunk(chunk);
  if (seq_len <= 0 || (chunk != 64 && chunk != 128 && chunk != 256)) return 0;
  return with_output ? prefill_vec_workspace(batch, n_kv_heads, seq_len, chunk) : 0;
}

oal_status oal_prefill_dim(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                           int d_v, oal_dtype in_dtype, const void* q, const void* k,
                           const void* v, const void* coeffs, int chunk, oal_state* state,
                           void* y, oal_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  chunk = resolve_chunk(chunk);
  const size_t need = oal_prefill_dim_workspace_bytes(batch, n_q_heads, n_kv_heads, seq_len, d_h,
                                                      d_v, chunk, y != nullptr);
  oal_status st = prefill_checks(batch, n_q_heads, n_kv_heads, seq_len, d_h, d_v, in_dtype, q, k, v,
                                 coeffs, chunk, state, y, out_dtype, workspace, workspace_bytes, need);
  if (st != OAL_OK || seq_len == 0) return st;
  st = launch_prefill_vec(batch, n_q_heads, n_kv_heads, seq_len, in_dtype, q, k, v, coeffs, chunk,
                          state ? state->data : nullptr, y, out_dtype, workspace, true, stream);
  if (st == OAL_OK && state) state->tokens += seq_len;
  return st;
}

size_t oal_prefill_backward_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int seq_len,
                                            int d_h, int d_v, int chunk) {
  if (check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v) != OAL_OK) return 0;
  chunk = resolve_chunk(chunk);
  if (seq_len <= 0 || (chunk != 64 && chunk != 128)) return 0;
  return backward_workspace(batch, n_q_heads, n_kv_heads, seq_len, chunk);
}

oal_status oal_prefill_backward(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                int d_v, oal_dtype in_dtype, const void* q, const void* k,
                                const void* v, const void* coeffs, const float* dy, int chunk,
                                float* dq, float* dk, float* dv, float* da, float* db, float* dC,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  oal_status st = check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  if (!valid_dtype(in_dtype)) return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (seq_len < 0) return set_error(OAL_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", seq_len);
  chunk = resolve_chunk(chunk);
  if (chunk != 64 && chunk != 128)
    return set_error(OAL_ERR_INVALID_ARG, "backward chunk must be 0, 64 or 128 (got %d)", chunk);
  const int n_coef = (da != nullptr) + (db != nullptr) + (dC != nullptr);
  if (n_coef != 0 && n_coef != 3)
    return set_error(OAL_ERR_INVALID_ARG, "da, db and dC must be all given or all null");
  if (seq_len == 0) {
    if (n_coef == 0) return OAL_OK;
    st = launch_fill_zero(da, (size_t)n_q_heads, stream);
    if (st == OAL_OK) st = launch_fill_zero(db, (size_t)n_q_heads * DH, stream);
    if (st == OAL_OK) st = launch_fill_zero(dC, (size_t)n_q_heads * DH * DH, stream);
    return st;
  }
  if (!q || !k || !v || !coeffs || !dy || !dq || !dk || !dv)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  if ((long long)seq_len * 64 * (long long)batch * n_q_heads > (1LL << 40))
    return set_error(OAL_ERR_UNSUPPORTED, "problem too large");
  const size_t need = backward_workspace(batch, n_q_heads, n_kv_heads, seq_len, chunk);
  if (!workspace || workspace_bytes < need)
    return set_error(OAL_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", need,
                     workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return set_error(OAL_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return launch_backward(batch, n_q_heads, n_kv_heads, seq_len, chunk, in_dtype, q, k, v, coeffs, dy,
                         dq, dk, dv, da, db, dC, workspace, stream);
}

oal_status oal_coeffs_backward(int n_q_heads, int d_h, int g_max, const int32_t* n_groups,
                               const int32_t* group_map, const float* L, const float* da,
                               const float* db, const float* dC, float* dL, hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (d_h != DH) return set_error(OAL_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
  if (g_max < 1 || g_max > GMAX)
    return set_error(OAL_ERR_UNSUPPORTED, "g_max must be in 1..%d (got %d)", GMAX, g_max);
  if (!n_groups || !group_map || !L || !da || !db || !dC || !dL)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_coeffs_backward(n_q_heads, g_max, n_groups, group_map, L, da, db, dC, dL, stream);
}

size_t oal_calib_workspace_bytes(int n_q_heads, int n_pos) {
  if (n_q_heads < 1 || n_pos < 1) return 0;
  return calib_workspace(n_q_heads, n_pos);
}

oal_status oal_calib_grad(int n_q_heads, int n_kv_heads, int seq_len, int d_h, int d_v,
                          oal_dtype in_dtype, const void* q, const void* k, const void* v,
                          const float* y_ref, const int32_t* positions, int n_pos, int g_max,
                          const int32_t* n_groups, const int32_t* group_map, const float* L,
                          float eps, float* dL, float* loss, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  oal_status st = check_heads(1, n_q_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  if (!valid_dtype(in_dtype)) return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (seq_len < 1) return set_error(OAL_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d)", seq_len);
  if (n_pos < 1) return set_error(OAL_ERR_INVALID_ARG, "n_pos must be >= 1 (got %d)", n_pos);
  if (g_max < 1 || g_max > GMAX)
    return set_error(OAL_ERR_UNSUPPORTED, "g_max must be in 1..%d (got %d)", GMAX, g_max);
  if (!(eps > 0.0f)) return set_error(OAL_ERR_INVALID_ARG, "eps must be > 0 (got %g)", (double)eps);
  if (!q || !k || !v || !y_ref || !positions || !n_groups || !group_map || !L || !dL || !loss)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  const size_t need = calib_workspace(n_q_heads, n_pos);
  if (!workspace || workspace_bytes < need)
    return set_error(OAL_ERR_INVALID_ARG, "workspace too small: need %zu bytes, got %zu", need,
                     workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return set_error(OAL_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return launch_calib_grad(n_q_heads, n_kv_heads, seq_len, in_dtype, q, k, v, y_ref, positions, n_pos,
                           g_max, n_groups, group_map, L, eps, dL, loss, workspace, stream);
}

oal_status oal_adam_step(int n_q_heads, int g_max, const int32_t* n_groups, float* L,
                         const float* dL, float* m, float* v, int step, float lr, float beta1,
                         float beta2, float eps, float clip_norm, hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (g_max < 1 || g_max > GMAX)
    return set_error(OAL_ERR_UNSUPPORTED, "g_max must be in 1..%d (got %d)", GMAX, g_max);
  if (step < 1) return set_error(OAL_ERR_INVALID_ARG, "step is 1-based (got %d)", step);
  if (!(lr > 0.0f) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) ||
      !(eps > 0.0f) || !(clip_norm > 0.0f))
    return set_error(OAL_ERR_INVALID_ARG, "invalid optimiser settings");
  if (!n_groups || !L || !dL || !m || !v) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_adam(n_q_heads, g_max, n_groups, L, dL, m, v, step, lr, beta1, beta2, eps, clip_norm,
                     stream);
}

oal_status oal_embed_global(int n_q_heads, int g_max, const int32_t* n_groups, int g_ld,
                            const float* L_global, float* L, hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (g_max < 1 || g_max > GMAX)
    return set_error(OAL_ERR_UNSUPPORTED, "g_max must be in 1..%d (got %d)", GMAX, g_max);
  if (g_ld < 2 || g_ld > LDIM) return set_error(OAL_ERR_INVALID_ARG, "g_ld must be in 2..%d", LDIM);
  if (!n_groups || !L_global || !L) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_embed_global(n_q_heads, g_max, g_ld, n_groups, L_global, L, stream);
}

oal_status oal_output_mse(int batch, int n_q_heads, int seq_len, int d_v, const float* y,
                          const float* y_ref, float* mse, hipStream_t stream) {
  if (batch < 1 || n_q_heads < 1 || seq_len < 1 || d_v < 1)
    return set_error(OAL_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!y || !y_ref || !mse) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_output_mse(batch, n_q_heads, seq_len, d_v, y, y_ref, mse, stream);
}

oal_status oal_contribution_scores(int n_q_heads, int n_kv_heads, int n_prompts, int total_tokens,
                                  int d_h, oal_dtype in_dtype, const void* q, const void* k,
                                  const int32_t* offsets, float* chi_prompt, float* chi,
                                  hipStream_t stream) {
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0)
    return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (d_h != DH) return set_error(OAL_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
  if (!valid_dtype(in_dtype)) return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (n_prompts < 1 || total_tokens < 0)
    return set_error(OAL_ERR_INVALID_ARG, "n_prompts must be >= 1 and total_tokens >= 0");
  if (!q || !k || !offsets || !chi_prompt) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_contrib(n_q_heads, n_kv_heads, n_prompts, total_tokens, in_dtype, q, k, offsets,
                        chi_prompt, chi, stream);
}

oal_status oal_bootstrap_grouping(int n_q_heads, int n_prompts, int d_h, const float* chi_prompt,
                                  int n_boot, const int32_t* boot_idx, float alpha, float tau,
                                  float gamma, int g_min, float eps, int32_t* group_map,
                                  int32_t* n_groups, float* support, float* gap,
                                  hipStream_t stream) {
  if (n_q_heads < 1) return set_error(OAL_ERR_INVALID_ARG, "n_q_heads must be >= 1");
  if (d_h != DH) return set_error(OAL_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
  if (n_prompts < 1 || n_prompts > grouping_max_prompts())
    return set_error(OAL_ERR_UNSUPPORTED, "n_prompts must be in 1..%d (got %d)", grouping_max_prompts(),
                     n_prompts);
  if (n_boot < 1) return set_error(OAL_ERR_INVALID_ARG, "n_boot must be >= 1 (got %d)", n_boot);
  if (!(alpha > 0.0f && alpha <= 1.0f) || !(tau > 0.0f) || !(gamma >= 0.0f && gamma <= 1.0f) ||
      g_min < 1 || !(eps > 0.0f))
    return set_error(OAL_ERR_INVALID_ARG, "invalid grouping settings");
  if (!chi_prompt || !boot_idx || !group_map || !n_groups)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_grouping(n_q_heads, n_prompts, chi_prompt, n_boot, boot_idx, alpha, tau, gamma, g_min,
                         eps, group_map, n_groups, support, gap, stream);
}

oal_status oal_softmax_attention(int batch, int n_q_heads, int n_kv_heads, int seq_len, int d_h,
                                 int d_v, oal_dtype in_dtype, const void* q, const void* k,
                                 const void* v, void* y, oal_dtype out_dtype, hipStream_t stream) {
  oal_status st = check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (in_dtype != OAL_BF16)
    return set_error(OAL_ERR_UNSUPPORTED, "oal_softmax_attention takes bf16 inputs only");
  if (seq_len < 0) return set_error(OAL_ERR_INVALID_ARG, "seq_len must be >= 0 (got %d)", seq_len);
  if (seq_len == 0) return OAL_OK;
  if (!q || !k || !v || !y) return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  return launch_softmax(batch, n_q_heads, n_kv_heads, seq_len, q, k, v, y, out_dtype, stream);
}

oal_status oal_decode_step(int batch, int n_q_heads, int n_kv_heads, int d_h, int d_v,
                           oal_dtype in_dtype, const void* q, const void* k, const void* v,
                           const void* coeffs, oal_state* state, void* y, oal_dtype out_dtype,
                           hipStream_t stream) {
  oal_status st = check_heads(batch, n_q_heads, n_kv_heads, d_h, d_v);
  if (st != OAL_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return set_error(OAL_ERR_INVALID_ARG, "unknown dtype");
  if (!q || !k || !v || !coeffs || !state || !y)
    return set_error(OAL_ERR_INVALID_ARG, "null pointer argument");
  if (state->batch != batch || state->n_kv_heads != n_kv_heads)
    return set_error(OAL_ERR_INVALID_ARG, "state shape (%d, %d) does not match (%d, %d)",
                     state->batch, state->n_kv_heads, batch, n_kv_heads);
  st = launch_decode(batch, n_q_heads, n_kv_heads, in_dtype, q, k, v, coeffs, state->data, y,
                     out_dtype, stream);
  if (st == OAL_OK) state->tokens += 1;
  return st;
}

}  // extern "C"
