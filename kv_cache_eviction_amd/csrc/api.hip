// C ABI of the chunked H2O step: validation, state bookkeeping, workspace
// carving and kernel orchestration.  All device work is enqueued on the
// caller's stream; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <math.h>
#include <string.h>

#include <algorithm>
#include <cstdlib>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "h2o.h"

#include "h2o_launch.h"

// Scratch of h2o_chunk_backward_static (see below).
constexpr size_t kStaticScratchBytes = size_t{72} << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kTimedKernels = 5;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// true if some non-null pointer is not 16-byte aligned
bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15u) return true;
  return false;
}

struct Layout {
  size_t partial_off, partial_bytes;
  size_t lse_off, lse_bytes;
  size_t targets_off, targets_bytes;     // target slot list of the current step
  size_t counters_off, counters_bytes;   // the device status word, then one read counter per (b, KV head)
  size_t split_off, split_bytes;         // attention key-split partial states
  size_t n_counters;                     // ints cleared at init
  size_t total;
};

int max_len(const h2o_config* c) { return c->max_chunk > c->max_prefill ? c->max_chunk : c->max_prefill; }

Layout layout_of(const h2o_config* c) {
  Layout L;
  const size_t heads = static_cast<size_t>(c->batch) * c->n_kv_heads;
  const size_t smax = static_cast<size_t>(max_len(c));
  L.partial_off = 0;
  // row splits of the masses: the score kernel's, or the fused short-chunk
  // kernel's 32-row parts
  const size_t n_splits = static_cast<size_t>(std::max(
      h2o::score_row_splits_max(), h2o::decode_fused_max_splits(c->n_q_heads / c->n_kv_heads, static_cast<int>(smax))));
  L.partial_bytes = align_up(heads * n_splits * (c->cache_slots + smax) * sizeof(float));
  L.lse_off = L.partial_off + L.partial_bytes;
  L.lse_bytes = align_up(static_cast<size_t>(c->batch) * c->n_q_heads * smax * sizeof(float));
  L.targets_off = L.lse_off + L.lse_bytes;
  L.targets_bytes = align_up(heads * smax * sizeof(int32_t));
  L.counters_off = L.targets_off + L.targets_bytes;
  L.n_counters = 1 + heads;
  L.counters_bytes = align_up(L.n_counters * sizeof(int32_t));
  L.split_off = L.counters_off + L.counters_bytes;
  L.split_bytes = c->dtype == H2O_BF16 ? align_up(h2o::attn_split_bytes(c->batch, c->n_q_heads, static_cast<int>(smax), c->head_dim)) : 0;
  L.total = L.split_off + L.split_bytes;
  return L;
}

struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};

}  // namespace

struct h2o_cache {
  h2o_config cfg;
  void* k_cache;
  void* v_cache;
  float* scores;
  int32_t* pos;
  char* ws;
  Layout lay;
  int64_t T;
  int filled;          // slots [0, filled) hold tokens, the rest are free; -1: unknown (adopted)
  int n_cu;            // compute units of the device current at h2o_cache_init
  int32_t last_hip_error;
  uint32_t timing_mask;      // bit k: bracket kernel id k with events
  uint32_t sync_target;      // running total of the select parts' reads (see select_scatter.hip)
  uint32_t spin_limit;       // bound of the select's wait (0: the library default)
  uint32_t sync_skew;        // added to the expected total (tests of the bounded wait only)
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> event_pool;
  double total_ms[kTimedKernels];
  int64_t launches[kTimedKernels];
};

namespace {

hipEvent_t take_event(h2o_cache* c) {
  if (!c->event_pool.empty()) {
    hipEvent_t e = c->event_pool.back();
    c->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on `st`; when timing is on, brackets it with events.
template <class F>
h2o_status timed(h2o_cache* c, int kid, hipStream_t st, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (c && ((c->timing_mask >> kid) & 1u)) {
    a = take_event(c);
    b = take_event(c);
    if (a && b && hipEventRecord(a, st) != hipSuccess) {
      c->event_pool.push_back(a);
      c->event_pool.push_back(b);
      a = b = nullptr;
    }
  }
  hipError_t e = launch();
  if (a && b) {
    if (hipEventRecord(b, st) == hipSuccess) {
      c->pending.push_back({kid, a, b});
    } else {
      c->event_pool.push_back(a);
      c->event_pool.push_back(b);
    }
  }
  if (e != hipSuccess) {
    if (c) c->last_hip_error = static_cast<int32_t>(e);
    return H2O_ERR_HIP;
  }
  return H2O_OK;
}

h2o::StepShape shape_of(const h2o_cache* c, int s) {
  const h2o_config& g = c->cfg;
  h2o::StepShape sh;
  sh.B = g.batch;
  sh.Hq = g.n_q_heads;
  sh.Hkv = g.n_kv_heads;
  sh.D = g.head_dim;
  sh.S = s;
  sh.M = g.cache_slots;
  sh.W = g.recent_window;
  sh.n_cache = c->filled >= 0 ? c->filled : g.cache_slots;
  sh.scale = g.softmax_scale > 0.f ? g.softmax_scale : 1.0f / sqrtf(static_cast<float>(g.head_dim));
  sh.policy = g.policy;
  sh.n_sink = g.n_sink;
  sh.n_cu = c->n_cu;
  // slots never become free again in forward steps: once the count of filled
  // slots reached M (known unless the state was adopted), all are filled
  sh.all_filled = c->filled == g.cache_slots;
  return sh;
}

h2o_status run_step(h2o_cache* c, const void* q, const void* k, const void* v, int32_t s, void* out,
                    float* lse, int32_t* slots_out, int32_t* pos_old, float* step_mass, void* k_old, void* v_old,
                    hipStream_t st) {
  const h2o::StepShape sh = shape_of(c, s);
  float* lse_buf = lse ? lse : reinterpret_cast<float*>(c->ws + c->lay.lse_off);
  float* partial = reinterpret_cast<float*>(c->ws + c->lay.partial_off);
  int32_t* status = reinterpret_cast<int32_t*>(c->ws + c->lay.counters_off);
  const int dtype = c->cfg.dtype;

  float* split_part = c->lay.split_bytes ? reinterpret_cast<float*>(c->ws + c->lay.split_off) : nullptr;
  h2o::AttnArgs aa{q, c->k_cache, c->v_cache, c->pos, k, v, out, lse_buf, split_part};
  // short chunks: attention and masses in one pass (row splits = the halves)
  const int halves = h2o::decode_fused_halves(sh, dtype);
  h2o_status r;
  int R = 0;
  if (halves > 0) {
    R = halves;
    r = timed(c, 0, st, [&] { return h2o::launch_decode_fused(sh, aa, partial, st); });
    if (r != H2O_OK) return r;
  } else {
    r = timed(c, 0, st, [&] { return h2o::launch_attn_fwd(sh, aa, dtype, st); });
    if (r != H2O_OK) return r;
    // the position policies keep no score: no mass pass
    if (sh.policy == H2O_POLICY_H2O) {
      R = h2o::score_row_splits(sh, dtype);
      h2o::ScoreArgs sa{q, c->k_cache, k, lse_buf, partial, R};
      r = timed(c, 1, st, [&] { return h2o::launch_score(sh, sa, dtype, st); });
      if (r != H2O_OK) return r;
    }
  }
  int32_t* targets = reinterpret_cast<int32_t*>(c->ws + c->lay.targets_off);
  h2o::SelectArgs xa{c->k_cache, c->v_cache, c->scores, c->pos, k, v, partial, R, targets,
                     slots_out, pos_old, step_mass, k_old, v_old, status, static_cast<int32_t>(c->T),
                     reinterpret_cast<uint32_t*>(status + 1), 0u, c->spin_limit};
  // every part but the first adds one read to its head's counter
  c->sync_target += static_cast<uint32_t>(h2o::select_parts(sh) - 1);
  xa.sync_target = c->sync_target + c->sync_skew;
  r = timed(c, 2, st, [&] { return h2o::launch_select(sh, xa, dtype, st); });
  if (r != H2O_OK) return r;
  if (!h2o::select_copies_rows(sh)) {
    r = timed(c, 4, st, [&] { return h2o::launch_scatter(sh, xa, dtype, st); });
    if (r != H2O_OK) return r;
  }
  c->T += s;
  if (c->filled >= 0) c->filled = c->filled + s > c->cfg.cache_slots ? c->cfg.cache_slots : c->filled + s;
  return H2O_OK;
}

h2o::StepShape backward_shape(const h2o_config* cfg, int32_t s) {
  h2o::StepShape sh;
  sh.B = cfg->batch;
  sh.Hq = cfg->n_q_heads;
  sh.Hkv = cfg->n_kv_heads;
  sh.D = cfg->head_dim;
  sh.S = s;
  sh.M = cfg->cache_slots;
  sh.W = cfg->recent_window;
  sh.n_cache = cfg->cache_slots;
  sh.scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / sqrtf(static_cast<float>(cfg->head_dim));
  return sh;
}

// recurrence step workspace: the backward's (the walk's gradients go
// straight into the caller's fp32 accumulators)
size_t rec_workspace_bytes(const h2o_config* cfg, int32_t s) {
  return h2o::backward_workspace_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, s, cfg->head_dim);
}

// Scratch of h2o_chunk_backward_static, for callers that cannot allocate:
// the backward's workspace (D_i per query row, fp32 partial dK/dV of the
// chunk keys) in a device array of fixed size that every GPU the library
// runs on holds until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host that name is only a stand-in): each
// device's address comes from hipGetSymbolAddress, taken once per device
// with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on first use).
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* h2o_status_str(h2o_status s) {
  switch (s) {
    case H2O_OK: return "ok";
    case H2O_ERR_NULL: return "null pointer";
    case H2O_ERR_CONFIG: return "invalid config";
    case H2O_ERR_SHAPE: return "chunk length out of range";
    case H2O_ERR_STATE: return "call not allowed in this cache state";
    case H2O_ERR_WORKSPACE: return "workspace too small";
    case H2O_ERR_HIP: return "HIP error";
    case H2O_ERR_UNSUPPORTED: return "unsupported request";
    case H2O_ERR_ALIGN: return "buffer pointer not 16-byte aligned";
    case H2O_ERR_TOO_LARGE: return "request needs more than the library's static scratch (72 MiB)";
  }
  return "unknown status";
}

h2o_status h2o_validate_config(const h2o_config* c) {
  if (!c) return H2O_ERR_NULL;
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1) return H2O_ERR_CONFIG;
  if (c->n_q_heads % c->n_kv_heads != 0) return H2O_ERR_CONFIG;
  if (c->head_dim != 64 && c->head_dim != 128) return H2O_ERR_CONFIG;
  if (c->dtype != H2O_BF16 && c->dtype != H2O_FP32) return H2O_ERR_CONFIG;
  if (c->cache_slots < 1 || c->cache_slots > 16384) return H2O_ERR_CONFIG;
  if (c->recent_window < 0 || c->max_chunk < 1 || c->max_prefill < 1) return H2O_ERR_CONFIG;
  if (c->max_prefill > c->cache_slots) return H2O_ERR_CONFIG;
  if (static_cast<int64_t>(c->cache_slots) - c->recent_window < c->max_chunk) return H2O_ERR_CONFIG;
  if (c->max_chunk > 16384 || c->max_prefill > 16384) return H2O_ERR_CONFIG;
  if (!(c->softmax_scale == c->softmax_scale)) return H2O_ERR_CONFIG;   // NaN
  // query rows of one KV group (G queries per chunk position) index with 24-bit arithmetic
  if (static_cast<int64_t>(c->n_q_heads / c->n_kv_heads) * max_len(c) > (int64_t{1} << 20))
    return H2O_ERR_CONFIG;
  // every tensor offset must fit in int64 and every chunk tensor below 2^31 elements
  const int64_t big = static_cast<int64_t>(c->batch) * c->n_q_heads * max_len(c) * c->head_dim;
  if (big >= (int64_t{1} << 31)) return H2O_ERR_CONFIG;
  if (c->policy != H2O_POLICY_H2O && c->policy != H2O_POLICY_RECENT && c->policy != H2O_POLICY_SINK_RECENT)
    return H2O_ERR_CONFIG;
  if (c->policy != H2O_POLICY_SINK_RECENT && c->n_sink != 0) return H2O_ERR_CONFIG;
  if (c->n_sink < 0) return H2O_ERR_CONFIG;
  if (static_cast<int64_t>(c->cache_slots) - c->recent_window - c->n_sink < c->max_chunk) return H2O_ERR_CONFIG;
  return H2O_OK;
}

size_t h2o_workspace_bytes(const h2o_config* c) {
  if (h2o_validate_config(c) != H2O_OK) return 0;
  return layout_of(c).total;
}

h2o_status h2o_cache_init(const h2o_config* cfg, void* k_cache, void* v_cache, float* scores,
                          int32_t* positions, void* workspace, size_t workspace_bytes, int32_t adopt,
                          int64_t tokens_seen, void* stream, h2o_cache** out) {
  if (!cfg || !k_cache || !v_cache || !scores || !positions || !workspace || !out) return H2O_ERR_NULL;
  *out = nullptr;
  if (misaligned({k_cache, v_cache, scores, positions, workspace})) return H2O_ERR_ALIGN;
  h2o_status r = h2o_validate_config(cfg);
  if (r != H2O_OK) return r;
  if (tokens_seen < 0 || (!adopt && tokens_seen != 0) || tokens_seen > INT32_MAX) return H2O_ERR_STATE;
  const Layout lay = layout_of(cfg);
  if (workspace_bytes < lay.total) return H2O_ERR_WORKSPACE;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    return H2O_ERR_HIP;
  h2o_cache* c = new h2o_cache();
  c->n_cu = n_cu;
  c->cfg = *cfg;
  c->k_cache = k_cache;
  c->v_cache = v_cache;
  c->scores = scores;
  c->pos = positions;
  c->ws = static_cast<char*>(workspace);
  c->lay = lay;
  c->T = tokens_seen;
  c->filled = adopt ? -1 : 0;
  c->last_hip_error = 0;
  c->timing_mask = 0;
  c->sync_target = 0;
  // test-only knobs of the select's bounded wait (unset in normal use)
  c->spin_limit = 0;
  c->sync_skew = 0;
  if (const char* e = getenv("H2O_SELECT_SPIN_LIMIT")) c->spin_limit = static_cast<uint32_t>(strtoul(e, nullptr, 10));
  if (const char* e = getenv("H2O_SELECT_SYNC_SKEW")) c->sync_skew = static_cast<uint32_t>(strtoul(e, nullptr, 10));
  for (int i = 0; i < kTimedKernels; ++i) {
    c->total_ms[i] = 0.0;
    c->launches[i] = 0;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n_slots = static_cast<int64_t>(cfg->batch) * cfg->n_kv_heads * cfg->cache_slots;
  const int64_t n_cnt = static_cast<int64_t>(lay.n_counters);
  int32_t* counters = reinterpret_cast<int32_t*>(c->ws + lay.counters_off);
  r = timed(c, 3, st, [&] {
    return h2o::launch_reset(adopt ? nullptr : scores, adopt ? nullptr : positions, adopt ? 0 : n_slots,
                             counters, n_cnt, st);
  });
  if (r != H2O_OK) {
    delete c;
    return r;
  }
  *out = c;
  return H2O_OK;
}

h2o_status h2o_prefill(h2o_cache* c, const void* q, const void* k, const void* v, int32_t n, void* out,
                       float* lse, void* stream) {
  if (!c || !q || !k || !v || !out) return H2O_ERR_NULL;
  if (misaligned({q, k, v, out, lse})) return H2O_ERR_ALIGN;
  if (n < 1 || n > c->cfg.max_prefill) return H2O_ERR_SHAPE;
  if (c->T != 0) return H2O_ERR_STATE;
  return run_step(c, q, k, v, n, out, lse, nullptr, nullptr, nullptr, nullptr, nullptr,
                  static_cast<hipStream_t>(stream));
}

h2o_status h2o_chunk_step(h2o_cache* c, const void* q, const void* k_new, const void* v_new, int32_t s,
                          void* out, float* lse, int32_t* slots_out, float* step_mass, void* k_old,
                          void* v_old, int32_t* pos_old, void* stream) {
  if (!c || !q || !k_new || !v_new || !out) return H2O_ERR_NULL;
  if ((k_old == nullptr) != (v_old == nullptr)) return H2O_ERR_NULL;
  if (misaligned({q, k_new, v_new, out, lse, slots_out, step_mass, k_old, v_old, pos_old})) return H2O_ERR_ALIGN;
  if (step_mass && c->cfg.policy != H2O_POLICY_H2O) return H2O_ERR_UNSUPPORTED;
  if (s < 1 || s > c->cfg.max_chunk) return H2O_ERR_SHAPE;
  if (c->T + s > INT32_MAX) return H2O_ERR_STATE;
  return run_step(c, q, k_new, v_new, s, out, lse, slots_out, pos_old, step_mass, k_old, v_old,
                  static_cast<hipStream_t>(stream));
}

h2o_status h2o_get_scores(const h2o_cache* c, float* scores_out, int32_t* positions_out, void* stream) {
  if (!c || !scores_out) return H2O_ERR_NULL;
  if (misaligned({scores_out, positions_out})) return H2O_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n = static_cast<size_t>(c->cfg.batch) * c->cfg.n_kv_heads * c->cfg.cache_slots;
  hipError_t e = hipMemcpyAsync(scores_out, c->scores, n * sizeof(float), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && positions_out)
    e = hipMemcpyAsync(positions_out, c->pos, n * sizeof(int32_t), hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) {
    const_cast<h2o_cache*>(c)->last_hip_error = static_cast<int32_t>(e);
    return H2O_ERR_HIP;
  }
  return H2O_OK;
}

int64_t h2o_tokens_seen(const h2o_cache* c) { return c ? c->T : -1; }

h2o_status h2o_device_status(h2o_cache* c, void* stream, int32_t* flags) {
  if (!c || !flags) return H2O_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* status = reinterpret_cast<int32_t*>(c->ws + c->lay.counters_off);
  int32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, status, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && host != 0) {
    const int32_t zero = 0;
    e = hipMemcpyAsync(status, &zero, sizeof(int32_t), hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  if (e != hipSuccess) {
    c->last_hip_error = static_cast<int32_t>(e);
    return H2O_ERR_HIP;
  }
  *flags = host;
  return H2O_OK;
}

h2o_status h2o_set_timing(h2o_cache* c, int32_t kernel_mask) {
  if (!c) return H2O_ERR_NULL;
  c->timing_mask = static_cast<uint32_t>(kernel_mask);
  return H2O_OK;
}

h2o_status h2o_get_timing(h2o_cache* c, int32_t kernel_id, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return H2O_ERR_NULL;
  if (kernel_id < 0 || kernel_id >= kTimedKernels) return H2O_ERR_SHAPE;
  for (const TimedLaunch& t : c->pending) {
    hipError_t e = hipEventSynchronize(t.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) {
      c->last_hip_error = static_cast<int32_t>(e);
      return H2O_ERR_HIP;
    }
    c->total_ms[t.kernel] += ms;
    c->launches[t.kernel] += 1;
    c->event_pool.push_back(t.start);
    c->event_pool.push_back(t.stop);
  }
  c->pending.clear();
  *total_ms = c->total_ms[kernel_id];
  *launches = c->launches[kernel_id];
  return H2O_OK;
}

void h2o_cache_destroy(h2o_cache* c) {
  if (!c) return;
  for (const TimedLaunch& t : c->pending) {
    (void)hipEventSynchronize(t.stop);
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  for (hipEvent_t e : c->event_pool) (void)hipEventDestroy(e);
  delete c;
}

int32_t h2o_last_hip_error(const h2o_cache* c) { return c ? c->last_hip_error : 0; }

size_t h2o_backward_workspace_bytes(const h2o_config* cfg, int32_t s) {
  if (h2o_validate_config(cfg) != H2O_OK || s < 1) return 0;
  return h2o::backward_workspace_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, s, cfg->head_dim);
}

h2o_status h2o_chunk_backward(const h2o_config* cfg, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* positions, const void* k_new,
                              const void* v_new, int32_t s, const void* out, const float* lse,
                              const void* d_out, void* dq, void* dk_cache, void* dv_cache,
                              void* dk_new, void* dv_new, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!cfg || !q || !k_cache || !v_cache || !positions || !k_new || !v_new || !out || !lse ||
      !d_out || !dq || !dk_cache || !dv_cache || !dk_new || !dv_new || !workspace)
    return H2O_ERR_NULL;
  if (misaligned({q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out, dq, dk_cache, dv_cache,
                  dk_new, dv_new, workspace}))
    return H2O_ERR_ALIGN;
  h2o_status r = h2o_validate_config(cfg);
  if (r != H2O_OK) return r;
  if (cfg->dtype != H2O_BF16) return H2O_ERR_UNSUPPORTED;
  if (s < 1 || s > max_len(cfg)) return H2O_ERR_SHAPE;
  if (workspace_bytes < h2o::backward_workspace_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, s, cfg->head_dim))
    return H2O_ERR_WORKSPACE;
  const h2o::StepShape sh = backward_shape(cfg, s);
  h2o::BackwardArgs a{q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out,
                      dq, dk_cache, dv_cache, dk_new, dv_new, workspace};
  const hipError_t e = h2o::launch_backward(sh, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H2O_OK : H2O_ERR_HIP;
}

h2o_status h2o_chunk_backward_static(const h2o_config* cfg, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* positions, const void* k_new,
                                     const void* v_new, int32_t s, const void* out, const float* lse,
                                     const void* d_out, void* dq, void* dk_cache, void* dv_cache,
                                     void* dk_new, void* dv_new, void* stream) {
  if (!cfg || !q || !k_cache || !v_cache || !positions || !k_new || !v_new || !out || !lse || !d_out ||
      !dq || !dk_cache || !dv_cache || !dk_new || !dv_new)
    return H2O_ERR_NULL;
  if (misaligned({q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out, dq, dk_cache, dv_cache,
                  dk_new, dv_new}))
    return H2O_ERR_ALIGN;
  h2o_status r = h2o_validate_config(cfg);
  if (r != H2O_OK) return r;
  if (cfg->dtype != H2O_BF16) return H2O_ERR_UNSUPPORTED;
  if (s < 1 || s > max_len(cfg)) return H2O_ERR_SHAPE;
  if (h2o::backward_workspace_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, s, cfg->head_dim) >
      kStaticScratchBytes)
    return H2O_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return H2O_ERR_HIP;
  const h2o::StepShape sh = backward_shape(cfg, s);
  h2o::BackwardArgs a{q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out,
                      dq, dk_cache, dv_cache, dk_new, dv_new, ws};
  const hipError_t e = h2o::launch_backward(sh, a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? H2O_OK : H2O_ERR_HIP;
}

size_t h2o_recurrence_workspace_bytes(const h2o_config* cfg, int32_t s) {
  if (h2o_validate_config(cfg) != H2O_OK || s < 1) return 0;
  return rec_workspace_bytes(cfg, s);
}

h2o_status h2o_recurrence_backward_step(const h2o_config* cfg, void* k_cache, void* v_cache,
                                        int32_t* positions, const int32_t* slots, const void* k_old,
                                        const void* v_old, const int32_t* pos_old, const void* q,
                                        const void* k_new, const void* v_new, int32_t s, const void* out,
                                        const float* lse, const void* d_out, float* acc_k, float* acc_v,
                                        void* dq, float* gk, float* gv, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!cfg || !k_cache || !v_cache || !positions || !slots || !k_old || !v_old || !pos_old || !q ||
      !k_new || !v_new || !out || !lse || !d_out || !acc_k || !acc_v || !dq || !gk || !gv || !workspace)
    return H2O_ERR_NULL;
  if (misaligned({k_cache, v_cache, positions, slots, k_old, v_old, pos_old, q, k_new, v_new, out, lse, d_out,
                  acc_k, acc_v, dq, gk, gv, workspace}))
    return H2O_ERR_ALIGN;
  h2o_status r = h2o_validate_config(cfg);
  if (r != H2O_OK) return r;
  if (cfg->dtype != H2O_BF16) return H2O_ERR_UNSUPPORTED;
  if (s < 1 || s > max_len(cfg)) return H2O_ERR_SHAPE;
  if (workspace_bytes < rec_workspace_bytes(cfg, s)) return H2O_ERR_WORKSPACE;
  const h2o::StepShape sh = backward_shape(cfg, s);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  h2o::RecurrenceArgs ra{k_cache, v_cache, positions, slots, k_old, v_old, pos_old, acc_k, acc_v, gk, gv};
  hipError_t e = h2o::launch_undo_gather(sh, ra, cfg->dtype, st);
  if (e != hipSuccess) return H2O_ERR_HIP;
  h2o::BackwardArgs a{q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out,
                      dq, acc_k, acc_v, gk, gv, workspace, true};
  e = h2o::launch_backward(sh, a, st);
  return e == hipSuccess ? H2O_OK : H2O_ERR_HIP;
}

}  // extern "C"
