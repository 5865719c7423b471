// C ABI of libgkv (declared in include/gkv.h).  Host code: validation, pool
// bookkeeping, the per-step planner and the staging of work lists; every
// step of the attention itself runs in the kernels of kernels.hip.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/gkv.h"
#include "kernels.h"
#include "plan.h"
#include "pools.h"
#include "registry.h"

namespace {

// Dispatcher threshold on M_eff = batch * (query heads per KV head).  Fit on
// MI355X over full decode steps (Llama-3.1-8B and Qwen-2.5-14B attention
// shapes, L_p = 16K, suffixes of 128..1024 tokens, M_eff 32..3840): the
// cascade backend was at least as fast at every point up to 3840, where
// the two tie, so dense is chosen only from 4096 on.  (The page's A100
// figure is 1024.)
constexpr int32_t kDefaultMSat = 4096;
constexpr int32_t kMaxQHeads = 256;

struct Layer {
  void* k_hot = nullptr;
  void* v_hot = nullptr;
  void* k_cold = nullptr;
  void* v_cold = nullptr;
  bool bound = false;
};

}  // namespace

struct gkv_ctx {
  gkv_config cfg;
  gkv::HotPool hot;
  gkv::ColdPool cold;
  gkv::Registry reg;   // owns the prefixes admitted through gkv_prefix_acquire
  std::vector<Layer> layers;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  bool ws_clear = false;    // counters of a newly bound workspace still to be zeroed
  int32_t m_sat;
  int32_t force;
  int32_t spin_limit = gkv::kDefaultSpinLimit;   // join wait bound (polls)
  bool topo_ready = false;  // device topology read (else the gfx950 defaults plan the step)
  int32_t dev_cus = gkv::kDefaultCus;
  int32_t dev_xcds = gkv::kDefaultCus / gkv::kCusPerXcd;
  std::string err;
  gkv::StepArgs args;   // work description of the current step (~24 KB; launched in the 6 KB form up to 128 requests)
  std::vector<hipEvent_t> timing_events;   // 2 per recorded call (kernel start, end)
  int32_t timing_capacity = 0;
  int32_t timing_used = 0;
  gkv_plan_info last{};
  bool have_last = false;
  int32_t static_device = -1;   // device of the last allocation-free step (its scratch holds a status word)
  uint64_t* trace = nullptr;    // per-workgroup timeline records (gkv_step_trace), null: off
  size_t trace_bytes = 0;

  explicit gkv_ctx(const gkv_config& c)
      : cfg(c),
        hot(c.hot_capacity_tokens, gkv::kHotBlock),
        cold(static_cast<int32_t>(c.cold_capacity_tokens)),
        reg(hot, cold),
        layers(c.n_layers),
        m_sat(c.m_sat > 0 ? c.m_sat : kDefaultMSat),
        force(c.force_backend) {}
};

namespace {

int fail(gkv_ctx* ctx, int code, const std::string& msg) {
  if (ctx) ctx->err = msg;
  return code;
}

int device_fail(gkv_ctx* ctx, const char* what, hipError_t e) {
  return fail(ctx, GKV_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// Arrival counters of the in-kernel join, one per (request, KV head), at the
// start of the workspace, then the status word in a line of its own.
// Zeroed by the first step on a newly bound workspace; every step leaves the
// counters zero again (each join takes its count back off).
size_t counter_bytes(const gkv_config& c) {
  return gkv::align256(static_cast<size_t>(gkv::kMaxBatch) * c.n_kv_heads * sizeof(int32_t));
}
size_t control_bytes(const gkv_config& c) { return counter_bytes(c) + 256; }

size_t elem_size(const gkv_config& c) { return c.dtype == GKV_BF16 ? 2 : 4; }
// bytes of one element of a partial row (fp32, or the input dtype)
size_t partial_size(const gkv_config& c) { return c.partials == GKV_PARTIALS_F32 ? 4 : elem_size(c); }

gkv::PlanShape shape_of(const gkv_config& c) {
  return gkv::PlanShape{c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype == GKV_BF16};
}

int check_layer(gkv_ctx* ctx, int32_t layer) {
  if (layer < 0 || layer >= ctx->cfg.n_layers)
    return fail(ctx, GKV_ERR_INVALID, "layer " + std::to_string(layer) + " out of range");
  if (!ctx->layers[layer].bound)
    return fail(ctx, GKV_ERR_INVALID, "layer " + std::to_string(layer) + " is not bound");
  return GKV_OK;
}

}  // namespace

extern "C" {

int32_t gkv_default_m_sat(void) { return kDefaultMSat; }

int gkv_create(const gkv_config* cfg, gkv_ctx** out) {
  if (!out) return GKV_ERR_INVALID;
  *out = nullptr;
  if (!cfg) return GKV_ERR_INVALID;
  const gkv_config& c = *cfg;
  if (c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.n_q_heads % c.n_kv_heads != 0) return GKV_ERR_INVALID;
  // partial-row indices (request x split x query head) stay 32-bit
  if (c.n_q_heads > kMaxQHeads) return GKV_ERR_INVALID;
  const int32_t group = c.n_q_heads / c.n_kv_heads;
  if (group > 16) return GKV_ERR_INVALID;
  if (c.head_dim != 64 && c.head_dim != 128) return GKV_ERR_INVALID;
  if (c.dtype != GKV_F32 && c.dtype != GKV_BF16) return GKV_ERR_INVALID;
  if (c.n_layers < 1) return GKV_ERR_INVALID;
  if (c.hot_capacity_tokens < 0 || c.cold_capacity_tokens < 0 ||
      c.cold_capacity_tokens > 0x7fffffffLL || c.hot_capacity_tokens > (1LL << 40))
    return GKV_ERR_INVALID;
  if (c.force_backend < GKV_BACKEND_AUTO || c.force_backend > GKV_BACKEND_DENSE) return GKV_ERR_INVALID;
  if (c.force_backend == GKV_BACKEND_DENSE && c.dtype != GKV_BF16) return GKV_ERR_INVALID;
  if (c.partials != GKV_PARTIALS_INPUT && c.partials != GKV_PARTIALS_F32) return GKV_ERR_INVALID;
  gkv_ctx* ctx = new (std::nothrow) gkv_ctx(c);
  if (!ctx) return GKV_ERR_INVALID;
  *out = ctx;
  return GKV_OK;
}

void gkv_destroy(gkv_ctx* ctx) {
  if (!ctx) return;
  // nothing can be reported from here: release what can be released
  for (hipEvent_t e : ctx->timing_events) {
    (void)hipEventSynchronize(e);
    (void)hipEventDestroy(e);
  }
  delete ctx;
}

const char* gkv_last_error(const gkv_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

int gkv_bind_layer(gkv_ctx* ctx, int32_t layer, void* k_hot, void* v_hot, void* k_cold, void* v_cold) {
  if (!ctx) return GKV_ERR_INVALID;
  if (layer < 0 || layer >= ctx->cfg.n_layers)
    return fail(ctx, GKV_ERR_INVALID, "layer " + std::to_string(layer) + " out of range");
  if (ctx->cfg.hot_capacity_tokens >= gkv::kHotBlock && (!k_hot || !v_hot))
    return fail(ctx, GKV_ERR_INVALID, "HOT pool pointers are NULL");
  if (ctx->cfg.cold_capacity_tokens > 0 && (!k_cold || !v_cold))
    return fail(ctx, GKV_ERR_INVALID, "COLD pool pointers are NULL");
  for (void* p : {k_hot, v_hot, k_cold, v_cold})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(ctx, GKV_ERR_INVALID, "pool pointers must be 16-byte aligned");
  ctx->layers[layer] = Layer{k_hot, v_hot, k_cold, v_cold, true};
  return GKV_OK;
}

int gkv_hot_pool_bytes(const gkv_ctx* ctx, size_t* bytes) {
  if (!ctx || !bytes) return GKV_ERR_INVALID;
  const gkv_config& c = ctx->cfg;
  *bytes = static_cast<size_t>(c.n_kv_heads) * static_cast<size_t>(c.hot_capacity_tokens / gkv::kHotBlock) *
           gkv::kHotBlock * c.head_dim * elem_size(c);
  return GKV_OK;
}

int gkv_hot_write(gkv_ctx* ctx, int32_t layer, int32_t prefix_id, int32_t token_begin, int32_t n,
                  const void* k_rows, const void* v_rows, void* stream) {
  if (!ctx) return GKV_ERR_INVALID;
  if (int r = check_layer(ctx, layer)) return r;
  int64_t off;
  int32_t len;
  if (!ctx->hot.lookup(prefix_id, &off, &len))
    return fail(ctx, GKV_ERR_NOTFOUND, "prefix id " + std::to_string(prefix_id) + " is not live");
  if (n < 0 || token_begin < 0 || static_cast<int64_t>(token_begin) + n > len)
    return fail(ctx, GKV_ERR_INVALID, "hot_write: rows [" + std::to_string(token_begin) + ", +" +
                                          std::to_string(n) + ") outside the slab of " + std::to_string(len));
  if (n == 0) return GKV_OK;
  if (!k_rows || !v_rows) return fail(ctx, GKV_ERR_INVALID, "hot_write: null rows");
  const gkv_config& c = ctx->cfg;
  const Layer& L = ctx->layers[layer];
  hipError_t e = gkv::launch_hot_write(k_rows, v_rows, n, off + token_begin, c.n_kv_heads, c.head_dim, c.dtype,
                                       c.hot_capacity_tokens / gkv::kHotBlock, L.k_hot, L.v_hot,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, "hot_write launch", e);
  return GKV_OK;
}

int gkv_workspace_size(const gkv_ctx* ctx, int32_t max_batch, int64_t max_suffix_tokens, size_t* bytes) {
  if (!ctx || !bytes || max_batch < 1 || max_suffix_tokens < 0) return GKV_ERR_INVALID;
  const gkv::PlanShape s = shape_of(ctx->cfg);
  const size_t row = static_cast<size_t>(ctx->cfg.head_dim) * partial_size(ctx->cfg);
  const int64_t pr = gkv::prefix_rows_bound(s, max_batch);
  const int64_t sr = gkv::suffix_rows_bound(s, max_batch, max_suffix_tokens);
  *bytes = control_bytes(ctx->cfg) + gkv::align256(pr * row) + gkv::align256(pr * 4) + gkv::align256(sr * row) +
           gkv::align256(sr * 4);
  return GKV_OK;
}

int gkv_bind_workspace(gkv_ctx* ctx, void* dev, size_t bytes) {
  if (!ctx) return GKV_ERR_INVALID;
  if (!dev || reinterpret_cast<uintptr_t>(dev) % 256 != 0)
    return fail(ctx, GKV_ERR_INVALID, "workspace must be a non-null 256-byte aligned device pointer");
  ctx->ws = dev;
  ctx->ws_bytes = bytes;
  ctx->ws_clear = true;   // the first step on it zeroes the counters first
  return GKV_OK;
}

int gkv_hot_pool_alloc(gkv_ctx* ctx, int32_t n_tokens, int32_t* prefix_id, int64_t* token_offset) {
  if (!ctx) return GKV_ERR_INVALID;
  if (!prefix_id || !token_offset || n_tokens <= 0)
    return fail(ctx, GKV_ERR_INVALID, "hot_pool_alloc: n_tokens must be >= 1 and outputs non-null");
  const int r = ctx->hot.alloc(n_tokens, prefix_id, token_offset);
  if (r == -2)
    return fail(ctx, GKV_ERR_NOSPACE, "no free HOT extent of " + std::to_string(n_tokens) + " tokens");
  return GKV_OK;
}

int gkv_hot_pool_free(gkv_ctx* ctx, int32_t prefix_id) {
  if (!ctx) return GKV_ERR_INVALID;
  if (ctx->reg.owns_hot(prefix_id))
    return fail(ctx, GKV_ERR_INVALID, "prefix id " + std::to_string(prefix_id) +
                                          " belongs to the prefix registry (gkv_prefix_release / gkv_prefix_evict)");
  if (ctx->hot.release(prefix_id) != 0)
    return fail(ctx, GKV_ERR_NOTFOUND, "prefix id " + std::to_string(prefix_id) + " is not live");
  return GKV_OK;
}

int gkv_hot_prefix_info(const gkv_ctx* ctx, int32_t prefix_id, int64_t* token_offset, int32_t* n_tokens) {
  if (!ctx || !token_offset || !n_tokens) return GKV_ERR_INVALID;
  return ctx->hot.lookup(prefix_id, token_offset, n_tokens) ? GKV_OK : GKV_ERR_NOTFOUND;
}

int gkv_cold_pool_alloc(gkv_ctx* ctx, int32_t n, int32_t* slots_out) {
  if (!ctx) return GKV_ERR_INVALID;
  if (n < 0 || (n > 0 && !slots_out)) return fail(ctx, GKV_ERR_INVALID, "cold_pool_alloc: bad arguments");
  if (ctx->cold.alloc(n, slots_out) != 0)
    return fail(ctx, GKV_ERR_NOSPACE, std::to_string(n) + " COLD slots requested, " +
                                          std::to_string(ctx->cold.free_count()) + " free");
  return GKV_OK;
}

int gkv_cold_pool_free(gkv_ctx* ctx, const int32_t* slots, int32_t n) {
  if (!ctx) return GKV_ERR_INVALID;
  if (n < 0 || (n > 0 && !slots)) return fail(ctx, GKV_ERR_INVALID, "cold_pool_free: bad arguments");
  for (int32_t i = 0; i < n; ++i)
    if (ctx->reg.owns_cold_slot(slots[i]))
      return fail(ctx, GKV_ERR_INVALID, "cold_pool_free: slot " + std::to_string(slots[i]) +
                                            " belongs to a registry prefix (gkv_prefix_release / gkv_prefix_evict)");
  if (ctx->cold.release(slots, n) != 0)
    return fail(ctx, GKV_ERR_NOTFOUND, "cold_pool_free: a slot is out of range, not allocated or repeated");
  return GKV_OK;
}

int gkv_pool_stats(const gkv_ctx* ctx, gkv_stats* out) {
  if (!ctx || !out) return GKV_ERR_INVALID;
  out->hot_free_tokens = ctx->hot.free_tokens();
  out->hot_largest_hole = ctx->hot.largest_hole();
  out->hot_live_prefixes = ctx->hot.live_count();
  out->hot_free_extents = ctx->hot.extent_count();
  out->cold_free_slots = ctx->cold.free_count();
  return GKV_OK;
}

int gkv_partition_capacity(int64_t total_tokens, double f_p, int64_t* hot_tokens, int64_t* cold_tokens) {
  if (!hot_tokens || !cold_tokens || total_tokens < 0 || !(f_p >= 0.0 && f_p <= 1.0)) return GKV_ERR_INVALID;
  const int64_t hot = static_cast<int64_t>(f_p * static_cast<double>(total_tokens)) / gkv::kHotBlock * gkv::kHotBlock;
  const int64_t cold = total_tokens - hot;
  if (cold > 0x7fffffffLL || hot > (1LL << 40)) return GKV_ERR_INVALID;
  *hot_tokens = hot;
  *cold_tokens = cold;
  return GKV_OK;
}

namespace {
void fill_ref(const gkv::PrefixEntry& e, bool fresh, gkv_prefix_ref* out) {
  out->pool = e.pool == 0 ? GKV_POOL_HOT : GKV_POOL_COLD;
  out->prefix_id = e.pool == 0 ? e.hot_id : -1;
  out->hot_offset = e.pool == 0 ? e.offset : -1;
  out->n_tokens = e.n;
  out->fresh = fresh ? 1 : 0;
  out->refs = e.refs;
  out->reserved = 0;
}
}  // namespace

int gkv_prefix_acquire(gkv_ctx* ctx, uint64_t key, int32_t n_tokens, gkv_prefix_ref* out) {
  if (!ctx) return GKV_ERR_INVALID;
  if (!out) return fail(ctx, GKV_ERR_INVALID, "prefix_acquire: out is null");
  const gkv::PrefixEntry* e = nullptr;
  bool fresh = false;
  if (int r = ctx->reg.acquire(key, n_tokens, &e, &fresh, ctx->err)) return r;
  fill_ref(*e, fresh, out);
  return GKV_OK;
}

int gkv_prefix_lookup(const gkv_ctx* ctx, uint64_t key, gkv_prefix_ref* out) {
  if (!ctx || !out) return GKV_ERR_INVALID;
  const gkv::PrefixEntry* e = ctx->reg.find(key);
  if (!e) return GKV_ERR_NOTFOUND;
  fill_ref(*e, false, out);
  return GKV_OK;
}

int gkv_prefix_cold_slots(const gkv_ctx* ctx, uint64_t key, int32_t* slots_out, int32_t max_slots) {
  if (!ctx || !slots_out) return GKV_ERR_INVALID;
  const gkv::PrefixEntry* e = ctx->reg.find(key);
  if (!e) return GKV_ERR_NOTFOUND;
  if (e->pool != 1 || max_slots < e->n) return GKV_ERR_INVALID;
  std::copy(e->slots.begin(), e->slots.end(), slots_out);
  return GKV_OK;
}

int gkv_prefix_release(gkv_ctx* ctx, uint64_t key) {
  if (!ctx) return GKV_ERR_INVALID;
  return ctx->reg.release(key, ctx->err);
}

int gkv_prefix_evict(gkv_ctx* ctx, uint64_t key) {
  if (!ctx) return GKV_ERR_INVALID;
  return ctx->reg.evict(key, ctx->err);
}

int gkv_prefix_reclaim_cold(gkv_ctx* ctx, int32_t n_free_slots) {
  if (!ctx) return GKV_ERR_INVALID;
  return ctx->reg.reclaim_cold(n_free_slots, ctx->err);
}

int gkv_registry_stats(const gkv_ctx* ctx, gkv_registry_counts* out) {
  if (!ctx || !out) return GKV_ERR_INVALID;
  const gkv::RegistryCounts c = ctx->reg.counts();
  out->resident_hot = c.resident_hot;
  out->resident_cold = c.resident_cold;
  out->referenced = c.referenced;
  out->cached = c.cached;
  out->hits = c.hits;
  out->hot_admits = c.hot_admits;
  out->cold_admits = c.cold_admits;
  out->evictions = c.evictions;
  return GKV_OK;
}

int gkv_cold_append(gkv_ctx* ctx, int32_t layer, const void* k_new, const void* v_new,
                    const int32_t* slots_dev, int32_t n, void* stream) {
  if (!ctx) return GKV_ERR_INVALID;
  if (int r = check_layer(ctx, layer)) return r;
  if (n < 0) return fail(ctx, GKV_ERR_INVALID, "cold_append: n < 0");
  if (n == 0) return GKV_OK;
  if (!k_new || !v_new || !slots_dev) return fail(ctx, GKV_ERR_INVALID, "cold_append: null pointer");
  if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
    return fail(ctx, GKV_ERR_INVALID, "cold_append: rows must be 16-byte aligned");
  if (ctx->cfg.cold_capacity_tokens == 0) return fail(ctx, GKV_ERR_INVALID, "COLD pool is empty");
  const Layer& L = ctx->layers[layer];
  const int64_t head_bytes = static_cast<int64_t>(ctx->cfg.head_dim) * elem_size(ctx->cfg);
  hipError_t e = gkv::launch_cold_append(k_new, v_new, slots_dev, n, L.k_cold, L.v_cold, ctx->cfg.n_kv_heads,
                                         head_bytes, static_cast<int32_t>(ctx->cfg.cold_capacity_tokens),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(ctx, "cold_append launch", e);
  return GKV_OK;
}

int gkv_select_backend(const gkv_ctx* ctx, int32_t batch, int32_t* backend) {
  if (!ctx || !backend || batch < 1) return GKV_ERR_INVALID;
  int32_t b = gkv::choose_backend(batch, ctx->cfg.n_q_heads / ctx->cfg.n_kv_heads, ctx->m_sat, ctx->force);
  if (b == GKV_BACKEND_DENSE && ctx->cfg.dtype != GKV_BF16) b = GKV_BACKEND_CASCADE;
  *backend = b;
  return GKV_OK;
}

int gkv_set_dispatch(gkv_ctx* ctx, int32_t force_backend, int32_t m_sat) {
  if (!ctx) return GKV_ERR_INVALID;
  if (force_backend < GKV_BACKEND_AUTO || force_backend > GKV_BACKEND_DENSE)
    return fail(ctx, GKV_ERR_INVALID, "unknown backend");
  if (force_backend == GKV_BACKEND_DENSE && ctx->cfg.dtype != GKV_BF16)
    return fail(ctx, GKV_ERR_INVALID, "the dense backend is bf16 only");
  ctx->force = force_backend;
  if (m_sat > 0) ctx->m_sat = m_sat;
  return GKV_OK;
}

int gkv_stream_read(const void* dev, size_t bytes, int32_t workgroups, uint32_t* sink_dev, void* stream) {
  if (!dev || !sink_dev || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dev) % 16 != 0 || workgroups < 1 ||
      workgroups > (1 << 20))
    return GKV_ERR_INVALID;
  if (gkv::launch_stream_read(dev, bytes, workgroups, sink_dev, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GKV_ERR_DEVICE;
  return GKV_OK;
}

int gkv_step_trace(gkv_ctx* ctx, void* trace_dev, size_t bytes) {
  if (!ctx) return GKV_ERR_INVALID;
  if (trace_dev && reinterpret_cast<uintptr_t>(trace_dev) % 8 != 0)
    return fail(ctx, GKV_ERR_INVALID, "trace buffer must be 8-byte aligned");
  ctx->trace = static_cast<uint64_t*>(trace_dev);
  ctx->trace_bytes = trace_dev ? bytes : 0;
  return GKV_OK;
}

int gkv_set_join_spin_limit(gkv_ctx* ctx, int32_t polls) {
  if (!ctx) return GKV_ERR_INVALID;
  if (polls < -1) return fail(ctx, GKV_ERR_INVALID, "spin limit must be >= 0 (or -1 for the default)");
  ctx->spin_limit = polls == -1 ? gkv::kDefaultSpinLimit : polls;
  return GKV_OK;
}

int gkv_step_status(gkv_ctx* ctx, void* stream, int32_t* joins_timed_out) {
  if (!ctx || !joins_timed_out) return GKV_ERR_INVALID;
  *joins_timed_out = 0;
  if (!ctx->ws && ctx->static_device < 0) return fail(ctx, GKV_ERR_INVALID, "no workspace bound");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t total = 0;
  auto read_word = [&](const int32_t* status, int32_t* v) -> int {
    hipError_t e = hipMemcpyAsync(v, status, sizeof(*v), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return device_fail(ctx, "status read", e);
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return device_fail(ctx, "status read (stream sync)", e);
    return GKV_OK;
  };
  if (ctx->ws && !ctx->ws_clear) {   // else no step has run on this workspace since it was bound
    int32_t v = 0;
    if (int r = read_word(reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(ctx->ws) +
                                                           counter_bytes(ctx->cfg)), &v))
      return r;
    // a step whose join gave up leaves its counters exact (the join takes its
    // count off either way); the whole control area is still cleared before
    // the next step, which also zeroes the status word
    if (v != 0) ctx->ws_clear = true;
    total += v;
  }
  if (ctx->static_device >= 0) {   // the static scratch of the current device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_fail(ctx, "hipGetDevice", e);
    uint8_t* p = nullptr;
    bool first = false;
    if ((e = gkv::scratch_region(dev, &p, &first)) != hipSuccess)
      return device_fail(ctx, "static scratch address (hipGetSymbolAddress)", e);
    if (first) {   // never used on this device: clear it for its first step
      if ((e = gkv::launch_zero_i32(reinterpret_cast<int32_t*>(p), gkv::kStaticControlBytes / 4, st)) != hipSuccess)
        return device_fail(ctx, "scratch clear launch", e);
    } else {
      int32_t v = 0;
      if (int r = read_word(reinterpret_cast<const int32_t*>(p), &v)) return r;
      if (v != 0 && (e = gkv::launch_zero_i32(reinterpret_cast<int32_t*>(p), 1, st)) != hipSuccess)
        return device_fail(ctx, "status clear launch", e);
      total += v;
    }
  }
  *joins_timed_out = total;
  return GKV_OK;
}

int gkv_last_plan(const gkv_ctx* ctx, gkv_plan_info* out) {
  if (!ctx || !out) return GKV_ERR_INVALID;
  if (!ctx->have_last) return GKV_ERR_NOTFOUND;
  *out = ctx->last;
  return GKV_OK;
}

int gkv_kernel_timing(gkv_ctx* ctx, int32_t capacity) {
  if (!ctx) return GKV_ERR_INVALID;
  if (capacity < 0 || capacity > (1 << 20)) return fail(ctx, GKV_ERR_INVALID, "timing capacity out of range");
  hipError_t first = hipSuccess;
  for (hipEvent_t e : ctx->timing_events) {
    hipError_t r = hipEventSynchronize(e);
    if (first == hipSuccess) first = r;
    r = hipEventDestroy(e);
    if (first == hipSuccess) first = r;
  }
  ctx->timing_events.clear();
  ctx->timing_capacity = 0;
  ctx->timing_used = 0;
  if (first != hipSuccess) return device_fail(ctx, "releasing timing events", first);
  for (int32_t i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return device_fail(ctx, "hipEventCreate(timing)", r);
    ctx->timing_events.push_back(e);
  }
  ctx->timing_capacity = capacity;
  return GKV_OK;
}

int gkv_kernel_timing_read(gkv_ctx* ctx, float* ms, int32_t max_calls, int32_t* n) {
  if (!ctx || !n || max_calls < 0 || (max_calls > 0 && !ms)) return GKV_ERR_INVALID;
  const int32_t k = std::min(ctx->timing_used, max_calls);
  for (int32_t i = 0; i < ctx->timing_used; ++i) {
    hipError_t r = hipEventSynchronize(ctx->timing_events[2 * i + 1]);
    if (r != hipSuccess) return device_fail(ctx, "timing event wait", r);
  }
  for (int32_t i = 0; i < k; ++i) {
    hipEvent_t* ev = &ctx->timing_events[2 * i];
    float t01 = 0.f;
    hipError_t r = hipEventElapsedTime(&t01, ev[0], ev[1]);
    if (r != hipSuccess) return device_fail(ctx, "hipEventElapsedTime", r);
    ms[i] = t01;
  }
  *n = k;
  ctx->timing_used = 0;
  return GKV_OK;
}

}  // extern "C"

namespace {

// Compute units and XCDs of the current device, read once per context.  The
// library is built for gfx950 only; another device is refused.  Without a
// device (host-only use) the gfx950 values stay and the launch reports the
// missing device.
int read_topology(gkv_ctx* ctx) {
  if (ctx->topo_ready) return GKV_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GKV_OK;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return GKV_OK;
  }
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(ctx, GKV_ERR_DEVICE, std::string("libgkv is built for gfx950; device ") + std::to_string(dev) +
                                         " is " + prop.gcnArchName);
  const int cus = prop.multiProcessorCount;
  if (cus < gkv::kCusPerXcd || cus % gkv::kCusPerXcd != 0)
    return fail(ctx, GKV_ERR_DEVICE, "unexpected compute-unit count " + std::to_string(cus) +
                                         " (gfx950 XCDs hold " + std::to_string(gkv::kCusPerXcd) + ")");
  ctx->dev_cus = cus;
  ctx->dev_xcds = cus / gkv::kCusPerXcd;
  ctx->topo_ready = true;
  return GKV_OK;
}

// Workspace layout of a planned step: [counters][status][prefix o][prefix
// lse][suffix o][suffix lse]; in the static scratch: [status][counters (room
// for any context)][the same partials].
struct StepLayout {
  size_t off_po, off_pl, off_so, off_sl, need;
};
StepLayout step_layout(const gkv_config& c, const gkv::Plan& plan, bool use_static) {
  const size_t row = static_cast<size_t>(c.head_dim) * partial_size(c);
  StepLayout l;
  l.off_po = use_static ? gkv::kStaticControlBytes : control_bytes(c);
  l.off_pl = l.off_po + gkv::align256(plan.prefix_rows * row);
  l.off_so = l.off_pl + gkv::align256(plan.prefix_rows * 4);
  l.off_sl = l.off_so + gkv::align256(plan.suffix_rows * row);
  l.need = l.off_sl + gkv::align256(plan.suffix_rows * 4);
  return l;
}

// The backend of a step of `batch` requests (the rule, or the forced one);
// dense with fp32 elements falls back to cascade unless forced (an error).
int step_backend(gkv_ctx* ctx, int32_t batch, int32_t* backend) {
  const gkv_config& c = ctx->cfg;
  *backend = gkv::choose_backend(batch, c.n_q_heads / c.n_kv_heads, ctx->m_sat, ctx->force);
  if (*backend == GKV_BACKEND_DENSE && c.dtype != GKV_BF16) {
    if (ctx->force == GKV_BACKEND_DENSE) return fail(ctx, GKV_ERR_INVALID, "the dense backend is bf16 only");
    *backend = GKV_BACKEND_CASCADE;
  }
  return GKV_OK;
}

gkv::PlanShape plan_shape(const gkv_ctx* ctx) {
  gkv::PlanShape shape = shape_of(ctx->cfg);
  shape.xcds = ctx->dev_xcds;
  shape.cus = ctx->dev_cus;
  return shape;
}

void fill_info(gkv_plan_info& i, const gkv::Plan& plan, int32_t backend, size_t need) {
  i.backend = backend;
  i.m_eff = plan.m_eff;
  i.n_classes = plan.n_classes;
  i.n_prefix_blocks = plan.prefix_blocks;
  i.n_suffix_blocks = plan.suffix_blocks;
  i.n_suffix_parts = plan.n_parts;
  i.joins_partials = plan.multi_part;
  i.suffix_part_tokens = plan.part_tokens;
  i.folded_parts = plan.fold;
  i.n_join_blocks = plan.join_blocks;
  i.n_short_requests = plan.n_short;
  i.workspace_bytes = static_cast<int64_t>(need);
}

// The decode step behind gkv_attn_decode (k_new == nullptr), gkv_decode_step
// (the batch's new tokens appended inside the launch) and
// gkv_decode_step_static (the same, its scratch in the library's static
// device array instead of the bound workspace).
int decode_impl(gkv_ctx* ctx, int32_t layer, const void* q, const void* k_new, const void* v_new,
                const int32_t* new_slots_d, int32_t batch, const int32_t* hot_prefix_ids,
                const int32_t* cold_indptr_h, const int32_t* cold_indices_d, void* out, float* lse,
                void* stream, int32_t* backend_out, bool use_static = false) {
  if (!ctx) return GKV_ERR_INVALID;
  const auto t_start = std::chrono::steady_clock::now();
  if (int r = read_topology(ctx)) return r;
  if (int r = check_layer(ctx, layer)) return r;
  if (batch < 1) return fail(ctx, GKV_ERR_INVALID, "batch must be >= 1");
  if (!q || !out || !lse || !hot_prefix_ids || !cold_indptr_h)
    return fail(ctx, GKV_ERR_INVALID, "attn_decode: null pointer argument");
  if (!use_static && !ctx->ws) return fail(ctx, GKV_ERR_INVALID, "no workspace bound");
  const gkv_config& c = ctx->cfg;
  const int32_t group = c.n_q_heads / c.n_kv_heads;
  const bool any_suffix = cold_indptr_h[batch] != cold_indptr_h[0];
  if (any_suffix && !cold_indices_d)
    return fail(ctx, GKV_ERR_INVALID, "attn_decode: slot table pointer is null");
  if (any_suffix && c.cold_capacity_tokens == 0)
    return fail(ctx, GKV_ERR_INVALID, "slot tables given but the COLD pool is empty");
  if (k_new) {
    if (!v_new || !new_slots_d) return fail(ctx, GKV_ERR_INVALID, "decode_step: null pointer argument");
    if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16)
      return fail(ctx, GKV_ERR_INVALID, "decode_step: new rows must be 16-byte aligned");
    for (int32_t b = 0; b < batch; ++b)
      if (cold_indptr_h[b + 1] <= cold_indptr_h[b])
        return fail(ctx, GKV_ERR_INVALID, "decode_step: request " + std::to_string(b) +
                                              " has an empty slot table (its new token must be its last entry)");
  }

  int32_t backend = 0;
  if (int r = step_backend(ctx, batch, &backend)) return r;

  gkv::Plan plan;
  std::string err;
  gkv::StepArgs& a = ctx->args;
  if (gkv::build_plan(plan_shape(ctx), ctx->hot, batch, hot_prefix_ids, cold_indptr_h, backend, a, plan, err) != 0)
    return fail(ctx, GKV_ERR_INVALID, err);

  const StepLayout lay = step_layout(c, plan, use_static);
  const size_t off_po = lay.off_po, off_pl = lay.off_pl, off_so = lay.off_so, off_sl = lay.off_sl;
  const size_t need = lay.need;
  if (use_static && need > gkv::kStaticScratchBytes)
    return fail(ctx, GKV_ERR_INVALID, "step needs " + std::to_string(need) + " bytes of scratch; the static "
                                      "scratch of gkv_decode_step_static holds " +
                                          std::to_string(gkv::kStaticScratchBytes) +
                                          " (use gkv_decode_step with a workspace)");
  if (!use_static && need > ctx->ws_bytes)
    return fail(ctx, GKV_ERR_INVALID, "workspace too small: step needs " + std::to_string(need) +
                                          " bytes, " + std::to_string(ctx->ws_bytes) + " bound");
  uint8_t* ws = static_cast<uint8_t*>(ctx->ws);
  bool clear_static = false;
  if (use_static) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_fail(ctx, "hipGetDevice", e);
    if ((e = gkv::scratch_region(dev, &ws, &clear_static)) != hipSuccess)
      return device_fail(ctx, "static scratch address (hipGetSymbolAddress)", e);
    ctx->static_device = dev;
  }
  const auto t_planned = std::chrono::steady_clock::now();

  const Layer& L = ctx->layers[layer];
  a.batch = batch;
  a.n_q = c.n_q_heads;
  a.n_kv = c.n_kv_heads;
  a.group = group;
  a.head_dim = c.head_dim;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(c.head_dim)));
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.k_hot = L.k_hot;
  a.v_hot = L.v_hot;
  a.hot_blocks = c.hot_capacity_tokens / gkv::kHotBlock;
  a.k_cold = L.k_cold;
  a.v_cold = L.v_cold;
  a.cold_cap = static_cast<int32_t>(c.cold_capacity_tokens);
  a.cold_mask = gkv::cold_mask_for(c.n_kv_heads);
  a.cold_indices = cold_indices_d;
  a.k_new = k_new;
  a.v_new = k_new ? v_new : nullptr;
  a.new_slots = k_new ? new_slots_d : nullptr;
  a.counters = reinterpret_cast<int32_t*>(ws + (use_static ? gkv::kStaticCounterOffset : 0));
  a.status = reinterpret_cast<int32_t*>(ws + (use_static ? 0 : counter_bytes(c)));
  a.spin_limit = ctx->spin_limit;
  a.partial_f32 = partial_size(c) == 4 ? 1 : 0;
  a.p_o = ws + off_po;
  a.p_lse = reinterpret_cast<float*>(ws + off_pl);
  a.s_o = ws + off_so;
  a.s_lse = reinterpret_cast<float*>(ws + off_sl);
  a.narrow_ws = need < 0x7fffffffull ? 1 : 0;   // partial stores may use 32-bit offsets
  const size_t grid = static_cast<size_t>(a.prefix_blocks) + a.suffix_blocks + a.join_blocks;
  a.trace = ctx->trace && ctx->trace_bytes >= grid * gkv::kTraceWords * sizeof(uint64_t) ? ctx->trace : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  hipEvent_t* ev = nullptr;
  if (ctx->timing_used < ctx->timing_capacity) {
    ev = &ctx->timing_events[2 * ctx->timing_used];
    ctx->timing_used++;
  }
  if (use_static && clear_static) {
    // first use of this device's scratch: status and every counter to zero
    // (each step leaves the counters at zero again)
    if ((e = gkv::launch_zero_i32(reinterpret_cast<int32_t*>(ws), gkv::kStaticControlBytes / 4, st)) != hipSuccess)
      return device_fail(ctx, "scratch clear launch", e);
  }
  if (!use_static && ctx->ws_clear) {
    if ((e = gkv::launch_zero_i32(a.counters, control_bytes(c) / 4, st)) != hipSuccess)
      return device_fail(ctx, "counter clear launch", e);
    ctx->ws_clear = false;
  }
  if ((e = gkv::launch_step(a, c.dtype, backend, st, ev)) != hipSuccess) return device_fail(ctx, "step launch", e);
  const auto t_launched = std::chrono::steady_clock::now();

  fill_info(ctx->last, plan, backend, need);
  ctx->last.host_plan_us = std::chrono::duration<double, std::micro>(t_planned - t_start).count();
  ctx->last.host_call_us = std::chrono::duration<double, std::micro>(t_launched - t_start).count();
  ctx->have_last = true;
  if (backend_out) *backend_out = backend;
  return GKV_OK;
}

}  // namespace

extern "C" {

int gkv_plan_step(gkv_ctx* ctx, int32_t batch, const int32_t* hot_prefix_ids, const int32_t* cold_indptr_h,
                  gkv_plan_info* out) {
  if (!ctx || !out) return GKV_ERR_INVALID;
  const auto t_start = std::chrono::steady_clock::now();
  if (int r = read_topology(ctx)) return r;
  if (batch < 1) return fail(ctx, GKV_ERR_INVALID, "batch must be >= 1");
  if (!hot_prefix_ids || !cold_indptr_h) return fail(ctx, GKV_ERR_INVALID, "plan_step: null pointer argument");
  int32_t backend = 0;
  if (int r = step_backend(ctx, batch, &backend)) return r;
  gkv::Plan plan;
  std::string err;
  if (gkv::build_plan(plan_shape(ctx), ctx->hot, batch, hot_prefix_ids, cold_indptr_h, backend, ctx->args, plan,
                      err) != 0)
    return fail(ctx, GKV_ERR_INVALID, err);
  gkv_plan_info info{};
  fill_info(info, plan, backend, step_layout(ctx->cfg, plan, false).need);
  info.host_plan_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t_start).count();
  info.host_call_us = 0.0;
  *out = info;
  return GKV_OK;
}

int gkv_attn_decode(gkv_ctx* ctx, int32_t layer, const void* q, int32_t batch,
                    const int32_t* hot_prefix_ids, const int32_t* cold_indptr_h,
                    const int32_t* cold_indptr_d, const int32_t* cold_indices_d, void* out,
                    float* lse, void* stream, int32_t* backend_out) {
  (void)cold_indptr_d;
  return decode_impl(ctx, layer, q, nullptr, nullptr, nullptr, batch, hot_prefix_ids, cold_indptr_h,
                     cold_indices_d, out, lse, stream, backend_out);
}

int gkv_decode_step(gkv_ctx* ctx, int32_t layer, const void* q, const void* k_new, const void* v_new,
                    const int32_t* new_slots_d, int32_t batch, const int32_t* hot_prefix_ids,
                    const int32_t* cold_indptr_h, const int32_t* cold_indices_d, void* out, float* lse,
                    void* stream, int32_t* backend_out) {
  if (!ctx) return GKV_ERR_INVALID;
  if (!k_new) return fail(ctx, GKV_ERR_INVALID, "decode_step: null pointer argument");
  return decode_impl(ctx, layer, q, k_new, v_new, new_slots_d, batch, hot_prefix_ids, cold_indptr_h,
                     cold_indices_d, out, lse, stream, backend_out);
}

int gkv_decode_step_static(gkv_ctx* ctx, int32_t layer, const void* q, const void* k_new, const void* v_new,
                           const int32_t* new_slots_d, int32_t batch, const int32_t* hot_prefix_ids,
                           const int32_t* cold_indptr_h, const int32_t* cold_indices_d, void* out, float* lse,
                           void* stream, int32_t* backend_out) {
  if (!ctx) return GKV_ERR_INVALID;
  if (!k_new) return fail(ctx, GKV_ERR_INVALID, "decode_step: null pointer argument");
  return decode_impl(ctx, layer, q, k_new, v_new, new_slots_d, batch, hot_prefix_ids, cold_indptr_h,
                     cold_indices_d, out, lse, stream, backend_out, true);
}

}  // extern "C"
