// extern "C" entry points of libskvd.so: error state, plan lifetime, validation and the
// launch sequence (partial kernel, then the plan's reducer) on the caller's stream.
// A decode call makes no allocation, no synchronization and no device-to-host read, so it
// can be captured into a HIP graph (llama-cpp-turboquant PR #176: the decode crash under
// graph capture came from allocating inside the captured launch).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "skvd_internal.h"

struct skvd_plan {
  skvd::Plan p;
};

namespace {

thread_local char g_err[512];

skvd_status set_err(skvd_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

skvd_status hip_err(int e, const char *what) {
  return set_err(SKVD_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
}

// The current HIP device must be the plan's (launches go to the current device).
skvd_status check_device(const skvd::Plan &p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(SKVD_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev != p.prm.device)
    return set_err(SKVD_ERR_DEVICE, "current device %d is not the plan's device %d", dev,
                   p.prm.device);
  return SKVD_OK;
}

skvd_status common_checks(const skvd_plan *plan, const skvd_decode_args *args, void *ws,
                          size_t ws_bytes) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  skvd_status st = skvd::check_args(plan->p, args, ws_bytes, g_err, sizeof g_err);
  if (st != SKVD_OK) return st;
  if (!ws) return set_err(SKVD_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws % skvd::kAlign)
    return set_err(SKVD_ERR_WORKSPACE, "workspace must be %zu-byte aligned", skvd::kAlign);
  return check_device(plan->p);
}

// skvd_append's host checks (shapes and layout the append kernel addresses; no HIP call).
skvd_status check_append(const skvd_plan *plan, const skvd_append_args *a) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  if (!a) return set_err(SKVD_ERR_NULL, "args is NULL");
  const skvd::Plan &p = plan->p;
  const bool q4 = p.prm.kv_dtype == SKVD_KV_Q4_0;
  const bool i8 = p.prm.kv_dtype == SKVD_KV_I8_F16SCALE32 || q4;  // f16 scales per 32 elements
  const bool f8 = p.prm.kv_dtype == SKVD_KV_FP8_E4M3;
  const auto al = [](const void *ptr, uintptr_t n) { return (uintptr_t)ptr % n == 0; };
  if (a->num_tokens < 0 || a->batch < 0)
    return set_err(SKVD_ERR_SHAPE, "num_tokens=%d and batch=%d must be >= 0", a->num_tokens,
                   a->batch);
  if (a->num_tokens > 0 && (!a->k_new || !a->v_new || !a->batch_idx || !a->positions))
    return set_err(SKVD_ERR_NULL, "k_new, v_new, batch_idx and positions must be non-NULL "
                   "when num_tokens > 0");
  if (!a->k_pages || !a->v_pages || !a->page_table)
    return set_err(SKVD_ERR_NULL, "k_pages, v_pages and page_table must be non-NULL");
  if ((i8 || f8) && (!a->k_scales || !a->v_scales))
    return set_err(SKVD_ERR_DTYPE, "%s cache needs k_scales and v_scales",
                   q4 ? "q4_0" : i8 ? "int8" : "fp8");
  if (!i8 && !f8 && (a->k_scales || a->v_scales))
    return set_err(SKVD_ERR_DTYPE, "f16 cache takes no scales");
  if (f8 && (!al(a->k_scales, 4) || !al(a->v_scales, 4)))
    return set_err(SKVD_ERR_LAYOUT, "fp8 k_scale / v_scale must be 4-byte aligned");
  if (!al(a->k_new, 16) || !al(a->v_new, 16) || a->new_tok_stride < 0 || a->new_head_stride < 0 ||
      a->new_tok_stride % 8 || a->new_head_stride % 8)
    return set_err(SKVD_ERR_LAYOUT, "k_new/v_new must be 16-byte aligned with token/head strides "
                   "that are non-negative multiples of 8 elements");
  const int64_t kv_vec = i8 || f8 ? 16 : 8;  // the decode's rule: strides of 16 bytes
  if (!al(a->k_pages, 16) || !al(a->v_pages, 16) || a->page_stride < 0 || a->tok_stride < 0 ||
      a->head_stride < 0 || a->page_stride % kv_vec || a->tok_stride % kv_vec ||
      a->head_stride % kv_vec)
    return set_err(SKVD_ERR_LAYOUT, "K/V pools must be 16-byte aligned and have page/token/head "
                   "strides that are non-negative multiples of 16 bytes");
  if (i8 && (!al(a->k_scales, 8) || !al(a->v_scales, 8) || a->scale_page_stride < 0 ||
             a->scale_tok_stride < 0 || a->scale_head_stride < 0 || a->scale_page_stride % 4 ||
             a->scale_tok_stride % 4 || a->scale_head_stride % 4))
    return set_err(SKVD_ERR_LAYOUT, "scale pools must be 8-byte aligned with non-negative "
                   "strides that are multiples of 4 elements");
  if (a->num_k_pages < 1 || a->num_v_pages < 1)
    return set_err(SKVD_ERR_SHAPE, "num_k_pages and num_v_pages must be >= 1");
  const int64_t need = (p.prm.max_kv_len + p.prm.page_size - 1) / p.prm.page_size;
  if (a->table_stride < need)
    return set_err(SKVD_ERR_LAYOUT, "table_stride=%lld below ceil(max_kv_len/P)=%lld",
                   (long long)a->table_stride, (long long)need);
  // The append kernel numbers its lanes (num_tokens * Hkv * D / 8) in 32 bits.
  if ((int64_t)a->num_tokens * p.prm.num_kv_heads * (p.prm.head_dim / 8) >= (int64_t(1) << 31))
    return set_err(SKVD_ERR_SHAPE, "num_tokens=%d too large for one append (split the call)",
                   a->num_tokens);
  return SKVD_OK;
}

// skvd_prefill's host checks: the decode's layout and shape checks with any number of query
// tokens per sequence (1..max_kv_len) and no workspace; G <= 64 (a workgroup's 64 rows).
skvd_status check_prefill(const skvd_plan *plan, const skvd_decode_args *a) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  if (!a) return set_err(SKVD_ERR_NULL, "args is NULL");
  const skvd::Plan &p = plan->p;
  if (a->q_per_seq < 1 || a->q_per_seq > p.prm.max_kv_len)
    return set_err(SKVD_ERR_SHAPE, "q_per_seq=%d outside 1..max_kv_len=%d", a->q_per_seq,
                   p.prm.max_kv_len);
  if (p.group > 64)
    return set_err(SKVD_ERR_SHAPE, "prefill needs Hq/Hkv <= 64 (got %d)", p.group);
  if (p.prm.head_dim != 128 && p.prm.head_dim != 256)
    return set_err(SKVD_ERR_SHAPE, "the multi-token route supports head_dim 128 and 256 (plan "
                   "has %d)", p.prm.head_dim);
  skvd_decode_args one = *a;
  one.q_per_seq = 1;  // the remaining checks do not depend on the token count
  return skvd::check_args(p, &one, p.ws_bytes, g_err, sizeof g_err);
}

// ---- the allocation-free decode's workspace: one file-scope device array per GPU. In host code
// `scratch` names a host-side stand-in, not device memory: every use goes through the device
// address hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = size_t(32) << 20;  // SKVD_NOALLOC_WORKSPACE_MAX
static_assert(kScratchBytes == SKVD_NOALLOC_WORKSPACE_MAX, "header and library agree");
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up once per device, with that device current).
skvd_status device_scratch(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices)
    return set_err(SKVD_ERR_DEVICE, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return set_err(SKVD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                     hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SKVD_OK;
}

}  // namespace

extern "C" {

const char *skvd_status_string(skvd_status s) {
  switch (s) {
    case SKVD_OK: return "ok";
    case SKVD_ERR_NULL: return "null pointer";
    case SKVD_ERR_SHAPE: return "bad shape";
    case SKVD_ERR_LAYOUT: return "bad layout";
    case SKVD_ERR_DTYPE: return "bad dtype";
    case SKVD_ERR_WORKSPACE: return "bad workspace";
    case SKVD_ERR_DEVICE: return "device error";
    case SKVD_ERR_PLAN: return "bad plan";
    case SKVD_ERR_HIP: return "hip error";
  }
  return "unknown status";
}

const char *skvd_last_error(void) { return g_err; }

int32_t skvd_abi_version(void) { return SKVD_ABI_VERSION; }

skvd_status skvd_plan_create(const skvd_plan_params *params, skvd_plan **out) {
  g_err[0] = 0;
  if (!params || !out) return set_err(SKVD_ERR_NULL, "params and out must be non-NULL");
  *out = nullptr;
  int cus = params->num_cus;
  if (cus <= 0) {
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                                         params->device);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return set_err(SKVD_ERR_DEVICE, "querying the CU count of device %d: %s", params->device,
                     hipGetErrorString(e));
    }
  }
  skvd_plan *pl = new (std::nothrow) skvd_plan;
  if (!pl) return set_err(SKVD_ERR_PLAN, "out of host memory");
  skvd_status st = skvd::make_plan(*params, cus, &pl->p, g_err, sizeof g_err);
  if (st != SKVD_OK) {
    delete pl;
    return st;
  }
  const char *log = getenv("SKVD_LOG_DISPATCH");
  if (log && log[0] == '1') {
    char buf[512];
    skvd_plan_describe(pl, buf, sizeof buf);
    fprintf(stderr, "[skvd] %s\n", buf);
  }
  *out = pl;
  return SKVD_OK;
}

void skvd_plan_destroy(skvd_plan *plan) { delete plan; }

size_t skvd_plan_workspace_bytes(const skvd_plan *plan) { return plan ? plan->p.ws_bytes : 0; }

skvd_status skvd_plan_get_info(const skvd_plan *plan, skvd_plan_info *info) {
  g_err[0] = 0;
  if (!plan || !info) return set_err(SKVD_ERR_NULL, "plan and info must be non-NULL");
  const skvd::Plan &p = plan->p;
  info->blocks_per_split = p.bps;
  info->splits_cap = p.splits_cap;
  info->reducer = p.reducer;
  info->hier_groups_cap = p.hier_groups_cap;
  info->rows_per_group = p.rows_per_wg;
  info->num_cus = p.num_cus;
  info->rows_cap = p.rows_cap;
  info->workspace_bytes = p.ws_bytes;
  info->status_offset = p.off_status;
  info->schedule = p.schedule;
  info->part_stride = p.part_stride;
  info->grid_wgs = p.grid_wgs;
  info->heads_per_wg = p.heads_per_wg;
  return SKVD_OK;
}

skvd_status skvd_plan_describe(const skvd_plan *plan, char *buf, size_t n) {
  g_err[0] = 0;
  if (!plan || !buf || n == 0) return set_err(SKVD_ERR_NULL, "plan and buf must be non-NULL");
  const skvd::Plan &p = plan->p;
  const int kv = p.prm.kv_dtype;
  const char *fmt = kv == SKVD_KV_F16             ? "f16"
                    : kv == SKVD_KV_FP8_E4M3      ? "fp8"
                    : kv == SKVD_KV_Q4_0          ? "q4_0"
                                                  : "int8";
  snprintf(buf, n,
           "plan Hq=%d Hkv=%d D=%d P=%d kv=%s max_batch=%d max_T=%d max_kv_len=%d cus=%d: "
           "blocks_per_split=%d splits=%d schedule=%s grid=%d heads_per_wg=%d reducer=%s "
           "hier_groups=%d rows_per_wg=%d workspace=%zu B",
           p.prm.num_qo_heads, p.prm.num_kv_heads, p.prm.head_dim, p.prm.page_size,
           fmt, p.prm.max_batch, p.prm.max_q_per_seq,
           p.prm.max_kv_len, p.num_cus, p.bps, p.splits_cap,
           p.schedule == SKVD_SCHEDULE_BALANCED ? "balanced" : "static", p.grid_wgs,
           p.heads_per_wg,
           skvd::reducer_name(p.reducer),
           p.hier_groups_cap, p.rows_per_wg, p.ws_bytes);
  return SKVD_OK;
}

skvd_status skvd_decode_check(const skvd_plan *plan, const skvd_decode_args *args,
                              size_t workspace_bytes) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  return skvd::check_args(plan->p, args, workspace_bytes, g_err, sizeof g_err);
}

skvd_status skvd_decode_partial(const skvd_plan *plan, const skvd_decode_args *args,
                                void *workspace, size_t workspace_bytes, void *stream) {
  skvd_status st = common_checks(plan, args, workspace, workspace_bytes);
  if (st != SKVD_OK || args->batch == 0) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, workspace, &la);
  int e = skvd::launch_partial(plan->p, la, stream);
  return e ? hip_err(e, "partial kernel launch") : SKVD_OK;
}

skvd_status skvd_decode_partial_timed(const skvd_plan *plan, const skvd_decode_args *args,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      void *start_event, void *stop_event) {
  skvd_status st = common_checks(plan, args, workspace, workspace_bytes);
  if (st != SKVD_OK || args->batch == 0) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, workspace, &la);
  int e = skvd::launch_partial(plan->p, la, stream, start_event, stop_event);
  return e ? hip_err(e, "partial kernel launch") : SKVD_OK;
}

skvd_status skvd_decode_merge(const skvd_plan *plan, const skvd_decode_args *args,
                              void *workspace, size_t workspace_bytes, void *stream) {
  skvd_status st = common_checks(plan, args, workspace, workspace_bytes);
  if (st != SKVD_OK || args->batch == 0) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, workspace, &la);
  int e = skvd::launch_merge(plan->p, la, stream);
  return e ? hip_err(e, "merge kernel launch") : SKVD_OK;
}

skvd_status skvd_decode(const skvd_plan *plan, const skvd_decode_args *args, void *workspace,
                        size_t workspace_bytes, void *stream) {
  skvd_status st = common_checks(plan, args, workspace, workspace_bytes);
  if (st != SKVD_OK || args->batch == 0) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, workspace, &la);
  int e = skvd::launch_partial(plan->p, la, stream);
  if (e) return hip_err(e, "partial kernel launch");
  e = skvd::launch_merge(plan->p, la, stream);
  return e ? hip_err(e, "merge kernel launch") : SKVD_OK;
}

skvd_status skvd_decode_noalloc(const skvd_plan *plan, const skvd_decode_args *args,
                                void *stream) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  if (plan->p.ws_bytes > kScratchBytes)
    return set_err(SKVD_ERR_WORKSPACE, "the plan's workspace of %zu bytes exceeds the %zu bytes "
                   "of the allocation-free decode's device array (use skvd_decode with a "
                   "workspace)", plan->p.ws_bytes, kScratchBytes);
  if (plan->p.prm.debug)
    return set_err(SKVD_ERR_PLAN, "debug plans record their status word in a caller workspace: "
                   "use skvd_decode");
  skvd_status st = skvd::check_args(plan->p, args, plan->p.ws_bytes, g_err, sizeof g_err);
  if (st == SKVD_OK) st = check_device(plan->p);
  if (st != SKVD_OK || args->batch == 0) return st;
  void *ws = nullptr;
  st = device_scratch(plan->p.prm.device, &ws);
  if (st != SKVD_OK) return st;
  // every partial the merge reads is written by the same call's partial kernel, so nothing in
  // the array needs clearing (the status word is only written by debug plans)
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, ws, &la);
  int e = skvd::launch_partial(plan->p, la, stream);
  if (e) return hip_err(e, "partial kernel launch");
  e = skvd::launch_merge(plan->p, la, stream);
  return e ? hip_err(e, "merge kernel launch") : SKVD_OK;
}

skvd_status skvd_attention(const skvd_plan *plan, const skvd_decode_args *args, void *workspace,
                           size_t workspace_bytes, void *stream) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  if (!args) return set_err(SKVD_ERR_NULL, "args is NULL");
  // the routing threshold of the pages: at most 8 query tokens (and the plan's bound) on the
  // split-KV decode, more on the tiled route
  if (args->q_per_seq <= plan->p.prm.max_q_per_seq)
    return skvd_decode(plan, args, workspace, workspace_bytes, stream);
  return skvd_prefill(plan, args, stream);
}

skvd_status skvd_gather_debug(const skvd_plan *plan, const skvd_decode_args *args,
                              int32_t max_len, void *dense_k, void *dense_v, void *dense_ks,
                              void *dense_vs, void *stream) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  skvd_status st = skvd::check_args(plan->p, args, plan->p.ws_bytes, g_err, sizeof g_err);
  if (st != SKVD_OK) return st;
  const bool i8 = plan->p.prm.kv_dtype == SKVD_KV_I8_F16SCALE32 ||
                  plan->p.prm.kv_dtype == SKVD_KV_Q4_0;  // per-row scales
  if (!dense_k || !dense_v || (i8 && (!dense_ks || !dense_vs)))
    return set_err(SKVD_ERR_NULL, "dense outputs must be non-NULL");
  if (max_len < 0 || max_len > plan->p.prm.max_kv_len)
    return set_err(SKVD_ERR_SHAPE, "max_len=%d outside 0..max_kv_len", max_len);
  // the partial kernel's stores: 16 bytes of f16 / 8 bytes of one-byte K and V rows, 2-byte
  // scales
  if (((uintptr_t)dense_k | (uintptr_t)dense_v) % 16 ||
      (i8 && ((uintptr_t)dense_ks | (uintptr_t)dense_vs) % 2))
    return set_err(SKVD_ERR_LAYOUT, "dense_k and dense_v must be 16-byte aligned, dense_ks and "
                   "dense_vs 2-byte aligned");
  st = check_device(plan->p);
  if (st != SKVD_OK) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, nullptr, &la);
  la.debug = 0;
  la.dbg_k = (char *)dense_k;
  la.dbg_v = (char *)dense_v;
  la.dbg_ks = (uint16_t *)dense_ks;
  la.dbg_vs = (uint16_t *)dense_vs;
  la.dbg_max_len = max_len;
  int e = skvd::launch_gather(plan->p, la, stream);
  return e ? hip_err(e, "gather kernel launch") : SKVD_OK;
}

skvd_status skvd_prefill_check(const skvd_plan *plan, const skvd_decode_args *args) {
  return check_prefill(plan, args);
}

skvd_status skvd_prefill(const skvd_plan *plan, const skvd_decode_args *args, void *stream) {
  skvd_status st = check_prefill(plan, args);
  if (st == SKVD_OK) st = check_device(plan->p);
  if (st != SKVD_OK) return st;
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, nullptr, &la);
  const int e = skvd::launch_prefill(la, stream);
  return e ? hip_err(e, "prefill kernel launch") : SKVD_OK;
}

skvd_status skvd_append_check(const skvd_plan *plan, const skvd_append_args *args) {
  return check_append(plan, args);
}

skvd_status skvd_append(const skvd_plan *plan, const skvd_append_args *a, void *stream) {
  skvd_status st = check_append(plan, a);
  if (st == SKVD_OK) st = check_device(plan->p);
  if (st != SKVD_OK) return st;
  const skvd::Plan &p = plan->p;
  skvd::AppendLaunch l{};
  l.k_new = a->k_new;
  l.v_new = a->v_new;
  l.new_tok_stride = a->new_tok_stride;
  l.new_head_stride = a->new_head_stride;
  l.batch_idx = a->batch_idx;
  l.positions = a->positions;
  l.k = a->k_pages;
  l.v = a->v_pages;
  l.page_stride = a->page_stride;
  l.tok_stride = a->tok_stride;
  l.head_stride = a->head_stride;
  l.num_k_pages = a->num_k_pages;
  l.num_v_pages = a->num_v_pages;
  l.ks = a->k_scales;
  l.vs = a->v_scales;
  l.s_page_stride = a->scale_page_stride;
  l.s_tok_stride = a->scale_tok_stride;
  l.s_head_stride = a->scale_head_stride;
  l.table = a->page_table;
  l.table_stride = a->table_stride;
  l.num_tokens = a->num_tokens;
  l.batch = a->batch;
  l.Hkv = p.prm.num_kv_heads;
  l.D = p.prm.head_dim;
  l.rows = (int64_t)a->num_tokens * l.Hkv;
  int sh = 0;
  while ((1 << sh) < p.prm.page_size) ++sh;
  l.page_shift = sh;
  l.max_len = p.prm.max_kv_len;
  l.int8 = p.prm.kv_dtype == SKVD_KV_I8_F16SCALE32;
  l.fp8 = p.prm.kv_dtype == SKVD_KV_FP8_E4M3;
  l.q4 = p.prm.kv_dtype == SKVD_KV_Q4_0;
  l.num_cus = p.num_cus;
  int e = skvd::launch_append(l, stream);
  return e ? hip_err(e, "append kernel launch") : SKVD_OK;
}

skvd_status skvd_merge_states(const void *o_states, int64_t o_state_stride, int64_t o_row_stride,
                              const float *lse_states, int64_t lse_state_stride,
                              int32_t num_states, int64_t rows, int32_t head_dim, void *o,
                              float *lse, void *stream) {
  g_err[0] = 0;
  if (!o_states || !lse_states || !o)
    return set_err(SKVD_ERR_NULL, "o_states, lse_states and o must be non-NULL");
  if (num_states < 1 || rows < 0 || rows > (int64_t(1) << 31))
    return set_err(SKVD_ERR_SHAPE, "num_states=%d must be >= 1 and rows=%lld in 0..2^31",
                   num_states, (long long)rows);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
    return set_err(SKVD_ERR_SHAPE, "head_dim=%d not in {64, 128, 256, 512}", head_dim);
  const int64_t vec = 8;  // f16 elements one lane reads (16 bytes)
  if ((uintptr_t)o_states % (2 * vec) || (uintptr_t)o % (2 * vec) || o_state_stride < 0 ||
      o_row_stride < 0 || o_state_stride % vec || o_row_stride % vec ||
      (uintptr_t)lse_states % 4 || (lse && (uintptr_t)lse % 4) || lse_state_stride < 0)
    return set_err(SKVD_ERR_LAYOUT, "o_states and o must be %lld-byte aligned with "
                   "non-negative strides that are multiples of %lld elements; lse arrays "
                   "4-byte aligned", (long long)(2 * vec), (long long)vec);
  skvd::MergeStatesArgs m{};
  m.o_states = o_states;
  m.o_state_stride = o_state_stride;
  m.o_row_stride = o_row_stride;
  m.lse_states = lse_states;
  m.lse_state_stride = lse_state_stride;
  m.num_states = num_states;
  m.head_dim = head_dim;
  m.rows = rows;
  m.o = o;
  m.lse = lse;
  const int e = skvd::launch_merge_states(m, stream);
  return e ? hip_err(e, "merge-states kernel launch") : SKVD_OK;
}

skvd_status skvd_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  g_err[0] = 0;
  if (!buf || !sink) return set_err(SKVD_ERR_NULL, "buf and sink must be non-NULL");
  if ((uintptr_t)buf % 16 || bytes % 16)
    return set_err(SKVD_ERR_LAYOUT, "buf must be 16-byte aligned and bytes a multiple of 16");
  int e = skvd::launch_stream_read(buf, bytes / 16, sink, stream);
  return e ? hip_err(e, "stream-read kernel launch") : SKVD_OK;
}

}  // extern "C"
