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

skvd_status common_checks(const skvd_plan *plan, const skvd_decode_args *args, void *ws,
                          size_t ws_bytes) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  skvd_status st = skvd::check_args(plan->p, args, ws_bytes, g_err, sizeof g_err);
  if (st != SKVD_OK) return st;
  if (!ws) return set_err(SKVD_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws % skvd::kAlign)
    return set_err(SKVD_ERR_WORKSPACE, "workspace must be %zu-byte aligned", skvd::kAlign);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(SKVD_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev != plan->p.prm.device)
    return set_err(SKVD_ERR_DEVICE, "current device %d is not the plan's device %d", dev,
                   plan->p.prm.device);
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
  snprintf(buf, n,
           "plan Hq=%d Hkv=%d D=%d P=%d kv=%s max_batch=%d max_T=%d max_kv_len=%d cus=%d: "
           "blocks_per_split=%d splits=%d schedule=%s grid=%d heads_per_wg=%d reducer=%s "
           "hier_groups=%d rows_per_wg=%d workspace=%zu B",
           p.prm.num_qo_heads, p.prm.num_kv_heads, p.prm.head_dim, p.prm.page_size,
           p.prm.kv_dtype == SKVD_KV_F16 ? "f16" : "int8", p.prm.max_batch, p.prm.max_q_per_seq,
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

skvd_status skvd_gather_debug(const skvd_plan *plan, const skvd_decode_args *args,
                              int32_t max_len, void *dense_k, void *dense_v, void *dense_ks,
                              void *dense_vs, void *stream) {
  g_err[0] = 0;
  if (!plan) return set_err(SKVD_ERR_NULL, "plan is NULL");
  skvd_status st = skvd::check_args(plan->p, args, plan->p.ws_bytes, g_err, sizeof g_err);
  if (st != SKVD_OK) return st;
  const bool i8 = plan->p.prm.kv_dtype == SKVD_KV_I8_F16SCALE32;
  if (!dense_k || !dense_v || (i8 && (!dense_ks || !dense_vs)))
    return set_err(SKVD_ERR_NULL, "dense outputs must be non-NULL");
  if (max_len < 0 || max_len > plan->p.prm.max_kv_len)
    return set_err(SKVD_ERR_SHAPE, "max_len=%d outside 0..max_kv_len", max_len);
  if (((uintptr_t)dense_k | (uintptr_t)dense_v) % 4)
    return set_err(SKVD_ERR_LAYOUT, "dense_k and dense_v must be 4-byte aligned");
  skvd::LaunchArgs la;
  skvd::fill_launch_args(plan->p, *args, nullptr, &la);
  la.debug = 0;
  int e = skvd::launch_gather(plan->p, la, max_len, dense_k, dense_v, dense_ks, dense_vs, stream);
  return e ? hip_err(e, "gather kernel launch") : SKVD_OK;
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
