// Host-only planning and validation: no HIP calls in this file.
//
// The plan fixes, from static shape bounds, everything a launch needs: the 64-token partial
// block (1bit-MONSTER/engine issue #115, comment "Closing the remaining half of this issue":
// key_value_capacity = ceil_div(kv_len, 64) * 64), how many blocks one split covers, the
// partial stride (from the capacity at max_kv_len, while the loop bounds stay runtime values
// read from kv_len on the device: the same issue, comments "Deep-context decode failures
// were JIT SGPR exhaustion" and "Residual >2048 fault root-caused and fixed"), the reducer,
// and the exact workspace layout, so that a decode call allocates nothing (llama-cpp-
// turboquant PR #176, problem statement: allocation inside a captured stream fails).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "skvd_internal.h"

namespace skvd {

static skvd_status fail(char *err, size_t n, skvd_status st, const char *fmt, ...) {
  if (err && n) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(err, n, fmt, ap);
    va_end(ap);
  }
  return st;
}

static size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

const char *reducer_name(int r) {
  switch (r) {
    case SKVD_REDUCER_DIRECT: return "direct";
    case SKVD_REDUCER_COOPERATIVE: return "cooperative";
    case SKVD_REDUCER_MULTIPASS: return "multipass";
    case SKVD_REDUCER_HIERARCHICAL: return "hierarchical";
    case SKVD_REDUCER_NONE: return "none";
    default: return "auto";
  }
}

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

skvd_status make_plan(const skvd_plan_params &prm, int num_cus, Plan *out, char *err,
                      size_t errn) {
  const int Hq = prm.num_qo_heads, Hkv = prm.num_kv_heads, D = prm.head_dim;
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0)
    return fail(err, errn, SKVD_ERR_SHAPE, "num_qo_heads=%d must be a positive multiple of "
                "num_kv_heads=%d", Hq, Hkv);
  if (D != 128 && D != 192 && D != 256 && D != 512)
    return fail(err, errn, SKVD_ERR_SHAPE, "head_dim=%d unsupported (128, 192, 256 or 512)", D);
  if (D == 192 && (prm.kv_dtype == SKVD_KV_I8_F16SCALE32 || prm.kv_dtype == SKVD_KV_Q4_0))
    return fail(err, errn, SKVD_ERR_SHAPE, "%s cache at head_dim 192 unsupported (its six "
                "group scales per row are not a whole number of the decode's 8-byte scale loads)",
                prm.kv_dtype == SKVD_KV_Q4_0 ? "q4_0" : "int8");
  if (!is_pow2(prm.page_size) || prm.page_size > 1024)
    return fail(err, errn, SKVD_ERR_SHAPE, "page_size=%d must be a power of two <= 1024",
                prm.page_size);
  if (prm.max_batch > 65535 || Hkv > 65535)
    return fail(err, errn, SKVD_ERR_SHAPE, "max_batch=%d and num_kv_heads=%d must be <= 65535 "
                "(grid dimensions)", prm.max_batch, Hkv);
  if (prm.max_batch < 1 || prm.max_kv_len < 1)
    return fail(err, errn, SKVD_ERR_SHAPE, "max_batch=%d and max_kv_len=%d must be >= 1",
                prm.max_batch, prm.max_kv_len);
  if (prm.max_q_per_seq < 1 || prm.max_q_per_seq > 8)
    return fail(err, errn, SKVD_ERR_SHAPE, "max_q_per_seq=%d must be in 1..8",
                prm.max_q_per_seq);
  const int G = Hq / Hkv;
  const int R = G * prm.max_q_per_seq;
  // Query rows of one KV head: up to 16 per wave (the 16x16 MFMA's rows), up to 4 such waves
  // per workgroup, and row groups of 64 beyond that.
  if (R > 1024)
    return fail(err, errn, SKVD_ERR_SHAPE, "group*max_q_per_seq=%d exceeds 1024 rows", R);
  if (prm.kv_dtype != SKVD_KV_F16 && prm.kv_dtype != SKVD_KV_I8_F16SCALE32 &&
      prm.kv_dtype != SKVD_KV_FP8_E4M3 && prm.kv_dtype != SKVD_KV_Q4_0)
    return fail(err, errn, SKVD_ERR_DTYPE, "kv_dtype=%d unknown", prm.kv_dtype);
  if (num_cus < 1) return fail(err, errn, SKVD_ERR_DEVICE, "num_cus=%d", num_cus);
  if (prm.force_reducer < 0 || prm.force_reducer > SKVD_REDUCER_NONE)
    return fail(err, errn, SKVD_ERR_PLAN, "force_reducer=%d unknown", prm.force_reducer);
  if (prm.force_blocks_per_split < 0)
    return fail(err, errn, SKVD_ERR_PLAN, "force_blocks_per_split=%d",
                prm.force_blocks_per_split);
  if (prm.schedule < SKVD_SCHEDULE_AUTO || prm.schedule > SKVD_SCHEDULE_BALANCED)
    return fail(err, errn, SKVD_ERR_PLAN, "schedule=%d unknown", prm.schedule);
  if (prm.wgs_per_cu < 0 || prm.wgs_per_cu > 64)
    return fail(err, errn, SKVD_ERR_PLAN, "wgs_per_cu=%d outside 0..64", prm.wgs_per_cu);
  // KV heads per workgroup: the single-quarter variants at D=128 come in 1, 2, 4 and 8.
  const bool multi_head_ok = D == 128 && G * prm.max_q_per_seq <= 4;
  int hw = prm.heads_per_wg;
  // A decode with no more (sequence, KV head, block) units than CUs is latency-bound: one
  // head per workgroup spreads it over the most CUs (measured: B=1, 1024 tokens, 12.5 vs 13.8
  // us per call; 8192 tokens prefers 4 heads).
  const int64_t units_all = (int64_t)prm.max_batch * Hkv * ((prm.max_kv_len + 63) / 64);
  if (hw == 0)
    hw = !multi_head_ok || units_all <= num_cus ? 1
         : Hkv % 4 == 0 ? 4
         : Hkv % 2 == 0 ? 2
         : 1;
  if (hw != 1 && (!multi_head_ok || (hw != 2 && hw != 4 && hw != 8) || Hkv % hw != 0))
    return fail(err, errn, SKVD_ERR_PLAN, "heads_per_wg=%d: only 1, or 2 / 4 / 8 dividing Hkv=%d "
                "at head_dim 128 with G*T <= 4", prm.heads_per_wg, Hkv);

  Plan p{};
  p.prm = prm;
  p.group = G;
  p.rows_per_wg = R;
  p.row_blocks = R <= 4 ? 1 : (R <= 8 ? 2 : 4);
  p.row_tiles = R <= kRowTile ? 1 : (R <= 2 * kRowTile ? 2 : 4);
  p.rows_per_group = std::min(R, kRowTile * p.row_tiles);
  p.row_groups = (R + p.rows_per_group - 1) / p.rows_per_group;
  p.num_cus = num_cus;
  p.max_blocks = (prm.max_kv_len + kBlockTokens - 1) / kBlockTokens;
  p.rows_cap = (int64_t)prm.max_batch * prm.max_q_per_seq * Hq;
  p.heads_per_wg = hw;
  p.sched_heads = (Hkv / hw) * p.row_groups;

  // Blocks per split. Two pressures: enough workgroups to fill the chip (about 16 per CU
  // when every sequence is at max_kv_len), and partial traffic (one (m, l, D floats) per row
  // and split, written then read back) at most ~3% of the split's K+V bytes.
  const double row_bytes = prm.kv_dtype == SKVD_KV_F16 ? 4.0 * D
                           : prm.kv_dtype == SKVD_KV_FP8_E4M3 ? 2.0 * D
                           : prm.kv_dtype == SKVD_KV_Q4_0 ? 2.0 * (D / 2 + 2 * (D / 32))
                                                          : 2.0 * (D + 2 * (D / 32));
  const double partial_bytes = 2.0 * R * (D + 2) * 4.0;
  int bps_min = (int)std::ceil(partial_bytes / (0.03 * kBlockTokens * row_bytes));
  if (bps_min < 1) bps_min = 1;
  const int64_t units = (int64_t)prm.max_batch * Hkv * p.max_blocks;
  int64_t bps = units / (16LL * num_cus);
  if (bps < bps_min) bps = bps_min;
  if (bps > 4LL * bps_min) bps = 4LL * bps_min;
  // ... but at least one workgroup per CU when the work allows it: with many query rows per KV
  // head (a large group times a multi-token draft) the traffic rule alone would leave a small
  // batch a handful of workgroups walking whole sequences
  const int64_t bps_fill = std::max<int64_t>(
      1, (int64_t)prm.max_batch * p.sched_heads * p.max_blocks / num_cus);
  if (bps > bps_fill) bps = bps_fill;
  // very short contexts: one split, one launch (up to 128 tokens; beyond, a second launch for
  // the merge costs less than one workgroup walking the chunks: 256 tokens 16.4 vs 12-13 us)
  if (p.max_blocks <= 2) bps = p.max_blocks;
  if (prm.force_blocks_per_split > 0) bps = prm.force_blocks_per_split;
  if (bps > p.max_blocks) bps = p.max_blocks;
  if (bps < 1) bps = 1;
  // The partial kernel's one-dimensional grid holds split_stride x schedule heads x sequences
  // < 2^31 workgroups, split_stride being splits_cap rounded up to odd.
  const int64_t per_split = (int64_t)p.sched_heads * prm.max_batch;
  const int64_t max_splits = INT32_MAX / per_split - 1;
  if (max_splits < 1)
    return fail(err, errn, SKVD_ERR_SHAPE, "schedule heads x max_batch = %lld exceeds the grid",
                (long long)per_split);
  const int64_t bps_grid = (p.max_blocks + max_splits - 1) / max_splits;
  if (bps < bps_grid) {
    if (prm.force_blocks_per_split > 0)
      return fail(err, errn, SKVD_ERR_PLAN, "force_blocks_per_split=%d gives more than 2^31 "
                  "partial workgroups", prm.force_blocks_per_split);
    bps = bps_grid;
  }
  p.bps = (int)bps;
  p.splits_cap = (p.max_blocks + p.bps - 1) / p.bps;

  // Schedule. Static: workgroups are (split, KV head, sequence) at fixed block offsets, so a
  // ragged batch leaves some compute units with more work than others once the grid fits the
  // chip in one round. Balanced: equal shares of the blocks actually present, cut on the device
  // from kv_len (up to 16 sequences per lane of one wave, hence the batch limit); partials go to
  // compact slots,
  // one per (schedule row, share) pair that meet — at most rows + shares — so the workspace does
  // not grow with the context and shares can be as small as one block.
  int sched = prm.schedule;
  // (the device cuts the shares in 32-bit arithmetic: the batch's blocks times the schedule
  // heads below 2^31, and the grid's square below 2^30, num_cus <= 512 at 64 per CU)
  const bool can_balance = p.splits_cap > 1 && prm.max_batch <= kBalancedMaxBatch &&
                           prm.force_reducer != SKVD_REDUCER_NONE &&
                           (int64_t)prm.max_batch * p.sched_heads * p.max_blocks < INT32_MAX &&
                           num_cus <= 512;
  if (sched == SKVD_SCHEDULE_AUTO)
    sched = can_balance ? SKVD_SCHEDULE_BALANCED : SKVD_SCHEDULE_STATIC;
  if (sched == SKVD_SCHEDULE_BALANCED && !can_balance)
    return fail(err, errn, SKVD_ERR_PLAN, "balanced schedule needs more than one split, "
                "max_batch <= %d, a reducer, max_batch x schedule heads x blocks < 2^31 and "
                "num_cus <= 512 (plan: %d splits, max_batch %d)",
                kBalancedMaxBatch, p.splits_cap, prm.max_batch);
  p.schedule = sched;
  if (sched == SKVD_SCHEDULE_BALANCED) {
    // Workgroups per CU (measured on MI355X): one wave per SIMD saturates the memory pipes of
    // an f16 stream, best as one workgroup of 4 KV heads reading each token row's heads
    // together. The one-byte formats widen every element on the vector ALU and do best with
    // three waves per SIMD, as three workgroups of 4 KV heads: fp8 on the GQA batch 44.6
    // us/call against 46.4 with 8 heads x 1 and 45.1 with 4 x 2, on the int8 batch's shape
    // 521.9 against 530.5 and 530.2; int8 on the int8 batch with head-major scale pools
    // (each head's scales of a page contiguous, so a 16-token tile's scales are one 128-byte
    // line) 560.7 us against 586.6 with 8 heads x 1, 592.7 with 8 x 2 (two rounds), 585.1 with
    // 4 x 2 and 580.8 with 2 x 6 (token-major scale pools: 617 with 4 x 3, whose twelve waves
    // per CU each touch 32 lines for a chunk's 256 bytes of scales).
    const bool byte = prm.kv_dtype != SKVD_KV_F16;
    // D = 256 f16 variants hold one wave per SIMD (over 256 registers with the accumulators)
    // and, a pure stream, do best with three workgroups per CU (the wide multi-token workload
    // 527 us against 537 with four; with two waves per SIMD no faster at three, slower at six or
    // eight). The one-byte formats at D = 192 / 256 widen every element and run two waves per
    // SIMD: eight workgroups per CU (on the wide multi-token workload's shape, against four
    // workgroups of one wave: int8 408 -> 290-300 us, fp8 377 -> 244-255, q4_0 393 -> 240-254).
    // head_dim 192 takes head_dim 256's counts; 512 holds one wave per SIMD: four for the
    // one-byte formats.
    const int auto_wpc = D != 128 ? (!byte ? 3 : D <= 256 ? 8 : 4)
                         : p.row_blocks == 1 ? (byte ? std::max(1, 12 / hw)
                                                     : std::max(1, kDefaultWgsPerCu / hw))
                                             : kDefaultWgsPerCu;
    // several row-tile waves per workgroup (more than 16 query rows per KV head): the same
    // waves per CU as one-wave workgroups
    const int auto_wgs = std::max(1, auto_wpc / p.row_tiles);
    p.grid_wgs = (prm.wgs_per_cu ? prm.wgs_per_cu : auto_wgs) * num_cus;
    // a forced split size becomes the balanced shares' minimum
    p.piece_min = prm.force_blocks_per_split > 0 ? p.bps : 1;
    const int64_t per_row = std::min<int64_t>(p.grid_wgs,
                                              (p.max_blocks + p.piece_min - 1) / p.piece_min + 1);
    p.part_stride = (int)per_row;
    p.slots_cap = (int64_t)prm.max_batch * p.sched_heads + p.grid_wgs;
  } else {
    p.part_stride = p.splits_cap;
    p.piece_min = p.bps;
    p.slots_cap = 0;
    p.grid_wgs = (int)((int64_t)(p.splits_cap | 1) * per_split);
  }

  // Reducer: total over every partial count.
  int red = prm.force_reducer;
  if (red == SKVD_REDUCER_AUTO) {
    if (p.part_stride == 1) red = SKVD_REDUCER_NONE;
    else if (p.part_stride <= 4) red = SKVD_REDUCER_DIRECT;
    else if (p.part_stride <= 64) red = SKVD_REDUCER_COOPERATIVE;
    // hierarchical only pays for its second launch when few rows hold very many partials
    else if (p.part_stride <= 1024 || p.rows_cap >= 2LL * num_cus) red = SKVD_REDUCER_MULTIPASS;
    else red = SKVD_REDUCER_HIERARCHICAL;
  }
  if (red == SKVD_REDUCER_NONE && p.part_stride != 1)
    return fail(err, errn, SKVD_ERR_PLAN, "reducer none needs one split, plan has %d",
                p.part_stride);
  if (red == SKVD_REDUCER_COOPERATIVE && p.part_stride > 64)
    return fail(err, errn, SKVD_ERR_PLAN, "cooperative reducer covers at most 64 partials, "
                "plan has %d", p.part_stride);
  p.reducer = red;
  p.hier_groups_cap = red == SKVD_REDUCER_HIERARCHICAL
                          ? (p.part_stride + kHierGroup - 1) / kHierGroup : 0;

  // Workspace: status word, then partials (and hierarchical intermediates).
  size_t off = 0;
  p.off_status = off;
  off = align_up(off + sizeof(uint32_t));
  const size_t parts = red == SKVD_REDUCER_NONE ? 0
                       : sched == SKVD_SCHEDULE_BALANCED
                           ? (size_t)p.slots_cap * hw * p.rows_per_group
                           : (size_t)p.rows_cap * p.part_stride;
  p.off_ml = off;
  off = align_up(off + parts * 2 * sizeof(float));
  p.off_o = off;
  off = align_up(off + parts * (size_t)D * sizeof(float));
  const size_t hparts = (size_t)p.rows_cap * p.hier_groups_cap;
  p.off_hml = off;
  off = align_up(off + hparts * 2 * sizeof(float));
  p.off_ho = off;
  off = align_up(off + hparts * (size_t)D * sizeof(float));
  p.ws_bytes = off;
  *out = p;
  return SKVD_OK;
}

static bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

skvd_status check_args(const Plan &p, const skvd_decode_args *a, size_t ws_bytes, char *err,
                       size_t errn) {
  if (!a) return fail(err, errn, SKVD_ERR_NULL, "args is NULL");
  const int D = p.prm.head_dim;
  const bool q4 = p.prm.kv_dtype == SKVD_KV_Q4_0;
  const bool i8 = p.prm.kv_dtype == SKVD_KV_I8_F16SCALE32 || q4;  // f16 scales per 32 elements
  const bool f8 = p.prm.kv_dtype == SKVD_KV_FP8_E4M3;
  const bool byte = i8 || f8;  // pools addressed in bytes
  const char *fmt = q4 ? "q4_0" : i8 ? "int8" : "fp8";
  if (a->reserved != 0) return fail(err, errn, SKVD_ERR_SHAPE, "reserved must be 0");
  if (a->batch < 0 || a->batch > p.prm.max_batch)
    return fail(err, errn, SKVD_ERR_SHAPE, "batch=%d outside 0..max_batch=%d", a->batch,
                p.prm.max_batch);
  if (a->q_per_seq < 1 || a->q_per_seq > p.prm.max_q_per_seq)
    return fail(err, errn, SKVD_ERR_SHAPE, "q_per_seq=%d outside 1..max_q_per_seq=%d",
                a->q_per_seq, p.prm.max_q_per_seq);
  if (!a->q || !a->k_pages || !a->v_pages || !a->page_table || !a->kv_len || !a->o)
    return fail(err, errn, SKVD_ERR_NULL, "q, k_pages, v_pages, page_table, kv_len and o "
                "must be non-NULL");
  if (byte && (!a->k_scales || !a->v_scales))
    return fail(err, errn, SKVD_ERR_DTYPE, "%s cache needs k_scales and v_scales", fmt);
  if (!byte && (a->k_scales || a->v_scales))
    return fail(err, errn, SKVD_ERR_DTYPE, "f16 cache takes no scales");
  if (f8 && (!aligned(a->k_scales, 4) || !aligned(a->v_scales, 4)))
    return fail(err, errn, SKVD_ERR_LAYOUT, "fp8 k_scale / v_scale must be 4-byte aligned");
  if (!std::isfinite(a->sm_scale))
    return fail(err, errn, SKVD_ERR_SHAPE, "sm_scale is not finite");
  // Vector loads: 16 bytes of q, o, K and f16 V rows; 8 bytes of int8 / fp8 V rows, 4 of
  // q4_0's.
  const int64_t kv_vec = byte ? 16 : 8;  // elements per 16-byte load
  if (!aligned(a->q, 16) || a->q_tok_stride % 8 || a->q_head_stride % 8 || a->q_tok_stride < 0 ||
      a->q_head_stride < 0)
    return fail(err, errn, SKVD_ERR_LAYOUT, "q must be 16-byte aligned with token/head "
                "strides that are non-negative multiples of 8 elements");
  if (!aligned(a->k_pages, 16) || !aligned(a->v_pages, 16) ||
      a->page_stride % kv_vec || a->tok_stride % kv_vec || a->head_stride % kv_vec ||
      a->page_stride < 0 || a->tok_stride < 0 || a->head_stride < 0)
    return fail(err, errn, SKVD_ERR_LAYOUT, "K/V pools must be 16-byte aligned and have "
                "page/token/head strides that are non-negative multiples of 16 bytes "
                "(head_dim dense, same strides for K and V)");
  // Scales: the D/32 scales of one token-head are read with 8-byte loads.
  if (i8 && (!aligned(a->k_scales, 8) || !aligned(a->v_scales, 8) || a->scale_page_stride < 0 ||
             a->scale_tok_stride < 0 || a->scale_head_stride < 0 || a->scale_page_stride % 4 ||
             a->scale_tok_stride % 4 || a->scale_head_stride % 4))
    return fail(err, errn, SKVD_ERR_LAYOUT, "scale pools must be 8-byte aligned with "
                "non-negative strides that are multiples of 4 elements");
  // Within a 16-token tile the kernels address rows with 32-bit byte offsets.
  const int64_t es = byte ? 1 : 2, row = q4 ? D / 2 : D;
  if ((16 * a->tok_stride + row) * es >= (int64_t(1) << 31) ||
      (i8 && 16 * a->scale_tok_stride + D / 32 >= (int64_t(1) << 30)))
    return fail(err, errn, SKVD_ERR_LAYOUT, "token stride too large for 32-bit in-tile offsets");
  if (a->num_k_pages < 1 || a->num_v_pages < 1)
    return fail(err, errn, SKVD_ERR_SHAPE, "num_k_pages and num_v_pages must be >= 1");
  const int64_t need_pages = (p.prm.max_kv_len + p.prm.page_size - 1) / p.prm.page_size;
  if (a->table_stride < need_pages)
    return fail(err, errn, SKVD_ERR_LAYOUT, "table_stride=%lld below ceil(max_kv_len/P)=%lld",
                (long long)a->table_stride, (long long)need_pages);
  if (!aligned(a->o, 16)) return fail(err, errn, SKVD_ERR_LAYOUT, "o must be 16-byte aligned");
  if (a->lse && !aligned(a->lse, 4))
    return fail(err, errn, SKVD_ERR_LAYOUT, "lse must be 4-byte aligned");
  if (ws_bytes < p.ws_bytes)
    return fail(err, errn, SKVD_ERR_WORKSPACE, "workspace of %zu bytes below the plan's %zu",
                ws_bytes, p.ws_bytes);
  return SKVD_OK;
}

void fill_launch_args(const Plan &p, const skvd_decode_args &a, void *ws, LaunchArgs *la) {
  LaunchArgs l{};
  l.q = a.q;
  l.q_tok_stride = a.q_tok_stride;
  l.q_head_stride = a.q_head_stride;
  l.k = a.k_pages;
  l.v = a.v_pages;
  l.page_stride = a.page_stride;
  l.tok_stride = a.tok_stride;
  l.head_stride = a.head_stride;
  l.num_k_pages = a.num_k_pages;
  l.num_v_pages = a.num_v_pages;
  l.ks = a.k_scales;
  l.vs = a.v_scales;
  l.s_page_stride = a.scale_page_stride;
  l.s_tok_stride = a.scale_tok_stride;
  l.s_head_stride = a.scale_head_stride;
  l.table = a.page_table;
  l.table_stride = a.table_stride;
  l.kv_len = a.kv_len;
  l.batch = a.batch;
  l.T = a.q_per_seq;
  l.Hq = p.prm.num_qo_heads;
  l.Hkv = p.prm.num_kv_heads;
  l.G = p.group;
  l.D = p.prm.head_dim;
  int sh = 0;
  while ((1 << sh) < p.prm.page_size) ++sh;
  l.page_shift = sh;
  l.scale_log2 = a.sm_scale * 1.4426950408889634f;
  l.bps = p.bps;
  l.splits_cap = p.splits_cap;
  l.split_stride = p.splits_cap | 1;
  l.balanced = p.schedule == SKVD_SCHEDULE_BALANCED;
  l.grid_wgs = p.grid_wgs;
  l.heads_per_wg = p.heads_per_wg;
  l.row_tiles = p.row_tiles;
  l.row_groups = p.row_groups;
  l.rows_per_group = p.rows_per_group;
  l.sched_heads = p.sched_heads;
  l.seqs_per_lane = std::max(1, (a.batch + 63) / 64);
  l.part_stride = p.part_stride;
  l.piece_min = p.piece_min;
  l.max_kv_len = p.prm.max_kv_len;
  l.hier_groups_cap = p.hier_groups_cap;
  l.int8 = p.prm.kv_dtype != SKVD_KV_F16;  // elements of at most one byte
  l.fp8 = p.prm.kv_dtype == SKVD_KV_FP8_E4M3;
  l.q4 = p.prm.kv_dtype == SKVD_KV_Q4_0;
  l.debug = p.prm.debug;
  char *w = (char *)ws;
  l.status = w ? (unsigned *)(w + p.off_status) : nullptr;
  l.ws_ml = w ? (float *)(w + p.off_ml) : nullptr;
  l.ws_o = w ? (float *)(w + p.off_o) : nullptr;
  l.ws_hml = w ? (float *)(w + p.off_hml) : nullptr;
  l.ws_ho = w ? (float *)(w + p.off_ho) : nullptr;
  l.o = a.o;
  l.lse = a.lse;
  l.single = p.reducer == SKVD_REDUCER_NONE;
  *la = l;
}

}  // namespace skvd
