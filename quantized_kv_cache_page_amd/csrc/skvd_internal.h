// Internal declarations shared by the host runtime (plan, validation, launch sequencing)
// and the HIP kernels. Not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/skvd.h"

namespace skvd {

constexpr int kBlockTokens = 64;  // one partial block: 64 consecutive KV positions
constexpr int kHierGroup = 64;    // partials merged by one first-level hierarchical workgroup
constexpr size_t kAlign = 256;
constexpr int kBalancedMaxBatch = 1024;  // balanced schedule: up to 16 sequences per lane of a wave
constexpr int kRowTile = 16;             // query rows of one wave (the 16x16 MFMA's rows)
constexpr int kDefaultWgsPerCu = 4;

struct Plan {
  skvd_plan_params prm;
  int group;          // G = Hq / Hkv
  int rows_per_wg;    // R = G * max_q_per_seq: query rows of one KV head
  int row_blocks;     // 16x16 MFMA row quarters in use per wave (1, 2 or 4; 4 when R > 16)
  int row_tiles;      // RT: waves per KV head in a workgroup, 16 rows each (1, 2 or 4)
  int row_groups;     // NRG = ceil(R / (16 RT)): workgroups per KV head (rows 16 RT each)
  int rows_per_group; // RPG = min(R, 16 RT): query rows one schedule head covers
  int sched_heads;    // Hg = (Hkv / heads_per_wg) * row_groups: schedule heads per sequence
  int num_cus;
  int max_blocks;     // ceil(max_kv_len / 64)
  int bps;            // 64-token blocks per split
  int splits_cap;     // ceil(max_blocks / bps): static splits per row at max_kv_len
  int schedule;       // resolved skvd_schedule
  int part_stride;    // partials per output row at most: static splits_cap (the row's slot
                      // stride); balanced min(grid, max_blocks / piece_min + 1)
  int piece_min;      // balanced: fewest 64-token blocks in a share
  int64_t slots_cap;  // balanced: compact slots (schedule rows + shares)
  int grid_wgs;       // partial-kernel grid (static: split_stride * Hkv / hw * max_batch)
  int heads_per_wg;   // hw: KV heads served by one workgroup, one wave each
  int reducer;        // resolved skvd_reducer
  int hier_groups_cap;
  int64_t rows_cap;
  size_t off_status, off_ml, off_o, off_hml, off_ho, ws_bytes;
};

// Everything a kernel launch needs, resolved on the host from the plan and the args.
struct LaunchArgs {
  const void *q;
  int64_t q_tok_stride, q_head_stride;
  const void *k, *v;
  int64_t page_stride, tok_stride, head_stride;
  int64_t num_k_pages, num_v_pages;
  const void *ks, *vs;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  const int32_t *kv_len;
  int batch, T, Hq, Hkv, G, D, page_shift;
  float scale_log2;  // sm_scale * log2(e): scores are kept in base 2
  int bps, splits_cap, split_stride, max_kv_len, hier_groups_cap;  // stride: odd, >= cap
  int balanced, grid_wgs, part_stride, piece_min;
  int heads_per_wg;  // KV heads (waves) per partial-kernel workgroup; divides Hkv
  int row_tiles, row_groups, rows_per_group, sched_heads;  // as in Plan
  int seqs_per_lane;  // balanced schedule: sequences per lane of the share computation
  int int8;         // elements of at most one byte (int8, fp8 or q4_0)
  int fp8;          // fp8 E4M3: ks / vs each point to one f32 tensor scale
  int q4;           // q4_0: rows of D/2 bytes, f16 scales per 32 elements
  int debug;
  // partials (static: [rows_cap][part_stride]; balanced: [slots][heads_per_wg][G*T]):
  float *ws_ml;      // [..][2]  (max in log2 units, sum)
  float *ws_o;       // [..][D]  unnormalized f32 output
  float *ws_hml;     // [rows_cap][hier_groups_cap][2]
  float *ws_ho;      // [rows_cap][hier_groups_cap][D]
  unsigned *status;
  void *o;
  float *lse;
  int single;        // the partial kernel writes o/lse (reducer NONE)
  // gather-debug launches only (the partial kernel's debug variant): raw K/V elements and
  // int8 scales as the kernel holds them at their point of use, into dense
  // [B, dbg_max_len, Hkv, D] / [B, dbg_max_len, Hkv, D/32] arrays
  char *dbg_k, *dbg_v;
  uint16_t *dbg_ks, *dbg_vs;  // f16 bits
  int dbg_max_len;
};

// plan.cpp (pure host)
skvd_status make_plan(const skvd_plan_params &prm, int num_cus, Plan *out, char *err, size_t errn);
skvd_status check_args(const Plan &p, const skvd_decode_args *a, size_t ws_bytes, char *err,
                       size_t errn);
const char *reducer_name(int r);
void fill_launch_args(const Plan &p, const skvd_decode_args &a, void *ws, LaunchArgs *la);

// kernels.hip (return a hipError_t as int; 0 = success)
// start_event/stop_event: NULL, or hipEvent_t that the partial kernel's dispatch stamps with its
// begin and end (hipExtLaunchKernel).
int launch_partial(const Plan &p, const LaunchArgs &la, void *stream, void *start_event = nullptr,
                   void *stop_event = nullptr);
int launch_merge(const Plan &p, const LaunchArgs &la, void *stream);
int launch_stream_read(const void *buf, size_t n16, uint32_t *sink, void *stream);
// The partial kernel's debug variant (the plan's own schedule and lane layout) writing the raw
// K/V rows and int8 scales it uses into la.dbg_* instead of any partial or output.
int launch_gather(const Plan &p, const LaunchArgs &la, void *stream);

// Per-format partial launchers (partial_<D>_<fmt>.hip), dispatched by launch_partial.
struct KernelEvents {
  void *start = nullptr, *stop = nullptr;  // hipEvent_t stamped by the dispatch, or NULL
};
#define SKVD_DECLARE_PARTIAL(D, KV)                                                            \
  int launch_partial_##D##_##KV(const Plan &p, const LaunchArgs &la, unsigned grid,            \
                                void *stream, const KernelEvents &ev, bool dbg);
SKVD_DECLARE_PARTIAL(128, 0)
SKVD_DECLARE_PARTIAL(128, 1)
SKVD_DECLARE_PARTIAL(128, 2)
SKVD_DECLARE_PARTIAL(128, 3)
SKVD_DECLARE_PARTIAL(256, 0)
SKVD_DECLARE_PARTIAL(256, 1)
SKVD_DECLARE_PARTIAL(256, 2)
SKVD_DECLARE_PARTIAL(256, 3)
SKVD_DECLARE_PARTIAL(192, 0)
SKVD_DECLARE_PARTIAL(192, 2)
SKVD_DECLARE_PARTIAL(512, 0)
SKVD_DECLARE_PARTIAL(512, 1)
SKVD_DECLARE_PARTIAL(512, 2)
SKVD_DECLARE_PARTIAL(512, 3)
#undef SKVD_DECLARE_PARTIAL

// Append launch (append.hip): resolved on the host from the plan and skvd_append_args.
struct AppendLaunch {
  const void *k_new, *v_new;
  int64_t new_tok_stride, new_head_stride;
  const int32_t *batch_idx, *positions;
  void *k, *v;
  int64_t page_stride, tok_stride, head_stride;
  int64_t num_k_pages, num_v_pages;
  void *ks, *vs;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  int64_t rows;        // num_tokens * Hkv
  int num_tokens, batch, Hkv, D, page_shift, max_len, int8;
  int fp8;              // fp8 E4M3 cache: ks / vs each point to one f32 tensor scale
  int q4;               // q4_0 cache: rows of D/2 code bytes, f16 scales per 32 elements
  int num_cus;          // compute units of the plan's device
  int lanes_per_token;  // set by launch_append: Hkv * D / 8 (one lane per 8 elements of a row)
  int tok_step;         // set by launch_append: tokens the whole grid covers per step
  unsigned blocks;      // set by launch_append: 256-lane workgroups launched
};

// prefill.hip: the multi-token route (T > 8) over the decode's LaunchArgs (f16, int8 or fp8
// cache); no workspace.
int launch_prefill(const LaunchArgs &la, void *stream);

// cascade.hip: merge of attention states (validated in api.cpp)
struct MergeStatesArgs {
  const void *o_states;  // f16, state s row r at s * o_state_stride + r * o_row_stride
  int64_t o_state_stride, o_row_stride;
  const float *lse_states;  // state s row r at s * lse_state_stride + r
  int64_t lse_state_stride;
  int num_states, head_dim;
  int64_t rows;
  void *o;     // f16 [rows, head_dim] dense
  float *lse;  // [rows] or NULL
};
int launch_merge_states(const MergeStatesArgs &a, void *stream);

// append.hip
constexpr int kAppendTokensPerLane = 4;  // tokens one append lane serves per round
int launch_append(AppendLaunch a, void *stream);

}  // namespace skvd
