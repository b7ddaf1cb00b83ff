/*
 * skvd.h - split-KV paged decode attention for MI355X (gfx950): the C ABI.
 *
 * What the library computes
 * -------------------------
 * Batch decode attention over a paged KV cache. Each sequence b has T query tokens (T <= 8)
 * and kv_len[b] cached positions held in pages of P tokens; query head h reads KV head
 * h / G (G = Hq / Hkv). For query token t of sequence b the visible positions are
 * j < kv_len[b] - T + t + 1 (the T query tokens are the last T cached positions, so T = 1
 * sees all of kv_len[b]); the result is
 *     o   = softmax(sm_scale * q K^T) V          (f16, dense [B*T, Hq, D])
 *     lse = ln sum_j exp(sm_scale * q . k_j)     (f32, [B*T, Hq]; natural log)
 * A row that sees no position gets o = 0 and lse = -inf.
 *
 * The method is the split-KV decode of 1bit-MONSTER/engine issue #115 ("HRX:
 * flash-attention decode-split template resolution fails ("all_rejected") at longer
 * context"): the KV length is cut into 64-token blocks (key_value_capacity is kv_len rounded
 * up to a multiple of 64, comment "Closing the remaining half of this issue"), each run of
 * blocks yields an online-softmax partial (running max, sum and f32 output), and the
 * partials are merged by a log-sum-exp reduction. The reducers here are direct,
 * cooperative (one lane per partial), multipass (lane-strided, any count) and hierarchical
 * (two levels); no capacity ceiling exists at 32 blocks / 2048 tokens or anywhere else.
 *
 * The call follows the statement of a read-only decode op in AMD-Ecosystem/flashinfer PR
 * #397 ("Stop declaring the paged KV cache mutated on read-only attention ops", sections
 * "Summary" and "What changed"): it takes q, separate K and V page pools that share page
 * shape and strides (their page counts may differ; only pages named by the table are read),
 * a page table and per-sequence lengths, and writes only o and lse, densely. The int8 cache
 * (one f16 scale per 32 contiguous head_dim elements, value = int8 * scale) is dequantized
 * inline with no f16 temporary, as the graph-safe VEC decode path of llama-cpp-turboquant
 * PR #176 ("HIP: fix turbo KV decode crash under graph capture; batch-aware VEC/TILE FA
 * routing", section "Changes") does; that PR's routing threshold (Q->ne[1] <= 8) is why this
 * decode call accepts at most 8 query tokens per sequence.
 *
 * Besides the decode, the library holds the operations around it on the same cache: the
 * multi-token route (skvd_prefill: any number of query tokens, MFMA tiles), the append that
 * writes new tokens into the pages (skvd_append: int8 quantized on write), and the merge of
 * attention states over disjoint key sets (skvd_merge_states: cascade / shared prefix). Each is
 * declared below with the passage that defines it.
 *
 * Conventions
 * -----------
 * - Ownership: every pointer in skvd_decode_args is caller-owned device memory on the plan's
 *   device. The library keeps none of them after a call returns. A plan is a host object;
 *   the workspace is caller-provided device memory of skvd_plan_workspace_bytes() bytes,
 *   256-byte aligned, used by one call at a time (one plan per stream at a time).
 * - Const-correctness is the declaration: q, both pools, both scale pools, the table and
 *   kv_len are read only. skvd_decode writes o, lse and the workspace, nothing else.
 * - Graph capture: skvd_decode performs no allocation, no synchronization and no device-to-
 *   host read; kernels read kv_len on the device. It may be called inside hipStreamBegin-
 *   Capture, including as the first call of a plan. Plans are created outside capture.
 * - Errors: every call returns a status. Host-checkable faults (shapes, dtypes, strides,
 *   alignment, batch above the plan, workspace too small) are reported before anything is
 *   launched. A launch failure returns SKVD_ERR_HIP after reading and clearing the HIP
 *   error. skvd_last_error() gives a thread-local message. No exception or abort crosses
 *   the ABI.
 * - Device-data contracts (page ids in range, q_per_seq <= kv_len[b] <= max_kv_len) are not
 *   checked with a synchronization: kernels clamp page ids into [0, num_pages) and kv_len
 *   into [0, max_kv_len], so a violation cannot read or write out of range; plans made with
 *   debug != 0 also set bits in the workspace status word (skvd_plan_info.status_offset).
 * - Strides are in elements of the array they index. head_dim is dense (stride 1).
 */
#ifndef SKVD_H
#define SKVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKVD_ABI_VERSION 11

typedef enum {
  SKVD_OK = 0,
  SKVD_ERR_NULL = 1,        /* a required pointer is NULL */
  SKVD_ERR_SHAPE = 2,       /* a size is out of range or inconsistent with the plan */
  SKVD_ERR_LAYOUT = 3,      /* a stride or alignment the kernels cannot address */
  SKVD_ERR_DTYPE = 4,       /* unknown kv_dtype, or scales present/absent against it */
  SKVD_ERR_WORKSPACE = 5,   /* workspace missing, too small or misaligned */
  SKVD_ERR_DEVICE = 6,      /* device query failed or the current device is not the plan's */
  SKVD_ERR_PLAN = 7,        /* invalid plan parameters (e.g. a forced reducer that cannot
                               cover the plan's partial count) */
  SKVD_ERR_HIP = 8          /* a HIP call or launch failed; detail in skvd_last_error() */
} skvd_status;

typedef enum {
  SKVD_KV_F16 = 0,           /* K/V pools hold f16 */
  SKVD_KV_I8_F16SCALE32 = 1, /* K/V pools hold int8; scale pools hold one f16 per 32 elements */
  SKVD_KV_FP8_E4M3 = 2,      /* K/V pools hold OCP E4M3 bytes (exponent bias 7, no infinities,
                                0x7F / 0xFF NaN); each pool has one f32 scale for the whole
                                tensor: element value = e4m3(byte) * k_scale for K and
                                * v_scale for V (AMD-Ecosystem/flashinfer PR #397, the two
                                commit messages: fp8 caches are read with per-tensor k_scale
                                and v_scale values passed by pointer). Decode, multi-token
                                route, gather and append (nearest-even E4M3 of x / scale,
                                saturating at 448). */
  SKVD_KV_Q4_0 = 3           /* q4_0 (named beside q8_0 among the KV cache types of
                                1bit-MONSTER/engine issue #115, comment "Closing the remaining
                                half of this issue"; read as the published ggml q4_0 block):
                                K/V pools hold uint8 rows of D/2 bytes, two 4-bit codes c per
                                byte -- in each group of 32 elements (bytes 16k .. 16k+15 of a
                                row for group k), byte i holds element i in its low nibble and
                                element i + 16 in its high nibble --, scale pools one f16 d per
                                32 elements laid out as int8's: value = (c - 8) * d. Pool
                                strides are in bytes. head_dim 128, 256 or 512; decode, gather
                                and append (see skvd_append); the multi-token route at head_dim
                                128 and 256. */
} skvd_kv_dtype;

typedef enum {
  SKVD_REDUCER_AUTO = 0,
  SKVD_REDUCER_DIRECT = 1,       /* one wave per row walks the partials serially */
  SKVD_REDUCER_COOPERATIVE = 2,  /* one lane per partial (at most 64 partials) */
  SKVD_REDUCER_MULTIPASS = 3,    /* lane-strided over any count (one wave when <= 64) */
  SKVD_REDUCER_HIERARCHICAL = 4, /* groups of 64 partials per workgroup, then a second merge */
  SKVD_REDUCER_NONE = 5          /* one split: the partial kernel writes o and lse itself */
} skvd_reducer;

/* How the partial kernel's workgroups divide the batch's 64-token blocks. */
typedef enum {
  SKVD_SCHEDULE_AUTO = 0,     /* balanced where it is allowed (below), else static */
  SKVD_SCHEDULE_STATIC = 1,   /* one workgroup per (split of blocks_per_split blocks, KV head,
                                 sequence); splits past a sequence's length exit at once */
  SKVD_SCHEDULE_BALANCED = 2  /* the launch's blocks, in (sequence, KV head, block) order, cut
                                 on the device into W equal contiguous shares, W = min(grid,
                                 blocks / blocks_per_split); a share may cover parts of several
                                 (sequence, KV head) rows and writes one partial per part.
                                 Needs max_batch <= 1024, more than one split, a reducer,
                                 max_batch * schedule heads * blocks per sequence < 2^31 and
                                 num_cus <= 512 (the device cuts the shares in 32-bit
                                 arithmetic). */
} skvd_schedule;

/* Static shape of a plan. All sizes are upper bounds of what skvd_decode may be given. */
typedef struct {
  int32_t num_qo_heads;   /* Hq; Hq % Hkv == 0 */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;       /* D: 128, 192, 256 or 512 (int8 and q4_0 caches: 128, 256 or 512;
                             the multi-token route: 128 or 256) */
  int32_t page_size;      /* P: power of two, 1..1024 */
  int32_t max_batch;      /* B upper bound, >= 1 */
  int32_t max_q_per_seq;  /* T upper bound: 1..8 (G * T <= 1024 query rows per KV head: up to 16
                             per wave, up to 4 waves of one KV head per workgroup, and groups of
                             64 rows beyond that) */
  int32_t max_kv_len;     /* kv_len upper bound, >= 1 */
  int32_t kv_dtype;       /* skvd_kv_dtype */
  int32_t device;         /* HIP device ordinal the calls run on */
  int32_t num_cus;        /* 0: query the device; > 0: plan for this many compute units
                             without touching HIP (host-only planning) */
  int32_t force_blocks_per_split; /* 0: heuristic; > 0: 64-token blocks per split */
  int32_t force_reducer;  /* skvd_reducer; 0 = choose by partial count */
  int32_t debug;          /* != 0: kernels record contract violations in the status word */
  int32_t schedule;       /* skvd_schedule; 0 = auto */
  int32_t wgs_per_cu;     /* balanced schedule: workgroups launched per compute unit (0: at
                             head_dim 128 with G*T <= 4, f16 max(1, 4 / heads_per_wg) and the
                             one-byte formats max(1, 12 / heads_per_wg); other head_dims, f16 3
                             and one-byte 8 (head_dim 192, 256) or 4 (512); 4 for more query
                             rows at head_dim 128; divided by the row tiles of a workgroup);
                             1..64 */
  int32_t heads_per_wg;   /* KV heads one partial-kernel workgroup serves, one wave each
                             (0 at head_dim 128 with G*T <= 4: 4, else 2, else 1 -- whichever
                             divides Hkv --, where the waves of a CU read each token's rows of
                             those heads together; 1 otherwise, and 1 when the plan has no more
                             (sequence, KV head, block) units than CUs). Values 2, 4, 8 only
                             for that variant and must divide Hkv (else SKVD_ERR_PLAN). */
} skvd_plan_params;

/* What a plan resolved to (for logs and tests). */
typedef struct {
  int32_t blocks_per_split; /* 64-token blocks each split covers */
  int32_t splits_cap;       /* partials per row at max_kv_len (partial stride) */
  int32_t reducer;          /* skvd_reducer actually used */
  int32_t hier_groups_cap;  /* first-level groups of the hierarchical reducer, else 0 */
  int32_t rows_per_group;   /* G * max_q_per_seq rows one workgroup serves */
  int32_t num_cus;          /* compute units planned for */
  int64_t rows_cap;         /* max_batch * max_q_per_seq * Hq */
  uint64_t workspace_bytes;
  uint64_t status_offset;   /* byte offset of the uint32 status word in the workspace */
  int32_t schedule;         /* skvd_schedule actually used */
  int32_t part_stride;      /* partial slots per row in the workspace (splits_cap, + 1 when
                               balanced: a row may straddle one more share boundary) */
  int32_t grid_wgs;         /* partial-kernel workgroups launched (upper bound) */
  int32_t heads_per_wg;     /* KV heads (waves) per partial-kernel workgroup */
} skvd_plan_info;

/* Status-word bits (debug plans). */
#define SKVD_STATUS_KV_LEN_CLAMPED 0x1u  /* some kv_len[b] was < 0 or > max_kv_len */
#define SKVD_STATUS_PAGE_CLAMPED 0x2u    /* some page id read was outside [0, num_pages) */

typedef struct skvd_plan skvd_plan;

/* Arguments of one decode. Element strides; every array lives on the plan's device. */
typedef struct {
  const void *q;             /* f16 [B*T, Hq, D]; row b*T + t; D dense; 16-byte aligned */
  int64_t q_tok_stride;      /* elements between rows b*T + t and b*T + t + 1 (multiple of 8) */
  int64_t q_head_stride;     /* elements between heads (multiple of 8) */
  const void *k_pages;       /* [num_k_pages, P, Hkv, D] f16, int8 or E4M3 bytes, or
                                [num_k_pages, P, Hkv, D/2] q4_0 code bytes; 16-byte aligned */
  const void *v_pages;       /* [num_v_pages, P, Hkv, D] (q4_0: D/2), same strides as K */
  int64_t page_stride;       /* elements between pages (shared by K and V; bytes for the
                                one-byte formats and q4_0); the three strides are non-negative
                                multiples of 16 bytes, else SKVD_ERR_LAYOUT */
  int64_t tok_stride;        /* elements between slots of a page */
  int64_t head_stride;       /* elements between KV heads */
  int64_t num_k_pages;       /* pages in the K pool (>= 1); ids are clamped below it */
  int64_t num_v_pages;       /* pages in the V pool (>= 1) */
  const void *k_scales;      /* int8, q4_0: f16 [num_k_pages, P, Hkv, D/32]; fp8: one f32
                                (k_scale, device memory, 4-byte aligned, read by the kernels at
                                each call, so a captured graph sees its current value); f16:
                                NULL */
  const void *v_scales;      /* int8, q4_0: f16 [num_v_pages, P, Hkv, D/32]; fp8: one f32
                                (v_scale); f16: NULL */
  int64_t scale_page_stride; /* int8, q4_0 (ignored otherwise): elements; shared by both scale
                                pools; the D/32 scales of a token-head are contiguous; pools
                                8-byte aligned and all three strides multiples of 4 elements
                                (else SKVD_ERR_LAYOUT) */
  int64_t scale_tok_stride;
  int64_t scale_head_stride;
  const int32_t *page_table; /* [B, table_stride]; entry i of row b is the page holding
                                positions i*P .. i*P+P-1; entries past ceil(kv_len/P) are
                                never read */
  int64_t table_stride;      /* >= ceil(max_kv_len / P) */
  const int32_t *kv_len;     /* [B] device int32 */
  int32_t batch;             /* B, 0..max_batch (0 launches nothing) */
  int32_t q_per_seq;         /* T, 1..max_q_per_seq */
  float sm_scale;            /* softmax scale applied to q . k (finite) */
  int32_t reserved;          /* must be 0 */
  void *o;                   /* f16 [B*T, Hq, D] dense, written */
  float *lse;                /* f32 [B*T, Hq] dense, written; may be NULL (not written) */
} skvd_decode_args;

/* Plan: validate the static shape, choose blocks per split and the reducer, and size the
 * workspace. This is the library's form of the selection step of 1bit-MONSTER/engine issue
 * #115: comment "Root-caused" has a decode-split template chosen by the KV capacity and a
 * reducer family by the number of 64-token producer blocks, and every candidate rejected
 * ("all_rejected") past 2048 tokens; comment "Closing the remaining half of this issue" gives
 * the capacity as ceil(n / 64) * 64 and covers any capacity with a multipass reducer. Here any
 * max_kv_len >= 1 is planned (no length is rejected), the reducer follows the partial count,
 * and each call derives its block counts from kv_len on the device, as that issue's comment
 * "Deep-context decode failures were JIT SGPR exhaustion" derives the producer block count from
 * the run-time token count rather than the compile-time capacity. Host only: no device
 * allocation; with num_cus > 0 no HIP call at all. The environment variable
 * SKVD_LOG_DISPATCH=1 prints the resolved plan to stderr here (never in a launch). On success
 * *out owns a plan to free with skvd_plan_destroy; on failure *out is NULL and the
 * status says why (see skvd_last_error). params and out must be non-NULL (SKVD_ERR_NULL). */
skvd_status skvd_plan_create(const skvd_plan_params *params, skvd_plan **out);
/* Frees a plan (NULL: no-op). The caller's workspace is the caller's to free. */
void skvd_plan_destroy(skvd_plan *plan);
/* Workspace bytes skvd_decode needs for this plan (0 for a NULL plan). */
size_t skvd_plan_workspace_bytes(const skvd_plan *plan);
/* What the plan resolved to, into *info (both non-NULL, else SKVD_ERR_NULL). */
skvd_status skvd_plan_get_info(const skvd_plan *plan, skvd_plan_info *info);
/* NUL-terminated one-line description of the resolved plan (blocks per split, splits,
 * schedule, reducer, workspace bytes), truncated to buf_len - 1 characters: the counterpart of
 * the dispatch log the pages turn on to confirm which kernel serves a given depth
 * (GGML_HRX_LOG_DISPATCH=1, 1bit-MONSTER/engine issue #115, comments "Fixed" and "Closing the
 * remaining half of this issue"). plan and buf non-NULL and buf_len > 0, else SKVD_ERR_NULL. */
skvd_status skvd_plan_describe(const skvd_plan *plan, char *buf, size_t buf_len);

/* Validation alone: the checks skvd_decode makes before launching, with no HIP call. */
skvd_status skvd_decode_check(const skvd_plan *plan, const skvd_decode_args *args,
                              size_t workspace_bytes);

/* Decode: partial kernel, then the plan's reducer, enqueued on `stream` (a hipStream_t;
 * NULL is the null stream). Asynchronous; writes o, lse and the workspace only. The
 * current HIP device must be the plan's device. */
skvd_status skvd_decode(const skvd_plan *plan, const skvd_decode_args *args, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Allocation-free decode, for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, result and errors as skvd_decode, but the workspace is a
 * device array inside the library of SKVD_NOALLOC_WORKSPACE_MAX bytes per GPU (held until
 * the process ends); plans whose skvd_plan_workspace_bytes() exceed it return
 * SKVD_ERR_WORKSPACE, and debug plans (whose status word the caller reads from its own
 * workspace) return SKVD_ERR_PLAN. No hipMalloc, hipFree or allocating call. The array's
 * device address is looked up on the first call on each device (do that first call outside
 * graph capture). Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads, other plans) race and must be ordered by the caller. */
#define SKVD_NOALLOC_WORKSPACE_MAX (((size_t)32) << 20)
skvd_status skvd_decode_noalloc(const skvd_plan *plan, const skvd_decode_args *args,
                                void *stream);

/* The two stages of skvd_decode, for callers that time or compose them. The partial stage
 * writes one (max, sum, f32 output) partial per split into the workspace, or o and lse
 * directly when the plan's reducer is SKVD_REDUCER_NONE; the merge stage reads those
 * partials and writes o and lse (and does nothing for SKVD_REDUCER_NONE). Running
 * skvd_decode_partial then skvd_decode_merge on one stream equals skvd_decode. */
skvd_status skvd_decode_partial(const skvd_plan *plan, const skvd_decode_args *args,
                                void *workspace, size_t workspace_bytes, void *stream);
skvd_status skvd_decode_merge(const skvd_plan *plan, const skvd_decode_args *args,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Measurement aid: skvd_decode_partial whose kernel dispatch itself records its begin time in
 * start_event and its end time in stop_event (hipExtLaunchKernel), so that
 * hipEventElapsedTime(start_event, stop_event) is the partial kernel's execution alone, with no
 * marker packets around it. Both are hipEvent_t that the caller created, with timing enabled,
 * on the plan's device; either may be NULL. With batch 0 nothing is launched and the events are
 * left untouched. */
skvd_status skvd_decode_partial_timed(const skvd_plan *plan, const skvd_decode_args *args,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      void *start_event, void *stop_event);

/* Test aid: copy the raw elements of every visible K/V row (position j < kv_len[b]) into
 * dense [B, max_len, Hkv, D] arrays (element size 2 for f16, 1 for int8 and fp8; q4_0 rows are
 * D/2 code bytes), and for int8 and q4_0 the raw f16 scales into dense [B, max_len, Hkv, D/32]
 * arrays (dense_ks/dense_vs; NULL for f16 and fp8, whose scales are per tensor).
 * It runs the plan's own partial-kernel variant -- the same schedule, page lookups, lane
 * offsets, loads and (int8, q4_0) register transposes as skvd_decode -- in a debug form that stores
 * each K/V element and scale it holds at the point where the decode consumes it, at the
 * position the decode attributes it to, and computes nothing else; a wrong address or lane
 * mapping in the decode shows up as a wrong element here. Rows at or beyond kv_len[b] are not
 * written. max_len >= every kv_len[b]; dense_k / dense_v 16-byte aligned, dense_ks / dense_vs
 * 2-byte aligned. o, lse and the workspace are not used. */
skvd_status skvd_gather_debug(const skvd_plan *plan, const skvd_decode_args *args,
                              int32_t max_len, void *dense_k, void *dense_v, void *dense_ks,
                              void *dense_vs, void *stream);

/* Measurement aid (not part of the decode): read `bytes` bytes at `buf` once with 16-byte
 * loads spread over the whole chip, so that a benchmark can report the HBM read bandwidth this
 * GPU actually sustains next to the decode's. buf is device memory, 16-byte aligned; bytes is
 * a multiple of 16; sink is a device uint32 that the kernel may write (keeps the loads live).
 * Asynchronous on `stream`. */
skvd_status skvd_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* --------------------------------------------------------------------------- prefill
 * The multi-token route: any number T >= 1 of query tokens per sequence (prompt processing,
 * long speculative drafts) over the same paged cache, with the same arguments, result, causal
 * reading and output layout as skvd_decode (the T query tokens are the last T cached positions;
 * token t sees positions j <= kv_len[b] - T + t). llama-cpp-turboquant PR #176 ("HIP: fix turbo
 * KV decode crash under graph capture; batch-aware VEC/TILE FA routing", section "Changes")
 * keeps the vector decode for at most 8 query tokens and routes larger batches to a tiled
 * matrix-core kernel; its tiled path first dequantized the quantized cache into f16 buffers.
 * This route is one tiled MFMA kernel that reads the pages itself and widens the one-byte
 * formats (int8: value = int8 * f16 scale per 32 elements; fp8: E4M3 * tensor scale; q4_0:
 * (c - 8) * f16 scale per 32 elements) on the way into LDS: no f16 temporary, no workspace.
 * Formats: f16, int8, fp8, q4_0; head_dim 128 or 256.
 *
 * - args: as skvd_decode_args, with q_per_seq = T in 1..max_kv_len (not bounded by the plan's
 *   max_q_per_seq); batch <= max_batch; o [B*T, Hq, D] f16 dense and lse [B*T, Hq] f32 (may be
 *   NULL) are written, nothing else. The plan's Hq / Hkv must be <= 64.
 * - Device-data contract: T <= kv_len[b] <= max_kv_len. Rows that see no position (kv_len[b] <
 *   T) get o = 0 and lse = -inf; kv_len is clamped and page ids are clamped into the pools as in
 *   the decode.
 * - Graph capture: no allocation, synchronization or device-to-host read; one kernel launch. */

/* Validation alone: the checks skvd_prefill makes before launching, with no HIP call. */
skvd_status skvd_prefill_check(const skvd_plan *plan, const skvd_decode_args *args);

/* Prefill: one kernel on `stream` (a hipStream_t; NULL is the null stream), asynchronous. The
 * current HIP device must be the plan's device. Errors as for skvd_decode. */
skvd_status skvd_prefill(const skvd_plan *plan, const skvd_decode_args *args, void *stream);

/* Batch-aware routing (llama-cpp-turboquant PR #176, section "Changes": at most 8 query
 * tokens per sequence stay on the decode path, larger batches go to the tiled matrix-core
 * kernel): skvd_decode when args->q_per_seq <= the plan's max_q_per_seq (itself <= 8), else
 * skvd_prefill. Same arguments, result and errors as the route taken; the workspace is used
 * only by the decode route. */
skvd_status skvd_attention(const skvd_plan *plan, const skvd_decode_args *args, void *workspace,
                           size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------- merge states
 * Cascade (shared-prefix) attention: merge S attention states of each row, computed over
 * disjoint key sets (e.g. the pages of a prefix shared by many sequences, and each sequence's
 * own suffix), into the state over their union, with the log-sum-exp reduction that merges the
 * split-KV partials (1bit-MONSTER/engine issue #115, comments "Root-caused" and "Closing the
 * remaining half of this issue"; AMD-Ecosystem/flashinfer PR #397 lists a cascade test under
 * "Test plan"):
 *     M = max_s lse_s,  w_s = exp(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
 *     lse = M + ln sum_s w_s     (natural log, as skvd_decode writes it)
 * A state with lse = -inf (an empty key set) contributes nothing; a row whose states are all
 * empty gets o = 0 and lse = -inf. The states are exactly what skvd_decode / skvd_prefill write
 * (o f16, lse f32), so a cascade is: decode the prefix, decode the suffixes, merge.
 *
 * - o_states: f16, state s of row r at o_states + s * o_state_stride + r * o_row_stride
 *   (elements), head_dim dense; lse_states: f32 at s * lse_state_stride + r. Read only.
 * - o: f16 [rows, head_dim] dense, written; lse: f32 [rows], written, may be NULL. They must not
 *   overlap the states.
 * - head_dim in {64, 128, 256, 512}; num_states >= 1; 0 <= rows <= 2^31 (0 launches nothing).
 *   o_states and o 16-byte aligned with strides multiples of 8 elements; lse arrays 4-byte
 *   aligned. Device pointers; one kernel on `stream`, asynchronous,
 *   no allocation (graph-capture safe). Errors as for skvd_decode. */
skvd_status skvd_merge_states(const void *o_states, int64_t o_state_stride, int64_t o_row_stride,
                              const float *lse_states, int64_t lse_state_stride,
                              int32_t num_states, int64_t rows, int32_t head_dim, void *o,
                              float *lse, void *stream);

/* ---------------------------------------------------------------------------- append
 * Writing new tokens into the paged cache: the step right before a decode, and the one
 * operation that writes the cache (AMD-Ecosystem/flashinfer PR #397, "Stop declaring the paged
 * KV cache mutated on read-only attention ops", section "What changed": append genuinely writes
 * the cache and keeps declaring it written; the decode above only reads it). New token i belongs
 * to sequence b = batch_idx[i] at logical position j = positions[i]; its K row of KV head g is
 * written to slot j % P of page page_table[b][j / P] -- the address the decode reads -- and its
 * V row to the same place in the V pool. An f16 cache receives the f16 elements verbatim. An
 * int8 cache (value = int8 * scale, one f16 scale per 32 contiguous head_dim elements: the
 * q8_0-style KV type named in 1bit-MONSTER/engine issue #115, comment "Fixed") is quantized on
 * write, symmetric, the largest magnitude of each group of 32 mapped to 127:
 *     s = f16(max|x| / 127)             (quotient in f32, rounded once to f16, nearest even)
 *     c = clip(rint(x / s), -127, 127)  (quotient in f32, rint to nearest even; s = 0 -> c = 0)
 * with no f16 temporary: each row is read once and written once. An fp8 cache (OCP E4M3 bytes
 * with one f32 scale s per tensor, AMD-Ecosystem/flashinfer PR #397 commit messages) stores for
 * each element the E4M3 value nearest to clip(x / s, -448, 448) (the quotient in f32, correctly
 * rounded; ties to the even mantissa; a NaN quotient stores 0); its scales are only read.
 * A q4_0 cache (SKVD_KV_Q4_0) takes the published ggml q4_0 rule per group of 32, in f32:
 *     m = the element of largest magnitude (the first on a tie; +0 if all are 0),
 *     d = m / -8,  r = 1 / d (0 if d = 0),  c = min(15, trunc(x * r + 8.5)),
 * the product and the sum each rounded to f32, and stores f16(d) (nearest even) as the scale.
 * Non-finite inputs: int8 -- a NaN element stores code 0 and is left out of its group's maximum;
 * an infinite element gives its group the scale f16(inf) = inf and every code 0. fp8 -- NaN
 * stores 0, +-inf saturates to +-448. q4_0 -- a NaN element stores code 8 and is left out of the
 * maximum; an infinite m gives the scale f16(-m / 8) = -+inf and every code 8.
 *
 * - Written: exactly the K/V elements (and, int8 and q4_0, the scales) of the slots the tokens
 *   name.
 *   Nothing else; no workspace. k_new, v_new, batch_idx, positions and the table are read only.
 * - Skips (device-data contract, not checked with a synchronization): a token whose batch_idx is
 *   outside [0, batch) or whose position is outside [0, the plan's max_kv_len) writes nothing; a
 *   page id outside [0, num_k_pages) (or num_v_pages) skips that pool's write. Two tokens naming
 *   the same slot leave it undefined (no ordering between them).
 * - The pools may be any views the strides describe (K and V share page shape and strides, as
 *   for the decode), but must not overlap each other or the inputs.
 * - Graph capture: no allocation, synchronization or device-to-host read; one kernel launch.
 * The plan supplies Hkv, D, P, the cache type, max_kv_len and the device; other plan fields are
 * not used. */
typedef struct {
  const void *k_new;          /* f16 [N, Hkv, D]; D dense; 16-byte aligned (k_new, v_new,
                                 batch_idx and positions may be NULL when N is 0) */
  const void *v_new;          /* f16 [N, Hkv, D], same strides as k_new; 16-byte aligned */
  int64_t new_tok_stride;     /* elements between tokens (non-negative multiple of 8) */
  int64_t new_head_stride;    /* elements between KV heads (non-negative multiple of 8) */
  const int32_t *batch_idx;   /* [N] device: sequence (page-table row) of each new token */
  const int32_t *positions;   /* [N] device: logical position of each new token */
  int32_t num_tokens;         /* N >= 0 (0 launches nothing) */
  int32_t batch;              /* rows of page_table, >= 0 */
  void *k_pages;              /* [num_k_pages, P, Hkv, D] f16, int8 or E4M3 (q4_0: D/2 code
                                 bytes), written; layout rules as in skvd_decode_args */
  void *v_pages;              /* [num_v_pages, P, Hkv, D], same strides as K, written */
  int64_t page_stride;        /* elements; shared by K and V */
  int64_t tok_stride;
  int64_t head_stride;
  int64_t num_k_pages;        /* >= 1 */
  int64_t num_v_pages;        /* >= 1 */
  void *k_scales;             /* int8, q4_0: f16 [num_k_pages, P, Hkv, D/32], written; fp8:
                                 one f32 (k_scale, device memory, 4-byte aligned), read; f16:
                                 NULL */
  void *v_scales;             /* int8, q4_0: f16 [num_v_pages, P, Hkv, D/32], written; fp8:
                                 one f32 (v_scale), read; f16: NULL */
  int64_t scale_page_stride;  /* elements; layout rules as in skvd_decode_args */
  int64_t scale_tok_stride;
  int64_t scale_head_stride;
  const int32_t *page_table;  /* [batch, table_stride] */
  int64_t table_stride;       /* >= ceil(max_kv_len / P) */
} skvd_append_args;

/* Validation alone: the checks skvd_append makes before launching, with no HIP call. */
skvd_status skvd_append_check(const skvd_plan *plan, const skvd_append_args *args);

/* Append: one kernel on `stream` (a hipStream_t; NULL is the null stream), asynchronous. The
 * current HIP device must be the plan's device. Host-checkable faults (NULL pointers, strides,
 * alignment, scales present/absent against the cache type, table_stride) return an error before
 * anything is launched; a launch failure returns SKVD_ERR_HIP. */
skvd_status skvd_append(const skvd_plan *plan, const skvd_append_args *args, void *stream);

/* Errors are statuses returned before anything runs, never a fault, an abort or a silent
 * fallback: the failures the pages trace were a selection that rejected every candidate
 * ("all_rejected", 1bit-MONSTER/engine issue #115, comment "Root-caused") and a launch that
 * returned res = -3 after the kernel's build failed (comment "Deep-context decode failures were
 * JIT SGPR exhaustion"). skvd_status_string names a status (a static string; "unknown status"
 * for other values). */
const char *skvd_status_string(skvd_status status);
/* Message of the last failed call on this thread ("" if none): which argument or limit a
 * status came from. The string is owned by the library and valid until this thread's next
 * call. */
const char *skvd_last_error(void);
/* SKVD_ABI_VERSION of the built library; the Python binding refuses a mismatch. */
int32_t skvd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKVD_H */
