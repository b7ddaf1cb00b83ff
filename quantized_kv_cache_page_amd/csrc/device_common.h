// Device helpers shared by the decode's partial kernel and its merge kernels: the cache's one
// address function, wavefront reductions and the balanced schedule's share arithmetic.
#pragma once

#include <hip/hip_runtime.h>

#include "skvd_internal.h"

namespace skvd {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------------------- addressing
// The one address function of the cache: the page holding logical position j of sequence b
// (clamped into [0, num_pages) so that a bad table entry cannot read out of range), and the
// element offset of (page, slot, KV head) in a pool.
__device__ __forceinline__ int64_t lookup_page(const int32_t *table, int64_t table_stride, int b,
                                               int j, int page_shift, int64_t num_pages,
                                               bool *clamped) {
  int64_t pg = table[(int64_t)b * table_stride + (j >> page_shift)];
  const bool bad = pg < 0 || pg >= num_pages;
  *clamped = bad;
  return bad ? (pg < 0 ? 0 : num_pages - 1) : pg;
}

__device__ __forceinline__ int64_t row_offset(int64_t page, int slot, int kvh, int64_t page_stride,
                                              int64_t tok_stride, int64_t head_stride) {
  return page * page_stride + (int64_t)slot * tok_stride + (int64_t)kvh * head_stride;
}

__device__ __forceinline__ int clamp_len(int L, int max_len, unsigned *status, int debug) {
  if (L < 0 || L > max_len) {
    if (debug) atomicOr(status, (unsigned)SKVD_STATUS_KV_LEN_CLAMPED);
    L = L < 0 ? 0 : max_len;
  }
  return L;
}

// ----------------------------------------------------------------------------- wave helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes on DPP, no LDS: shifts right by 1, 2, 4 and 8 within
// each 16-lane row (lanes shifted in from outside the row add 0), then lane 15's total into
// rows 1 and 3 and lane 31's into rows 2 and 3 (the row broadcasts).
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned dpp_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ unsigned wave_inclusive_sum(unsigned x) {
  x += dpp_u<0x111, 0xF>(x);  // row_shr:1
  x += dpp_u<0x112, 0xF>(x);  // row_shr:2
  x += dpp_u<0x114, 0xF>(x);  // row_shr:4
  x += dpp_u<0x118, 0xF>(x);  // row_shr:8
  x += dpp_u<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x += dpp_u<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// max / sum over the 16 lanes of a DPP row (xor 1, xor 2, half-mirror, mirror)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane-swap sums (gfx950 v_permlane32_swap / v_permlane16_swap, which trade the upper 32
// lanes of their first operand with the lower 32 of the second, and the odd 16-lane rows of the
// first with the even rows of the second). swap_sum32: lanes 0..31 get a(l) + a(l + 32), lanes
// 32..63 get b(l - 32) + b(l). swap_sum16: rows 0 and 2 (lanes / 16) get a(l) + a(l ^ 16),
// rows 1 and 3 get b(l ^ 16) + b(l). Vector ALU only, no LDS.
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS hand-off between the lanes of a one-wave workgroup: a wavefront-scope fence and wave
// barrier order the LDS accesses without waiting on outstanding global loads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// ----------------------------------------------------------------------------- balanced schedule
// The batch's 64-token blocks in (sequence, schedule head, block) order, cut into n_shares
// equal contiguous shares: share w covers [w N / W, (w + 1) N / W). A schedule head is a group
// of KV heads served by one workgroup, or, when a KV head has more query rows than one
// workgroup holds, one row group of a KV head (LaunchArgs::sched_heads of them per sequence).
// Lane l of the wave that computes the shares holds the sequences [l s, l s + s), s =
// LaunchArgs::seqs_per_lane (1 up to 64 sequences, more for larger batches): their block count
// and the blocks of all earlier lanes' sequences. Every lane of the wave must be active.
typedef const __attribute__((address_space(4))) int32_t *cint_t;  // scalar-loaded int32 array

struct Shares {
  int len_l;         // seqs_per_lane == 1: the clamped length of the lane's sequence
  unsigned nb_l;     // blocks of the lane's sequences
  unsigned pre_l;    // blocks of all earlier lanes' sequences
  int64_t n_blocks;  // N = schedule heads * sum of block counts (below 2^31)
  int n_shares;      // W = min(grid, N / piece_min), at least 1 when N > 0
};

__device__ __forceinline__ Shares balanced_shares(const LaunchArgs &a, int debug) {
  const int lane = threadIdx.x & 63;
  const int spl = a.seqs_per_lane;
  Shares sh;
  sh.len_l = 0;
  unsigned nb = 0;
  for (int i = 0; i < spl; ++i) {
    const int b = lane * spl + i;
    const int L = b < a.batch ? clamp_len(a.kv_len[b], a.max_kv_len, a.status, debug) : 0;
    if (i == 0) sh.len_l = L;
    nb += (unsigned)(L + 63) >> 6;
  }
  sh.nb_l = nb;
  const unsigned inc = wave_inclusive_sum(nb);
  sh.pre_l = inc - nb;
  // (readlane: the total is wave-uniform, so it and everything derived from it stay scalar;
  // the plan keeps N below 2^31, so 32-bit arithmetic: a 64-bit division is a long scalar
  // sequence on the launch's critical path)
  const unsigned n = (unsigned)__builtin_amdgcn_readlane((int)inc, 63) * (unsigned)a.sched_heads;
  const unsigned pieces = a.piece_min == 1 ? n : n / (unsigned)a.piece_min;
  sh.n_blocks = n;
  sh.n_shares = n == 0 ? 0 : (int)max(1u, min((unsigned)a.grid_wgs, pieces));
  return sh;
}

// One sequence of the balanced schedule: its index, the blocks of all earlier sequences, its
// block count and clamped length. Wave-uniform.
struct SeqRef {
  int b;
  unsigned pre;
  int nb;
  int L;
};

// Walk the sequences of lane l from the first, starting at `pre` blocks, until the one whose
// blocks hold sequence-block index xq (or, with stop_b >= 0, until sequence stop_b). Scalar
// loads of kv_len; at most seqs_per_lane steps.
__device__ __forceinline__ SeqRef walk_lane(const LaunchArgs &a, int l, unsigned pre, unsigned xq,
                                            int stop_b) {
  const cint_t kl = (cint_t)a.kv_len;
  const int spl = a.seqs_per_lane;
  int b = l * spl;
  for (int i = 0;; ++i, ++b) {
    const int raw = b < a.batch ? kl[b] : 0;
    const int L = raw < 0 ? 0 : (raw > a.max_kv_len ? a.max_kv_len : raw);
    const int nb = (L + 63) >> 6;
    const bool here = stop_b >= 0 ? b == stop_b : xq < pre + (unsigned)nb;
    if (here || i == spl - 1) return {b, pre, nb, L};
    pre += (unsigned)nb;
  }
}

// The sequence whose blocks hold sequence-block index xq (xq < total blocks).
__device__ __forceinline__ SeqRef seq_at(const LaunchArgs &a, const Shares &sh, unsigned xq) {
  const bool mine = sh.pre_l <= xq && xq < sh.pre_l + sh.nb_l;
  const int l = __builtin_ctzll(__ballot(mine));
  const unsigned pre = (unsigned)__builtin_amdgcn_readlane((int)sh.pre_l, l);
  if (a.seqs_per_lane == 1)
    return {l, pre, __builtin_amdgcn_readlane((int)sh.nb_l, l),
            __builtin_amdgcn_readlane(sh.len_l, l)};
  return walk_lane(a, l, pre, xq, -1);
}

// Sequence b's place in the block list.
__device__ __forceinline__ SeqRef seq_info(const LaunchArgs &a, const Shares &sh, int b) {
  const int l = b / a.seqs_per_lane;
  const unsigned pre = (unsigned)__builtin_amdgcn_readlane((int)sh.pre_l, l);
  if (a.seqs_per_lane == 1)
    return {b, pre, __builtin_amdgcn_readlane((int)sh.nb_l, l),
            __builtin_amdgcn_readlane(sh.len_l, l)};
  return walk_lane(a, l, pre, 0u, b);
}

// The share holding global block x (0 <= x < N): the largest w with floor(w N / W) <= x, that
// is floor(((x + 1) W - 1) / N). In double, exactly: the numerator (below 2^46) and N are
// exact, the division is correctly rounded, and a quotient that is not an integer lies at least
// 1/N > 2^-31 below the next integer, far beyond the rounding error at quotients up to W <= 2^15
// (a 64-bit integer division is a long scalar sequence).
__device__ __forceinline__ int share_of(int64_t x, int64_t n_blocks, int n_shares) {
  return (int)__builtin_floor(((double)(x + 1) * (double)n_shares - 1.0) / (double)n_blocks);
}

}  // namespace skvd
