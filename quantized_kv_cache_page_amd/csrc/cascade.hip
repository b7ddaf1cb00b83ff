// Merge of attention states (cascade / shared-prefix attention): the log-sum-exp reduction that
// merges the split-KV partials, applied to whole (o, lse) states computed over disjoint key
// sets -- e.g. a prefix of pages shared by many sequences, decoded once per row, and each
// sequence's own suffix (1bit-MONSTER/engine issue #115, comments "Root-caused" and "Closing
// the remaining half of this issue": partials merged by a log-sum-exp reducer; AMD-Ecosystem/
// flashinfer PR #397 lists a cascade test under "Test plan").
//   M = max_s lse_s, w_s = e^(lse_s - M), o = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s,
// states with lse = -inf skipped, all-empty rows -> o = 0, lse = -inf.
//
// D/8 lanes per row (8 consecutive head_dim elements each, one 16-byte load per state), states
// merged in order with an online max in base 2, several states' loads in flight at once; every
// state's row is one contiguous D*2-byte read and the output one contiguous write: an HBM
// stream.
#include <hip/hip_runtime.h>

#include "skvd_internal.h"

namespace skvd {
namespace {

constexpr float kCLog2e = 1.4426950408889634f;
constexpr float kCLn2 = 0.6931471805599453f;

typedef _Float16 mh8 __attribute__((ext_vector_type(8)));
constexpr float kCNegInf = -__builtin_huge_valf();
constexpr int kStatesPerRound = 4;  // states whose loads are issued together

// D/8 lanes per row, 8 elements (one 16-byte load) per lane per state; a 256-lane workgroup
// covers 2048/D rows. The loads of up to kStatesPerRound states are issued before any of them
// is merged, so each lane keeps several 16-byte reads in flight.
template <int D>
__global__ __launch_bounds__(256) void merge_states_kernel(MergeStatesArgs a) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  if (row >= a.rows) return;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float m = kCNegInf, w_sum = 0.f;
  const _Float16 *base = (const _Float16 *)a.o_states + row * a.o_row_stride + 8 * part;
  for (int s0 = 0; s0 < a.num_states; s0 += kStatesPerRound) {
    float x[kStatesPerRound];
    mh8 o[kStatesPerRound];
#pragma unroll
    for (int k = 0; k < kStatesPerRound; ++k) {
      const int s = min(s0 + k, a.num_states - 1);  // past the last state: re-read, weight 0
      x[k] = s0 + k < a.num_states ? a.lse_states[s * a.lse_state_stride + row] * kCLog2e
                                   : kCNegInf;
      o[k] = *(const mh8 *)(base + s * a.o_state_stride);
    }
#pragma unroll
    for (int k = 0; k < kStatesPerRound; ++k) {
      // an empty state (lse = -inf) has weight 0 and leaves the running max alone
      const float m_new = fmaxf(m, x[k]);
      const float scale_old = m_new == kCNegInf ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
      const float w = x[k] == kCNegInf ? 0.f : __builtin_amdgcn_exp2f(x[k] - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * scale_old + w * (float)o[k][e];
      w_sum = w_sum * scale_old + w;
      m = m_new;
    }
  }
  mh8 out;
  const float inv = w_sum > 0.f ? 1.f / w_sum : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (_Float16)(acc[e] * inv);
  *(mh8 *)((_Float16 *)a.o + row * D + 8 * part) = out;
  if (part == 0 && a.lse) a.lse[row] = w_sum > 0.f ? (m + __log2f(w_sum)) * kCLn2 : kCNegInf;
}

}  // namespace

int launch_merge_states(const MergeStatesArgs &a, void *stream) {
  if (a.rows == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const unsigned blocks = (unsigned)((a.rows * (a.head_dim / 8) + 255) / 256);
  switch (a.head_dim) {
    case 64: merge_states_kernel<64><<<blocks, 256, 0, st>>>(a); break;
    case 128: merge_states_kernel<128><<<blocks, 256, 0, st>>>(a); break;
    case 256: merge_states_kernel<256><<<blocks, 256, 0, st>>>(a); break;
    default: merge_states_kernel<512><<<blocks, 256, 0, st>>>(a); break;
  }
  return (int)hipGetLastError();
}

}  // namespace skvd
