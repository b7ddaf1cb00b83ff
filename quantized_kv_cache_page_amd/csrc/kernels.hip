// HIP kernels for split-KV paged decode attention on gfx950 (CDNA4, wave64): the merge of the
// partial kernel's partials (partial.h holds the partial kernel), the launch sequence, and a
// streaming-read reference kernel.
//
// Merge kernels: the log-sum-exp reduction of the partials of one row,
//   M = max m_s, S = sum_s l_s 2^(m_s - M), o = sum_s 2^(m_s - M) o_s / S,
//   lse = (M + log2 S) ln 2,
// as direct (serial), cooperative (one lane per partial, <= 64), multipass (lane-strided,
// any count) and hierarchical (64 partials per workgroup, then a multipass over groups).
// Loop bounds come from kv_len on the device; the partial stride is the plan's capacity.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"

namespace skvd {

// ----------------------------------------------------------------------------- merge kernels
// The partials of output row `row` (sequence b, query head -> KV head): their count, the
// index of the first and the index step between consecutive ones. Static: the splits covering
// the sequence's blocks, contiguous at row * part_stride. Balanced: the shares the (sequence,
// schedule head) schedule row r meets, w_first .. w_last, in compact slots r + w, by the
// partial kernel's own integer arithmetic. Called by the whole wave.
struct RowParts {
  int64_t first;
  int64_t stride;
  int count;
};

// (Called first in every merge kernel: it also brings in the argument block's lines that the
// merge reads later (kv_len's, the workspace and output pointers') with the first batch of
// argument loads, one memory round trip fewer. Rows are a 1-D grid index, below 2^31: 32-bit
// divisions.)
__device__ __forceinline__ RowParts row_parts(const LaunchArgs &a, int64_t row) {
  asm volatile("" ::"s"(a.kv_len), "s"(a.ws_ml));
  const unsigned per_seq = (unsigned)a.T * (unsigned)a.Hq;
  const int b = (int)((unsigned)row / per_seq);
  if (!a.balanced) {
    const int L = clamp_len(a.kv_len[b], a.max_kv_len, a.status, 0);
    const int nblk = (L + 63) >> 6;
    return {row * a.part_stride, 1, (nblk + a.bps - 1) / a.bps};
  }
  const int rem = (int)((unsigned)row - (unsigned)b * per_seq);
  const int t = rem / a.Hq, qh = rem - t * a.Hq;
  const int kvh = qh / a.G, hg = qh - kvh * a.G;
  const int r = hg + a.G * t;  // query row within the KV head
  const int RPG = a.rows_per_group, NRG = a.row_groups;
  const int rg = r / RPG;      // its row group
  const int HW = a.heads_per_wg, Hg = a.sched_heads;
  const int kgrp = kvh / HW, head_w = kvh - kgrp * HW;
  const int grp = kgrp * NRG + rg;  // the schedule head
  const Shares sh = balanced_shares(a, 0);
  const SeqRef s = seq_info(a, sh, b);
  const int64_t pre_b = s.pre, nb_b = s.nb;
  if (nb_b == 0) return {0, 1, 0};
  const int64_t x0 = Hg * pre_b + grp * nb_b;  // the schedule row's first block
  const int w0 = share_of(x0, sh.n_blocks, sh.n_shares);
  const int w1 = share_of(x0 + nb_b - 1, sh.n_blocks, sh.n_shares);
  const int64_t sr = (int64_t)b * Hg + grp;
  return {((sr + w0) * HW + head_w) * RPG + (r - rg * RPG), (int64_t)HW * RPG, w1 - w0 + 1};
}

// Final write of one row from an unnormalized accumulator (wave 0's lanes hold D/64 each).
template <int D>
__device__ __forceinline__ void write_row(const LaunchArgs &a, int64_t row, const float *acc,
                                          float M, float S) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const bool empty = !(S > 0.f) || M == kNegInf;
  _Float16 *o = (_Float16 *)a.o + row * D + PER * lane;
  const float inv = empty ? 0.f : 1.f / S;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = (_Float16)(empty ? 0.f : acc[i] * inv);
  if (a.lse && lane == 0) a.lse[row] = empty ? kNegInf : (M + __log2f(S)) * kLn2;
}

// Weight of a partial against the row max (0 for an empty partial).
__device__ __forceinline__ float part_weight(float m, float M) {
  return m == kNegInf ? 0.f : fast_exp2(m - M);
}

// A running merge state (max in log2 units, sum relative to it, PER accumulator elements).
template <int PER>
struct MergeAcc {
  float M = kNegInf, S = 0.f;
  float acc[PER] = {};
  // fold in another state of the same form: the log-sum-exp combination
  __device__ __forceinline__ void fold(float M2, float S2, const float *acc2) {
    const float Mn = fmaxf(M, M2);
    if (Mn == kNegInf) return;
    const float wa = part_weight(M, Mn), wb = part_weight(M2, Mn);
    S = S * wa + S2 * wb;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = acc[i] * wa + acc2[i] * wb;
    M = Mn;
  }
};

// One lane's slice of PER consecutive floats of a partial's output row (PER = D / 64: 2, 3, 4
// or 8), with the widest loads its alignment allows.
template <int PER>
__device__ __forceinline__ void load_slice(const float *p, float (&v)[PER]) {
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const float4v x = *(const float4v *)(p + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[i + k] = x[k];
    }
  } else if constexpr (PER % 2 == 0) {
    typedef float float2v __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < PER; i += 2) {
      const float2v x = *(const float2v *)(p + i);
      v[i] = x[0];
      v[i + 1] = x[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = p[i];
  }
}

// Cooperative step: up to 64 partials (indices first, first + stride, ...) one per lane of this
// wave. Each lane's (m, l) gives the wave max and sum; the lanes then walk the partials' output
// slices (PER elements per lane) in rounds of U loads, each weight broadcast from the lane that
// owns the partial: U = 8 for up to 8 partials, else 64 / PER (a wave's 32 partials of a long
// single sequence at head_dim 128 in one round trip instead of four). The loads are
// unconditional (an index past the count re-reads the last partial, weighted 0): conditional
// ones became a branch around each load. Slices are addressed from the first one's row (a
// uniform base) with 32-bit byte offsets: consecutive partials are at most HW * RPG (128) rows
// apart, times the multipass waves' NW (4), so 63 steps of D floats stay below 2^26 bytes.
template <int D>
__device__ __forceinline__ void merge_lanes(const float *ml, const float *po, int64_t first,
                                            int64_t stride, int cnt, MergeAcc<D / 64> *out) {
  constexpr int PER = D / 64;
  typedef float float2v __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  float2v mlv = {kNegInf, 0.f};
  if (lane < cnt) mlv = *(const float2v *)(ml + 2 * (first + stride * lane));
  const float M = wave_max(mlv[0]);
  const float w = M == kNegInf ? 0.f : part_weight(mlv[0], M);
  const float S = wave_sum(w * mlv[1]);
  const char *base = (const char *)(po + first * D);
  const unsigned step = (unsigned)stride * (unsigned)(D * 4);
  const unsigned lane_off = (unsigned)(PER * 4 * lane);
  float acc[PER] = {};
  auto rounds = [&](auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    for (int k0 = 0; k0 < cnt; k0 += U) {
      float ov[U][PER];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const unsigned jj = (unsigned)min(k0 + j, cnt - 1);
        load_slice<PER>((const float *)(base + (lane_off + jj * step)), ov[j]);
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float wj = k0 + j < cnt ? readlane_f(w, k0 + j) : 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(wj, ov[j][i], acc[i]);
      }
    }
  };
  if (cnt > 8)
    rounds(std::integral_constant<int, 64 / PER>{});
  else
    rounds(std::integral_constant<int, 8>{});
  out->fold(M, S, acc);
}

// Multipass: the NW waves of the workgroup take partials w, w + NW, ... in rounds of 64 per
// wave; the per-wave states are combined through LDS. Wave 0 returns the row's state.
template <int D, int NW>
__device__ __forceinline__ MergeAcc<D / 64> merge_waves(const float *ml, const float *po,
                                                        int64_t first, int64_t stride, int n) {
  constexpr int PER = D / 64;
  __shared__ float st_lds[NW][2 + D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  MergeAcc<PER> r;
  const int nw = n > wave ? (n - wave + NW - 1) / NW : 0;  // this wave's partials
  for (int c0 = 0; c0 < nw; c0 += 64)
    merge_lanes<D>(ml, po, first + stride * (wave + (int64_t)NW * c0), stride * NW,
                   min(64, nw - c0), &r);
  if constexpr (NW > 1) {
    if (lane == 0) {
      st_lds[wave][0] = r.M;
      st_lds[wave][1] = r.S;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) st_lds[wave][2 + PER * lane + i] = r.acc[i];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int v = 1; v < NW; ++v) {
        float a2[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) a2[i] = st_lds[v][2 + PER * lane + i];
        r.fold(st_lds[v][0], st_lds[v][1], a2);
      }
    }
  }
  return r;
}

constexpr int kMergeWaves = 4;

// Direct: one wave; every lane walks all n partials in order (few partials).
template <int D>
__global__ __launch_bounds__(64) void merge_direct(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  const RowParts rp = row_parts(a, row);
  const int n = rp.count;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, a.ws_ml[2 * (rp.first + rp.stride * s)]);
  float S = 0.f, acc[PER] = {};
  for (int s0 = 0; s0 < n; s0 += 4) {
    float ov[4][PER];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (s0 + j < n) {
        load_slice<PER>(a.ws_o + (rp.first + rp.stride * (s0 + j)) * D + PER * threadIdx.x,
                        ov[j]);
      } else {
#pragma unroll
        for (int i = 0; i < PER; ++i) ov[j][i] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (s0 + j >= n) continue;
      const float *mlj = a.ws_ml + 2 * (rp.first + rp.stride * (s0 + j));
      const float w = part_weight(mlj[0], M);
      S += w * mlj[1];
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, ov[j][i], acc[i]);
    }
  }
  write_row<D>(a, row, acc, M, S);
}

// Cooperative (one wave, lane per partial, rounds of 64) and multipass (NW waves, lane-strided
// rounds): one workgroup per row. A multipass row with at most 64 partials is merged by wave 0
// alone (the count is uniform over the workgroup, so no wave reaches the LDS barrier).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void merge_rows(LaunchArgs a) {
  const int64_t row = blockIdx.x;
  const RowParts rp = row_parts(a, row);
  if constexpr (NW > 1) {
    if (rp.count <= 64) {
      if (threadIdx.x >= 64) return;
      MergeAcc<D / 64> r;
      merge_lanes<D>(a.ws_ml, a.ws_o, rp.first, rp.stride, rp.count, &r);
      write_row<D>(a, row, r.acc, r.M, r.S);
      return;
    }
  }
  const MergeAcc<D / 64> r = merge_waves<D, NW>(a.ws_ml, a.ws_o, rp.first, rp.stride, rp.count);
  if (threadIdx.x < 64) write_row<D>(a, row, r.acc, r.M, r.S);
}

// Hierarchical level 1: workgroup (row, g) merges the row's partials 64g .. 64g+63
// (cooperatively) into one unnormalized partial of the same form.
template <int D>
__global__ __launch_bounds__(64) void merge_hier1(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  const int g = blockIdx.y;
  const RowParts rp = row_parts(a, row);
  const int s0 = g * kHierGroup;
  if (s0 >= rp.count) return;
  MergeAcc<PER> r;
  merge_lanes<D>(a.ws_ml, a.ws_o, rp.first + rp.stride * s0, rp.stride,
                 min(kHierGroup, rp.count - s0), &r);
  float *dst = a.ws_ho + (row * a.hier_groups_cap + g) * D + PER * threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] = r.acc[i];
  if (threadIdx.x == 0) {
    float *hm = a.ws_hml + (row * a.hier_groups_cap + g) * 2;
    hm[0] = r.M;
    hm[1] = r.S;
  }
}

// Hierarchical level 2: multipass over the row's groups.
template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_hier2(LaunchArgs a) {
  const int64_t row = blockIdx.x;
  const int ng = (row_parts(a, row).count + kHierGroup - 1) / kHierGroup;
  const MergeAcc<D / 64> r = merge_waves<D, kMergeWaves>(
      a.ws_hml, a.ws_ho, row * a.hier_groups_cap, 1, ng);
  if (threadIdx.x < 64) write_row<D>(a, row, r.acc, r.M, r.S);
}

// ----------------------------------------------------------------------------- stream read (measurement aid)
// Every thread reads one 16-byte word per step with a grid-wide stride, so at any moment the
// chip sweeps one contiguous window: the plainest way to run HBM at its sustainable rate.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4v *p, size_t n, uint32_t *sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (; i < n; i += stride) {
    const uint4v v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

int launch_stream_read(const void *buf, size_t n16, uint32_t *sink, void *stream) {
  if (n16 == 0) return 0;
  stream_read_kernel<<<2048, 256, 0, (hipStream_t)stream>>>((const uint4v *)buf, n16, sink);
  return (int)hipGetLastError();
}

// ----------------------------------------------------------------------------- launchers
// Partial-kernel grid: balanced, the plan's share count bound; static, split fastest over
// (split, schedule head, sequence) (the plan keeps the count below 2^31).
static unsigned partial_grid(const LaunchArgs &la) {
  return la.balanced ? (unsigned)la.grid_wgs
                     : (unsigned)((int64_t)la.split_stride * la.sched_heads * la.batch);
}

static int launch_partial_any(const Plan &p, const LaunchArgs &la, void *stream,
                              const KernelEvents &ev, bool dbg) {
  const unsigned grid = partial_grid(la);
  const int kv = la.q4 ? 3 : la.fp8 ? 2 : la.int8 ? 1 : 0;
  switch (la.D) {
    case 128:
      if (kv == 3) return launch_partial_128_3(p, la, grid, stream, ev, dbg);
      if (kv == 2) return launch_partial_128_2(p, la, grid, stream, ev, dbg);
      if (kv == 1) return launch_partial_128_1(p, la, grid, stream, ev, dbg);
      return launch_partial_128_0(p, la, grid, stream, ev, dbg);
    case 256:
      if (kv == 3) return launch_partial_256_3(p, la, grid, stream, ev, dbg);
      if (kv == 2) return launch_partial_256_2(p, la, grid, stream, ev, dbg);
      if (kv == 1) return launch_partial_256_1(p, la, grid, stream, ev, dbg);
      return launch_partial_256_0(p, la, grid, stream, ev, dbg);
    case 192:  // f16 and fp8 (the plan refuses int8 and q4_0 at head_dim 192)
      if (kv == 2) return launch_partial_192_2(p, la, grid, stream, ev, dbg);
      return launch_partial_192_0(p, la, grid, stream, ev, dbg);
    default:
      if (kv == 3) return launch_partial_512_3(p, la, grid, stream, ev, dbg);
      if (kv == 2) return launch_partial_512_2(p, la, grid, stream, ev, dbg);
      if (kv == 1) return launch_partial_512_1(p, la, grid, stream, ev, dbg);
      return launch_partial_512_0(p, la, grid, stream, ev, dbg);
  }
}

int launch_partial(const Plan &p, const LaunchArgs &la, void *stream, void *start_event,
                   void *stop_event) {
  KernelEvents ev;
  ev.start = start_event;
  ev.stop = stop_event;
  return launch_partial_any(p, la, stream, ev, false);
}

int launch_gather(const Plan &p, const LaunchArgs &la, void *stream) {
  if (la.batch == 0) return 0;
  return launch_partial_any(p, la, stream, KernelEvents{}, true);
}

template <int D>
static void launch_merge_t(const Plan &p, const LaunchArgs &la, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)la.batch * la.T * la.Hq);
  switch (p.reducer) {
    case SKVD_REDUCER_DIRECT: merge_direct<D><<<rows, 64, 0, st>>>(la); break;
    case SKVD_REDUCER_COOPERATIVE: merge_rows<D, 1><<<rows, 64, 0, st>>>(la); break;
    case SKVD_REDUCER_MULTIPASS: {
      // Balanced: a schedule row (sequence, schedule head) meets on average at most
      // shares / rows + 1 partials; while that fits one wave's lanes, one wave per output row
      // (rounds of 64 cover the outliers) beats four.
      const int64_t sched_rows = (int64_t)la.batch * la.sched_heads;
      if (la.balanced && la.grid_wgs / sched_rows + 1 <= 64)
        merge_rows<D, 1><<<rows, 64, 0, st>>>(la);
      else
        merge_rows<D, kMergeWaves><<<rows, 64 * kMergeWaves, 0, st>>>(la);
      break;
    }
    case SKVD_REDUCER_HIERARCHICAL:
      merge_hier1<D><<<dim3(rows, p.hier_groups_cap), 64, 0, st>>>(la);
      merge_hier2<D><<<rows, 64 * kMergeWaves, 0, st>>>(la);
      break;
    default: break;
  }
}

int launch_merge(const Plan &p, const LaunchArgs &la, void *stream) {
  if (p.reducer == SKVD_REDUCER_NONE || la.batch == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  switch (la.D) {
    case 128: launch_merge_t<128>(p, la, st); break;
    case 192: launch_merge_t<192>(p, la, st); break;
    case 256: launch_merge_t<256>(p, la, st); break;
    default: launch_merge_t<512>(p, la, st); break;
  }
  return (int)hipGetLastError();
}

}  // namespace skvd
