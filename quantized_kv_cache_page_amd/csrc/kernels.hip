// HIP kernels for split-KV paged decode attention on gfx950 (CDNA4, wave64).
//
// Partial kernel: one wave64 workgroup per (split, KV head, sequence). A split is a run of
// 64-token blocks (1bit-MONSTER/engine issue #115, "Closing the remaining half of this
// issue": one producer partial per 64-token block; here a workgroup covers `bps` blocks).
// For each chunk of tokens it
//   1. gathers K and V rows through the page table straight into registers (16-byte loads;
//      the page id of a 16-token tile is wave-uniform when P >= 16),
//   2. computes the scores of the G*T query rows against 16-token tiles with the 16x16x32
//      f16 MFMA (query rows x tokens, contraction over head_dim; int8 K is widened to f16
//      exactly and its per-32 scale applied to each 32-element partial dot product in f32),
//   3. masks positions past the split, the sequence and (T > 1) the causal limit, and updates
//      the running max and sum in base 2 (online softmax),
//   4. accumulates P.V on the vector ALU in f32, lanes owning 8 head_dim elements of a V
//      row and reading the probabilities from LDS (int8 V: the scale is folded into p).
// It writes one partial (max, sum, f32 output) per query row, or o and lse directly when
// the plan has a single split.
//
// Merge kernels: the log-sum-exp reduction of the partials of one row,
//   M = max m_s, S = sum_s l_s 2^(m_s - M), o = sum_s 2^(m_s - M) o_s / S,
//   lse = (M + log2 S) ln 2,
// as direct (serial), cooperative (one lane per partial, <= 64), multipass (lane-strided,
// any count) and hierarchical (64 partials per workgroup, then a multipass over groups).
// Loop bounds come from kv_len on the device; the partial stride is the plan's capacity.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "skvd_internal.h"

namespace skvd {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
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

// LDS hand-off between the lanes of a one-wave workgroup: a wavefront-scope fence and wave
// barrier order the LDS accesses without waiting on outstanding global loads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 8 signed bytes -> 8 f16 (exact).
__device__ __forceinline__ half8 i8x8_to_h8(uint2v w) {
  half8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned word = i < 4 ? w.x : w.y;
    const int v = (int)(signed char)((word >> (8 * (i & 3))) & 0xff);
    r[i] = (_Float16)v;
  }
  return r;
}

__device__ __forceinline__ void h8_to_f(const half8 &h, float *f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ __forceinline__ void i8x8_to_f(uint2v w, float *f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned word = i < 4 ? w.x : w.y;
    f[i] = (float)(int)(signed char)((word >> (8 * (i & 3))) & 0xff);
  }
}

// ----------------------------------------------------------------------------- partial kernel
// D: head_dim (128/256). RB: 4-row quarters of the 16 MFMA rows in use (rows = G*T <= 4*RB).
// I8: int8 cache with f16 scales per 32 elements. FAST: page_size >= 16, so each 16-token
// tile lies in one page and its page id is wave-uniform.
template <int D, int RB, bool I8, bool FAST, int CH>
__global__ __launch_bounds__(64) void partial_kernel(LaunchArgs a) {
  // CH: tokens per chunk (16, 32 or 64). The K and V registers of a chunk (CH*D*4 bytes per
  // wave) bound how many waves fit on a SIMD; residency, not ALU work, sets the bandwidth.
  static_assert(CH == 16 || CH == 32 || CH == 64, "chunk");
  constexpr int NT = CH / 16;    // 16-token MFMA tiles per chunk
  constexpr int KS = D / 32;     // MFMA contraction steps of 32 head_dim elements
  constexpr int LPR = D / 8;     // P.V lanes per V row, 8 elements each
  constexpr int TPS = 64 / LPR;  // tokens per P.V step
  constexpr int NS = CH / TPS;   // P.V steps per chunk
  constexpr int RM = 4 * RB;     // query rows held (padded)
  using Vec = std::conditional_t<I8, uint2v, half8>;  // one lane's 8 elements of a row

  __shared__ float4v p_lds[CH][RB];  // probabilities of each chunk token, 4 rows per float4

  const int lane = threadIdx.x;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int T = a.T, G = a.G, R = G * T;
  const int L = clamp_len(a.kv_len[b], a.max_kv_len, a.status, a.debug);
  const int nblk = (L + 63) >> 6;
  const int blk0 = split * a.bps;
  if (!a.single && blk0 >= nblk) return;  // beyond this sequence: no partial is read
  const int tok0 = blk0 * 64;
  const int tok_end = min(min(blk0 + a.bps, nblk) * 64, L);
  const int P1 = (1 << a.page_shift) - 1;

  const char *kbase = (const char *)a.k;
  const char *vbase = (const char *)a.v;
  constexpr int ES = I8 ? 1 : 2;  // element bytes
  const _Float16 *ksc = (const _Float16 *)a.ks;
  const _Float16 *vsc = (const _Float16 *)a.vs;

  // Query rows as the MFMA A operand: lane holds row (lane & 15), elements 8*(lane>>4)..+7
  // of each 32-element contraction step.
  const int g4 = lane >> 4, c16 = lane & 15;
  half8 qa[KS];
  {
    const int r = c16;
    if (r < R) {
      const int t = r / G, hg = r - (r / G) * G;
      const _Float16 *qp = (const _Float16 *)a.q + ((int64_t)b * T + t) * a.q_tok_stride +
                           (int64_t)(kvh * G + hg) * a.q_head_stride + 8 * g4;
#pragma unroll
      for (int k = 0; k < KS; ++k) qa[k] = *(const half8 *)(qp + 32 * k);
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) qa[k] = (half8)(_Float16)0;
    }
  }
  // Rows of this lane's MFMA outputs: 4*g4 + e. Positions a row sees: j < L - T + t + 1.
  int nvis[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * g4 + e;
    const int n = r < R ? L - T + r / G + 1 : 0;
    nvis[e] = min(n, tok_end);
  }

  float m[4], lsum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { m[e] = kNegInf; lsum[e] = 0.f; }
  float acc[RM][8];
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[r][i] = 0.f;

  bool clamped_any = false;
  const int vlane_tok = lane / LPR, vlane_el = 8 * (lane % LPR);

  // Loads are branch-free: a token past the split is clamped to the split's last token
  // (a re-read of lines already fetched, masked out of the softmax), so every load of a chunk
  // is issued unconditionally and the in-order load counter can be waited on precisely.
  // FAST: the page of each 16-token tile is wave-uniform; a chunk's page ids are read from the
  // table through the constant address space (scalar loads, counted apart from the vector
  // loads) one chunk ahead of their use.
  const int last_tile = (tok_end - 1) & ~15;
  typedef const __attribute__((address_space(4))) int32_t *ctable_t;
  const ctable_t trow = (ctable_t)(a.table + (int64_t)b * a.table_stride);
  auto chunk_pages = [&](int c0, int *pg) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) pg[t] = trow[min(c0 + 16 * t, last_tile) >> a.page_shift];
  };
  auto clamp_page = [&](int pg, int64_t npages) __attribute__((always_inline)) -> int64_t {
    const bool bad = pg < 0 || pg >= npages;
    clamped_any |= bad;
    return bad ? (pg < 0 ? 0 : npages - 1) : (int64_t)pg;
  };

  Vec kb[NT][KS];
  float ks_tok[NT][KS];
  Vec vb[NS];
  float vs_tok[NS];

  // K rows of chunk c0 in the MFMA B-operand layout: tile t, lane (g4, c16) holds elements
  // 32k + 8*g4 .. +7 of token 16t + c16.
  auto load_k = [&](int c0, const int *pgs) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int jt = c0 + 16 * t;
      const int j = min(jt + c16, tok_end - 1);
      int64_t pg;
      if constexpr (FAST) {
        pg = clamp_page(pgs[t], a.num_k_pages);
      } else {
        bool cl;
        pg = lookup_page(a.table, a.table_stride, b, j, a.page_shift, a.num_k_pages, &cl);
        clamped_any |= cl;
      }
      const int64_t off = row_offset(pg, j & P1, kvh, a.page_stride, a.tok_stride, a.head_stride);
      const char *kp = kbase + (off + 8 * g4) * ES;
#pragma unroll
      for (int k = 0; k < KS; ++k) kb[t][k] = *(const Vec *)(kp + 32 * k * ES);
      if constexpr (I8) {
        const int64_t so = row_offset(pg, j & P1, kvh, a.s_page_stride, a.s_tok_stride,
                                      a.s_head_stride);
#pragma unroll
        for (int k = 0; k < KS; ++k) ks_tok[t][k] = (float)ksc[so + k];
      }
    }
  };
  // V rows of chunk c0 in the P.V layout: step s, lane holds elements vlane_el .. +7 of
  // token TPS*s + vlane_tok.
  auto load_v = [&](int c0, const int *pgs) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int js = c0 + TPS * s2;
      const int j = min(js + vlane_tok, tok_end - 1);
      int64_t pg;
      if constexpr (FAST) {
        pg = clamp_page(pgs[(TPS * s2) >> 4], a.num_v_pages);
      } else {
        bool cl;
        pg = lookup_page(a.table, a.table_stride, b, j, a.page_shift, a.num_v_pages, &cl);
        clamped_any |= cl;
      }
      const int64_t off = row_offset(pg, j & P1, kvh, a.page_stride, a.tok_stride, a.head_stride);
      vb[s2] = *(const Vec *)(vbase + (off + vlane_el) * ES);
      if constexpr (I8) {
        const int64_t so = row_offset(pg, j & P1, kvh, a.s_page_stride, a.s_tok_stride,
                                      a.s_head_stride);
        vs_tok[s2] = (float)vsc[so + vlane_el / 32];
      }
    }
  };

  int pg_cur[NT], pg_next[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) pg_cur[t] = pg_next[t] = 0;
  if (tok0 < tok_end) {
    if constexpr (FAST) chunk_pages(tok0, pg_cur);
    load_k(tok0, pg_cur);
    __builtin_amdgcn_sched_barrier(0);
    load_v(tok0, pg_cur);
    __builtin_amdgcn_sched_barrier(0);
  }
  // One chunk: scores of the chunk's K (loaded one step ahead), prefetch of the next K,
  // softmax, P.V with the chunk's V, prefetch of the next V. The first call is peeled off
  // the loop so that the loop is entered with the same load order as its back edge (K
  // before V) and the in-order load counter is waited on for K alone at the loop top.
  auto chunk = [&](int c0) __attribute__((always_inline)) {
    const int c1 = c0 + CH;
    if constexpr (FAST) chunk_pages(c1, pg_next);
    // ---- scores: S[t] = rows x 16 tokens of tile t (lane: token c16, rows 4*g4 + e)
    // The MFMA chains run for every tile, also the ones past the split (their K is a clamped
    // re-read and their scores are masked): a branch between an MFMA and the reads of its
    // result let the compiler's wait-state insertion miss the taken path.
    float4v S[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      S[t] = (float4v)0.f;
      if constexpr (I8) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          float4v part = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], i8x8_to_h8(kb[t][k]),
                                                                (float4v)0.f, 0, 0, 0);
          S[t] += part * ks_tok[t][k];
        }
      } else {
#pragma unroll
        for (int k = 0; k < KS; ++k)
          S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], kb[t][k], S[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- prefetch the next chunk's K while this chunk's softmax and P.V run (past the end
    // of the split this re-reads the last token: cached, and never used)
    load_k(c1, pg_next);
    __builtin_amdgcn_sched_barrier(0);

    // ---- mask, online softmax (base 2)
    float alpha[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cmax = kNegInf;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int j = c0 + 16 * t + c16;
        const float sc = j < nvis[e] ? S[t][e] * a.scale_log2 : kNegInf;
        S[t][e] = sc;
        cmax = fmaxf(cmax, sc);
      }
      cmax = row16_max(cmax);
      const float mnew = fmaxf(m[e], cmax);
      const bool dead = mnew == kNegInf;
      alpha[e] = dead ? 1.f : fast_exp2(m[e] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float p = dead ? 0.f : fast_exp2(S[t][e] - mnew);
        S[t][e] = p;
        ps += p;
      }
      lsum[e] = lsum[e] * alpha[e] + ps;
      m[e] = mnew;
    }
    if (g4 < RB) {
#pragma unroll
      for (int t = 0; t < NT; ++t) p_lds[16 * t + c16][g4] = S[t];
    }
    float al[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) al[r] = readlane_f(alpha[r & 3], 16 * (r >> 2));
    wave_sync();

    // ---- P.V
    bool rescale = false;
#pragma unroll
    for (int r = 0; r < RM; ++r) rescale |= al[r] != 1.f;
    if (rescale) {
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] *= al[r];
    }
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int tk = TPS * s2 + vlane_tok;
      float4v pr[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) pr[q] = p_lds[tk][q];
      float v[8];
      if constexpr (I8) {
        i8x8_to_f(vb[s2], v);
#pragma unroll
        for (int q = 0; q < RB; ++q) pr[q] *= vs_tok[s2];
      } else {
        h8_to_f(vb[s2], v);
      }
#pragma unroll
      for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[r][i] = fmaf(pr[r >> 2][r & 3], v[i], acc[r][i]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- prefetch the next chunk's V while the next chunk's scores run
    load_v(c1, pg_next);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) pg_cur[t] = pg_next[t];
    wave_sync();
  };
  if (tok0 < tok_end) {
    chunk(tok0);
    for (int c0 = tok0 + CH; c0 < tok_end; c0 += CH) chunk(c0);
  }
  if (a.debug && clamped_any) atomicOr(a.status, (unsigned)SKVD_STATUS_PAGE_CLAMPED);

  // ---- per-row max and sum (wave-uniform)
  float mr[RM], lr[RM];
#pragma unroll
  for (int e = 0; e < 4; ++e) lsum[e] = row16_sum(lsum[e]);
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    mr[r] = readlane_f(m[r & 3], 16 * (r >> 2));
    lr[r] = readlane_f(lsum[r & 3], 16 * (r >> 2));
  }
  // ---- sum the token groups of the P.V lanes: lanes l, l^LPR, ... share head_dim elements
#pragma unroll
  for (int r = 0; r < RM; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = acc[r][i];
      if constexpr (TPS >= 4) x += __shfl_xor(x, 16);
      if constexpr (TPS >= 2) x += __shfl_xor(x, 32);
      acc[r][i] = x;
    }
  if (lane >= LPR) return;

  const int Hq = a.Hq;
#pragma unroll
  for (int r = 0; r < RM; ++r) {
    if (r >= R) continue;
    const int t = r / G, hg = r - (r / G) * G;
    const int64_t row = ((int64_t)b * T + t) * Hq + kvh * G + hg;
    if (a.single) {
      const float l = lr[r];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      half8 out;
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = (_Float16)(acc[r][i] * inv);
      *(half8 *)((_Float16 *)a.o + row * D + vlane_el) = out;
      if (a.lse && lane == 0) a.lse[row] = l > 0.f ? (mr[r] + __log2f(l)) * kLn2 : kNegInf;
    } else {
      float *dst = a.ws_o + (row * a.splits_cap + split) * D + vlane_el;
      *(float4v *)dst = float4v{acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
      *(float4v *)(dst + 4) = float4v{acc[r][4], acc[r][5], acc[r][6], acc[r][7]};
      if (lane == 0) {
        float *ml = a.ws_ml + (row * a.splits_cap + split) * 2;
        ml[0] = mr[r];
        ml[1] = lr[r];
      }
    }
  }
}

// ----------------------------------------------------------------------------- merge kernels
__device__ __forceinline__ void row_coords(const LaunchArgs &a, int64_t row, int *b) {
  *b = (int)(row / ((int64_t)a.T * a.Hq));
}

__device__ __forceinline__ int splits_of(const LaunchArgs &a, int b) {
  const int L = clamp_len(a.kv_len[b], a.max_kv_len, a.status, 0);
  const int nblk = (L + 63) >> 6;
  return (nblk + a.bps - 1) / a.bps;
}

// Final write of one row from a normalized accumulator.
template <int D>
__device__ __forceinline__ void write_row(const LaunchArgs &a, int64_t row, const float *acc,
                                          float M, float S) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
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

// Direct: every lane walks all n partials (few partials).
template <int D>
__global__ __launch_bounds__(64) void merge_direct(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  int b;
  row_coords(a, row, &b);
  const int n = splits_of(a, b);
  const float *ml = a.ws_ml + row * a.splits_cap * 2;
  const float *po = a.ws_o + row * a.splits_cap * D + PER * threadIdx.x;
  float M = kNegInf;
  for (int s = 0; s < n; ++s) M = fmaxf(M, ml[2 * s]);
  float S = 0.f, acc[PER] = {};
  for (int s = 0; s < n; ++s) {
    const float w = part_weight(ml[2 * s], M);
    S += w * ml[2 * s + 1];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, po[(int64_t)s * D + i], acc[i]);
  }
  write_row<D>(a, row, acc, M, S);
}

// Lane-strided merge of n partials at (ml, po) with stride D between partials. Produces the
// row max M, the sum S relative to M, and the unnormalized accumulator. Cooperative when
// n <= 64 (one lane per partial, one pass); multipass otherwise.
template <int D>
__device__ __forceinline__ void merge_span(const float *ml, const float *po, int n, float *M_out,
                                           float *S_out, float *acc) {
  constexpr int PER = D / 64;
  __shared__ float w_lds[64];
  const int lane = threadIdx.x;
  // pass 1: running (max, sum) per lane over partials lane, lane+64, ...
  float mloc = kNegInf, sloc = 0.f;
  for (int s = lane; s < n; s += 64) {
    const float ms = ml[2 * s], ls = ml[2 * s + 1];
    const float mn = fmaxf(mloc, ms);
    if (mn != kNegInf) {
      sloc = sloc * part_weight(mloc, mn) + ls * part_weight(ms, mn);
      mloc = mn;
    }
  }
  const float M = wave_max(mloc);
  const float S = wave_sum(M == kNegInf ? 0.f : sloc * part_weight(mloc, M));
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  // pass 2: weights of 64 partials at a time through LDS, lanes over head_dim
  for (int base = 0; base < n; base += 64) {
    const int s = base + lane;
    w_lds[lane] = (s < n && M != kNegInf) ? part_weight(ml[2 * s], M) : 0.f;
    __syncthreads();
    const int cnt = min(64, n - base);
    for (int i2 = 0; i2 < cnt; ++i2) {
      const float w = w_lds[i2];
      const float *src = po + (int64_t)(base + i2) * D + PER * lane;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, src[i], acc[i]);
    }
    __syncthreads();
  }
  *M_out = M;
  *S_out = S;
}

// Cooperative / multipass: one wave per row over all of the row's partials.
template <int D>
__global__ __launch_bounds__(64) void merge_rows(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  int b;
  row_coords(a, row, &b);
  const int n = splits_of(a, b);
  float M, S, acc[PER];
  merge_span<D>(a.ws_ml + row * a.splits_cap * 2, a.ws_o + row * a.splits_cap * D, n, &M, &S,
                acc);
  write_row<D>(a, row, acc, M, S);
}

// Hierarchical level 1: workgroup (row, g) merges partials 64g .. 64g+63 into one
// unnormalized partial of the same form.
template <int D>
__global__ __launch_bounds__(64) void merge_hier1(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  const int g = blockIdx.y;
  int b;
  row_coords(a, row, &b);
  const int n = splits_of(a, b);
  const int s0 = g * kHierGroup;
  if (s0 >= n) return;
  const int cnt = min(kHierGroup, n - s0);
  float M, S, acc[PER];
  merge_span<D>(a.ws_ml + (row * a.splits_cap + s0) * 2, a.ws_o + (row * a.splits_cap + s0) * D,
                cnt, &M, &S, acc);
  float *dst = a.ws_ho + (row * a.hier_groups_cap + g) * D + PER * threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[i] = acc[i];
  if (threadIdx.x == 0) {
    float *hm = a.ws_hml + (row * a.hier_groups_cap + g) * 2;
    hm[0] = M;
    hm[1] = S;
  }
}

// Hierarchical level 2: multipass over the row's groups.
template <int D>
__global__ __launch_bounds__(64) void merge_hier2(LaunchArgs a) {
  constexpr int PER = D / 64;
  const int64_t row = blockIdx.x;
  int b;
  row_coords(a, row, &b);
  const int n = splits_of(a, b);
  const int ng = (n + kHierGroup - 1) / kHierGroup;
  float M, S, acc[PER];
  merge_span<D>(a.ws_hml + row * a.hier_groups_cap * 2, a.ws_ho + row * a.hier_groups_cap * D,
                ng, &M, &S, acc);
  write_row<D>(a, row, acc, M, S);
}

// ----------------------------------------------------------------------------- gather (test aid)
template <int D, bool I8>
__global__ __launch_bounds__(64) void gather_kernel(LaunchArgs a, int max_len, char *dk, char *dv,
                                                    _Float16 *dks, _Float16 *dvs) {
  constexpr int ES = I8 ? 1 : 2;
  const int j = blockIdx.x * 64 + threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(a.kv_len[b], a.max_kv_len, a.status, a.debug);
  if (j >= L || j >= max_len) return;
  const int P1 = (1 << a.page_shift) - 1;
  bool ck, cv;
  const int64_t pk = lookup_page(a.table, a.table_stride, b, j, a.page_shift, a.num_k_pages, &ck);
  const int64_t pv = lookup_page(a.table, a.table_stride, b, j, a.page_shift, a.num_v_pages, &cv);
  if (a.debug && (ck || cv)) atomicOr(a.status, (unsigned)SKVD_STATUS_PAGE_CLAMPED);
  const int64_t ok = row_offset(pk, j & P1, kvh, a.page_stride, a.tok_stride, a.head_stride);
  const int64_t ov = row_offset(pv, j & P1, kvh, a.page_stride, a.tok_stride, a.head_stride);
  const int64_t dst = (((int64_t)b * max_len + j) * a.Hkv + kvh);
  const char *ks = (const char *)a.k + ok * ES;
  const char *vs = (const char *)a.v + ov * ES;
  for (int i = 0; i < D * ES; i += 4) {
    *(unsigned *)(dk + dst * D * ES + i) = *(const unsigned *)(ks + i);
    *(unsigned *)(dv + dst * D * ES + i) = *(const unsigned *)(vs + i);
  }
  if constexpr (I8) {
    const int64_t sk = row_offset(pk, j & P1, kvh, a.s_page_stride, a.s_tok_stride, a.s_head_stride);
    const int64_t sv = row_offset(pv, j & P1, kvh, a.s_page_stride, a.s_tok_stride, a.s_head_stride);
    for (int g = 0; g < D / 32; ++g) {
      dks[dst * (D / 32) + g] = ((const _Float16 *)a.ks)[sk + g];
      dvs[dst * (D / 32) + g] = ((const _Float16 *)a.vs)[sv + g];
    }
  }
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
// Tokens per chunk for each variant, chosen so that the kernel keeps at most 168 registers
// (three waves per SIMD) where the row count allows.
template <int D, int RB>
constexpr int chunk_tokens() {
  return D == 128 ? (RB <= 2 ? 32 : 16) : 16;
}

template <int D, int RB, bool I8>
static void launch_partial_t(const LaunchArgs &la, dim3 grid, hipStream_t st, bool fast) {
  constexpr int CH = chunk_tokens<D, RB>();
  if (fast)
    partial_kernel<D, RB, I8, true, CH><<<grid, 64, 0, st>>>(la);
  else
    partial_kernel<D, RB, I8, false, CH><<<grid, 64, 0, st>>>(la);
}

template <int D, bool I8>
static void launch_partial_rb(const Plan &p, const LaunchArgs &la, dim3 grid, hipStream_t st) {
  const bool fast = p.prm.page_size >= 16;
  switch (p.row_blocks) {
    case 1: launch_partial_t<D, 1, I8>(la, grid, st, fast); break;
    case 2: launch_partial_t<D, 2, I8>(la, grid, st, fast); break;
    default: launch_partial_t<D, 4, I8>(la, grid, st, fast); break;
  }
}

int launch_partial(const Plan &p, const LaunchArgs &la, void *stream) {
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(p.splits_cap, la.Hkv, la.batch);
  const bool i8 = la.int8;
  if (la.D == 128) {
    if (i8) launch_partial_rb<128, true>(p, la, grid, st);
    else launch_partial_rb<128, false>(p, la, grid, st);
  } else {
    if (i8) launch_partial_rb<256, true>(p, la, grid, st);
    else launch_partial_rb<256, false>(p, la, grid, st);
  }
  return (int)hipGetLastError();
}

template <int D>
static void launch_merge_t(const Plan &p, const LaunchArgs &la, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)la.batch * la.T * la.Hq);
  switch (p.reducer) {
    case SKVD_REDUCER_DIRECT: merge_direct<D><<<rows, 64, 0, st>>>(la); break;
    case SKVD_REDUCER_COOPERATIVE:
    case SKVD_REDUCER_MULTIPASS: merge_rows<D><<<rows, 64, 0, st>>>(la); break;
    case SKVD_REDUCER_HIERARCHICAL:
      merge_hier1<D><<<dim3(rows, p.hier_groups_cap), 64, 0, st>>>(la);
      merge_hier2<D><<<rows, 64, 0, st>>>(la);
      break;
    default: break;
  }
}

int launch_merge(const Plan &p, const LaunchArgs &la, void *stream) {
  if (p.reducer == SKVD_REDUCER_NONE || la.batch == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  if (la.D == 128) launch_merge_t<128>(p, la, st);
  else launch_merge_t<256>(p, la, st);
  return (int)hipGetLastError();
}

int launch_gather(const Plan &p, const LaunchArgs &la, int max_len, void *dk, void *dv, void *dks,
                  void *dvs, void *stream) {
  hipStream_t st = (hipStream_t)stream;
  dim3 grid((max_len + 63) / 64, la.Hkv, la.batch);
  if (grid.x == 0 || la.batch == 0) return 0;
  char *k = (char *)dk, *v = (char *)dv;
  _Float16 *ks = (_Float16 *)dks, *vs = (_Float16 *)dvs;
  if (la.D == 128) {
    if (la.int8) gather_kernel<128, true><<<grid, 64, 0, st>>>(la, max_len, k, v, ks, vs);
    else gather_kernel<128, false><<<grid, 64, 0, st>>>(la, max_len, k, v, ks, vs);
  } else {
    if (la.int8) gather_kernel<256, true><<<grid, 64, 0, st>>>(la, max_len, k, v, ks, vs);
    else gather_kernel<256, false><<<grid, 64, 0, st>>>(la, max_len, k, v, ks, vs);
  }
  (void)p;
  return (int)hipGetLastError();
}

}  // namespace skvd
