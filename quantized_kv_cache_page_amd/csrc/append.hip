// Append kernel: new K/V rows into the paged cache, f16 verbatim, or int8, fp8 or q4_0
// quantized on write.
//
// The slot of new token i is (page_table[b][j / P], j % P) for b = batch_idx[i], j =
// positions[i]: the address the decode reads. Each lane owns 8 consecutive head_dim elements of
// one (token, KV head) row, in K and in V: one 16-byte load of each and one store of each (16
// bytes of f16, or 8 bytes of int8 codes), so a row of D elements is D/8 lanes and a wave covers
// 64*8/D rows; consecutive rows of a [N, Hkv, D] input are consecutive memory, so a wave's loads
// are one contiguous run. The kernel is a pure stream (read the new rows once, write the slots
// once, both non-temporal: neither is read again by this kernel, and the decode that reads the
// slots later comes after many other launches); it is bound by HBM, or by launch latency for a
// decode step's handful of tokens.
//
// int8 (one f16 scale per 32 elements; AMD-Ecosystem/flashinfer PR #397 names append as the op
// that writes the cache, 1bit-MONSTER/engine issue #115 comment "Fixed" names the q8_0-style KV
// type): the four lanes of a 32-element group take the group's largest magnitude with two
// quad-permute DPP steps, then
//     s = f16(amax / 127)                 f32 quotient, rounded once to f16 (nearest even)
//     c = clip(rint(x / s), -127, 127)    f32 quotient, nearest even; s = 0 gives c = 0
// and the group's first lane writes s. The scale's quotient is an IEEE-correctly rounded f32
// division; the codes take the correctly rounded quotient's decision through a reciprocal
// multiply checked against the rounding boundary (code_of), so they are those of any correctly
// rounded f32 evaluation of the same rule.
//
// fp8 (OCP E4M3 bytes with one f32 scale s per tensor, read from device memory; the
// AMD-Ecosystem/flashinfer PR #397 commit messages name fp8 caches with per-tensor k_scale and
// v_scale): each element stores the E4M3 value nearest to clip(x / s, -448, 448), x / s the
// correctly rounded f32 quotient, ties to the even mantissa; a NaN quotient stores 0.
#include <hip/hip_runtime.h>

#include "skvd_internal.h"

namespace skvd {
namespace {

typedef _Float16 half8a __attribute__((ext_vector_type(8)));
typedef unsigned uint2a __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// The 8 codes of one lane and the f16 scale of its 32-element group (all four lanes of the
// group run this together: the DPP steps read within the lane quad).
//
// Codes: rint(x / s) with x / s the correctly rounded f32 quotient, clipped to [-127, 127]. The
// product q = x * rcp(s) (rcp to 1 ulp) is within 1.5 ulp-relative of x / s, i.e. within 6e-5 of
// it for |x / s| < 256 (always: s is max|x| / 127 rounded to f16), so rint(q) is the quotient's
// integer unless q lies within 2^-12 of a half-integer. Lanes holding such an element (rare)
// redo it with the division, so the decision is that of the correctly rounded quotient while
// nearly every element costs one multiply.
__device__ __forceinline__ uint2a quantize8(half8a x, _Float16 *scale) {
  constexpr float kNear = 0.5f - 0x1p-12f;
  // 1.5 * 2^23: adding it to a value of magnitude below 2^22 rounds that value to an integer
  // (nearest even) held in the low mantissa bits, two's complement in the low byte
  constexpr float kMagic = 12582912.0f;
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)x[e];
    amax = fmaxf(amax, fabsf(f[e]));
  }
  amax = fmaxf(amax, quad_dpp<0xB1>(amax));  // quad_perm [1,0,3,2]: lane xor 1
  amax = fmaxf(amax, quad_dpp<0x4E>(amax));  // quad_perm [2,3,0,1]: lane xor 2
  const _Float16 sh = (_Float16)(amax / 127.0f);
  const float s = (float)sh;
  const float rs = __builtin_amdgcn_rcpf(s);
  // clip(rint(q), -127, 127) = rint(clip(q, -127, 127)): clamp, then one add rounds and the low
  // byte is the code; q - rint(q) from the same add flags the elements near a half-integer
  unsigned c[8];
  bool near = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = f[e] * rs;
    const float qc = __builtin_amdgcn_fmed3f(q, -127.0f, 127.0f);
    const float t = qc + kMagic;
    // a NaN quotient (a NaN element, or an infinite one over an infinite scale) stores 0
    c[e] = q != q ? 0u : __float_as_uint(t) & 0xFFu;
    near |= fabsf(qc - (t - kMagic)) > kNear;
  }
  if (near && s > 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qc = __builtin_amdgcn_fmed3f(f[e] * rs, -127.0f, 127.0f);
      if (fabsf(qc - rintf(qc)) > kNear && f[e] == f[e])
        c[e] = (unsigned)(int)__builtin_amdgcn_fmed3f(rintf(f[e] / s), -127.0f, 127.0f) & 0xFFu;
    }
  }
  const unsigned keep = s > 0.0f ? 0xFFFFFFFFu : 0u;  // s = 0: every code 0
  *scale = sh;
  uint2a r;
  r[0] = (c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24) & keep;
  r[1] = (c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24) & keep;
  return r;
}

// E4M3 byte of one f32 value q (see above). Below 2^-6 the E4M3 grid is 2^-9 (subnormals, and
// 2^-6 itself as 8 steps), so the code is rint(|q| * 512); above, the f32 bits are rounded to
// three mantissa bits (nearest, ties to even, by adding 0x7FFFF plus the kept lowest bit) and
// the exponent is rebased from f32's bias 127 to E4M3's 7. |q| <= 448 keeps the code <= 0x7E.
__device__ __forceinline__ unsigned e4m3_of(float q) {
  const unsigned sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float m = fminf(fabsf(q), 448.0f);
  unsigned code;
  if (m < 0x1p-6f) {
    code = (unsigned)rintf(m * 512.0f);
  } else {
    const unsigned b = __float_as_uint(m);
    code = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return q != q ? 0u : (sign | code);
}

// True when q lies within 4 ulps of a point where the E4M3 rounding changes (a midpoint
// between neighbouring values): above 2^-6 the 20 f32 mantissa bits below the kept three are
// within 4 of 0x80000 (the bits of q itself: sign and exponent are masked off; a q beyond 448
// that tests near only costs the slow path). Below 2^-6, where the grid is 2^-9, every nonzero q
// counts as near. Binade edges are E4M3 values themselves, and 448 is one, so the clip adds no
// other decision point.
__device__ __forceinline__ bool e4m3_near_tie(float q) {
  return (fabsf(q) < 0x1p-6f && q != 0.0f) || (__float_as_uint(q) & 0xFFFFFu) - 0x7FFFCu <= 8u;
}

// The 8 E4M3 codes of one lane's elements over the tensor scale s, as if from the correctly
// rounded quotients x / s. The product q = x * rcp(s) (rcp to 1 ulp) is within 2 ulps of x / s,
// so away from the rounding midpoints its code is the quotient's: the hardware conversion
// (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950, nearest even) of q clamped to +-448 gives it, four
// bytes per two instructions. A lane with an element near a midpoint (or with s or 1/s outside
// the normal range) recomputes its codes in software from the division for those elements.
__device__ __forceinline__ uint2a quantize_fp8(half8a x, float s) {
  const float r = __builtin_amdgcn_rcpf(s);
  const bool normal = s >= 0x1p-125f && s <= 0x1p125f;
  float f[8], q[8];
  bool near = !normal;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)x[e];
    q[e] = f[e] * r;
    // (a NaN quotient takes the software path, which stores 0: the hardware clamp would not)
    near |= e4m3_near_tie(q[e]) || q[e] != q[e];
  }
  uint2a w;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float *qk = q + 4 * k;
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(qk[0], -448.0f, 448.0f),
                                            __builtin_amdgcn_fmed3f(qk[1], -448.0f, 448.0f), 0,
                                            false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(qk[2], -448.0f, 448.0f),
                                        __builtin_amdgcn_fmed3f(qk[3], -448.0f, 448.0f), v, true);
    w[k] = (unsigned)v;
  }
  if (near) {
    unsigned c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      c[e] = e4m3_of(!normal || e4m3_near_tie(q[e]) ? f[e] / s : q[e]);
    w[0] = c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24;
    w[1] = c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24;
  }
  return w;
}

template <int CTRL>
__device__ __forceinline__ unsigned quad_dpp_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// q4_0 (the published ggml q4_0 rule; the cache type is named beside q8_0 in 1bit-MONSTER/engine
// issue #115, comment "Closing the remaining half of this issue"): lane r of a group's quad holds
// its elements 8r .. 8r + 7. The group's extreme m -- largest magnitude, the first in element
// order on a tie, NaN excluded, +0 when every magnitude is 0 -- comes from a quad max over keys
// (f16 magnitude bits, then 31 - index, then the sign bit). Then, in f32 with no fused
// operations (the rule rounds the product and the sum separately):
//     d = m / -8,  r = 1 / d (0 if d = 0),  c = min(15, trunc(x * r + 8.5))  (NaN -> 8)
// and the scale stored is f16(d). Lanes 0 and 1 of the quad return the group's code bytes
// 8r .. 8r + 7 (codes 8r + i in the low nibbles, 16 + 8r + i from lane r + 2 in the high ones).
__device__ __forceinline__ uint2a quantize_q4(half8a x, int r, _Float16 *scale) {
#pragma clang fp contract(off)
  unsigned key = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // (bit_cast of a vector element would cast element 0: copy the element out first)
    const _Float16 xe = x[e];
    const unsigned h = __builtin_bit_cast(unsigned short, xe);
    const unsigned mag = h & 0x7FFFu;
    const unsigned k = mag > 0x7C00u ? 0u : (mag << 6) | ((31u - (8u * r + e)) << 1) | (h >> 15);
    key = max(key, k);
  }
  key = max(key, quad_dpp_u<0xB1>(key));  // quad_perm [1,0,3,2]: lane xor 1
  key = max(key, quad_dpp_u<0x4E>(key));  // quad_perm [2,3,0,1]: lane xor 2
  const unsigned mag = key >> 6;
  const float amax = (float)__builtin_bit_cast(_Float16, (unsigned short)mag);
  const float m = mag == 0 ? 0.0f : (key & 1u ? -amax : amax);
  const float d = m / -8.0f;
  const float rd = d != 0.0f ? 1.0f / d : 0.0f;
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float xr = (float)x[e] * rd;
    const float t = xr + 8.5f;
    const unsigned c = t != t ? 8u : (unsigned)min(15, (int)t);
    w[e >> 2] |= c << (8 * (e & 3));
  }
  // lanes 0, 1 take the high nibbles from lanes 2, 3
  const unsigned h0 = quad_dpp_u<0x4E>(w[0]), h1 = quad_dpp_u<0x4E>(w[1]);
  *scale = (_Float16)d;
  uint2a out;
  out[0] = w[0] | (h0 << 4);
  out[1] = w[1] | (h1 << 4);
  return out;
}

// KV: 0 f16, 1 int8 with per-32 f16 scales, 2 fp8 with the tensor scale tscale, 3 q4_0.
template <int D, int KV>
__device__ __forceinline__ void store_row(const AppendLaunch &a, half8a x, void *pool,
                                          void *scales, float tscale, int64_t page, int slot,
                                          int kvh, int part) {
  const int64_t row = page * a.page_stride + (int64_t)slot * a.tok_stride +
                      (int64_t)kvh * a.head_stride;
  const int64_t off = row + part * 8;
  if constexpr (KV == 3) {
    _Float16 sh;
    const uint2a codes = quantize_q4(x, part & 3, &sh);
    if ((part & 3) < 2)
      __builtin_nontemporal_store(
          codes, (uint2a *)((uint8_t *)pool + row + 16 * (part >> 2) + 8 * (part & 3)));
    if ((part & 3) == 0) {
      const int64_t soff = page * a.s_page_stride + (int64_t)slot * a.s_tok_stride +
                           (int64_t)kvh * a.s_head_stride + (part >> 2);
      ((_Float16 *)scales)[soff] = sh;
    }
  } else if constexpr (KV == 0) {
    __builtin_nontemporal_store(x, (half8a *)((_Float16 *)pool + off));
  } else if constexpr (KV == 2) {
    __builtin_nontemporal_store(quantize_fp8(x, tscale), (uint2a *)((int8_t *)pool + off));
  } else {
    _Float16 sh;
    const uint2a codes = quantize8(x, &sh);
    __builtin_nontemporal_store(codes, (uint2a *)((int8_t *)pool + off));
    if ((part & 3) == 0) {
      const int64_t soff = page * a.s_page_stride + (int64_t)slot * a.s_tok_stride +
                           (int64_t)kvh * a.s_head_stride + (part >> 2);
      ((_Float16 *)scales)[soff] = sh;
    }
  }
}

// A lane owns one 8-element part of one KV-head row and serves kTokensPerLane tokens that are
// tok_step apart (the grid holds a whole number of tokens' lanes, so a lane keeps its head and
// part; one division at entry). All of a round's loads -- new K and V rows, sequence indices,
// positions -- are issued together, then all of its page-table reads, then the quantization and
// stores: two dependent memory round trips per kTokensPerLane tokens. Loads are branch-free
// (token indices clamped into the batch, invalid tokens masked), so nothing waits early.
constexpr int kTokensPerLane = kAppendTokensPerLane;

template <int D, int KV>
__global__ __launch_bounds__(256) void append_kernel(AppendLaunch a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int U = kTokensPerLane;
  const unsigned gid = blockIdx.x * 256u + threadIdx.x;
  const unsigned lpt = (unsigned)a.lanes_per_token;
  const int tok0 = (int)(gid / lpt);
  if (tok0 >= a.tok_step) return;
  const unsigned rem = gid - (unsigned)tok0 * lpt;
  const int kvh = (int)(rem / kLanesPerRow);   // lanes of one row (and quad) share every branch
  const int part = (int)(rem % kLanesPerRow);
  const int64_t head_off = (int64_t)kvh * a.new_head_stride + part * 8;
  const _Float16 *kn = (const _Float16 *)a.k_new;
  const _Float16 *vn = (const _Float16 *)a.v_new;
  const int slot_mask = (1 << a.page_shift) - 1;
  const int last = a.num_tokens - 1;
  // fp8: the tensor scales (scalar loads, once)
  const float ksc = KV == 2 ? *(const float *)a.ks : 0.0f;
  const float vsc = KV == 2 ? *(const float *)a.vs : 0.0f;
  for (int base = tok0; base < a.num_tokens; base += U * a.tok_step) {
    half8a xk[U], xv[U];
    int b[U], j[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(base + u * a.tok_step, last);
      const int64_t src = (int64_t)t * a.new_tok_stride + head_off;
      xk[u] = __builtin_nontemporal_load((const half8a *)(kn + src));
      xv[u] = __builtin_nontemporal_load((const half8a *)(vn + src));
      b[u] = a.batch_idx[t];
      j[u] = a.positions[t];
    }
    int64_t page[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = base + u * a.tok_step <= last && b[u] >= 0 && b[u] < a.batch &&
                      j[u] >= 0 && j[u] < a.max_len;
      const int bb = ok ? b[u] : 0, jj = ok ? j[u] : 0;  // row 0, entry 0 exist (batch >= 1)
      const int64_t pg = a.table[(int64_t)bb * a.table_stride + (jj >> a.page_shift)];
      page[u] = ok ? pg : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (page[u] < 0) continue;
      const int slot = j[u] & slot_mask;
      if (page[u] < a.num_k_pages)
        store_row<D, KV>(a, xk[u], a.k, a.ks, ksc, page[u], slot, kvh, part);
      if (page[u] < a.num_v_pages)
        store_row<D, KV>(a, xv[u], a.v, a.vs, vsc, page[u], slot, kvh, part);
    }
  }
}

template <int D>
void launch_d(const AppendLaunch &a, hipStream_t st) {
  if (a.q4) append_kernel<D, 3><<<a.blocks, 256, 0, st>>>(a);
  else if (a.fp8) append_kernel<D, 2><<<a.blocks, 256, 0, st>>>(a);
  else if (a.int8) append_kernel<D, 1><<<a.blocks, 256, 0, st>>>(a);
  else append_kernel<D, 0><<<a.blocks, 256, 0, st>>>(a);
}

}  // namespace

int launch_append(AppendLaunch a, void *stream) {
  if (a.rows == 0 || a.batch == 0) return 0;  // nothing to write (and no table row to read)
  // Grid: a whole number of tokens' lanes (so a lane keeps its head and part while it strides),
  // each lane serving up to kTokensPerLane tokens per round; at most one round of resident
  // 256-lane workgroups (int8: 77 registers -> 6 waves per SIMD; fp8: 69 -> 7; f16: 58 -> 8),
  // fewer for a small append.
  a.lanes_per_token = a.Hkv * a.D / 8;
  int64_t x = a.lanes_per_token, y = 256;
  while (y) {
    const int64_t t = x % y;
    x = y;
    y = t;
  }
  const int64_t g0 = a.lanes_per_token / x;  // workgroups per whole number of tokens
  const int64_t toks = (a.num_tokens + kTokensPerLane - 1) / kTokensPerLane;
  const int64_t want = (toks * a.lanes_per_token + 255) / 256;
  const int64_t cap = (a.fp8 ? 7LL : a.int8 || a.q4 ? 6LL : 8LL) * a.num_cus;
  int64_t blocks = want < cap ? want : cap;
  blocks = (blocks + g0 - 1) / g0 * g0;
  a.blocks = (unsigned)blocks;
  a.tok_step = (int)(blocks * 256 / a.lanes_per_token);
  hipStream_t st = (hipStream_t)stream;
  switch (a.D) {
    case 128: launch_d<128>(a, st); break;
    case 192: launch_d<192>(a, st); break;
    case 256: launch_d<256>(a, st); break;
    default: launch_d<512>(a, st); break;
  }
  return (int)hipGetLastError();
}

}  // namespace skvd
