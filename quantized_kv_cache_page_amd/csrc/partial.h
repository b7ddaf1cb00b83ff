// The decode's partial kernel (template) and its launch dispatch, instantiated per head_dim and
// cache format in partial_<D>_<format>.hip.
//
// Workgroups of one wave per (KV head, row tile) served, each covering a run of 64-token blocks
// of one or more (sequence, schedule head) rows (1bit-MONSTER/engine issue #115, "Closing the
// remaining half of this issue": one producer partial per 64-token block; here a workgroup
// covers a split of `bps` blocks, or an equal share of the batch's blocks under the balanced
// schedule). For each chunk of tokens it
//   1. gathers K and V rows through the page table straight into registers (16-byte loads;
//      the page id of a 16-token tile is wave-uniform when P >= 16),
//   2. computes the scores of up to 16 query rows per wave against 16-token tiles with the
//      16x16x32 f16 MFMA (query rows x tokens, contraction over head_dim). int8 K: the bytes of
//      a token are redistributed across the four lane groups so that each MFMA step contracts
//      one 32-element scale group, widened exactly to f16; the step's f32 result is multiplied
//      by that token's group scale (the exact int8 * scale value, no rounding of the product).
//      fp8 K is widened exactly to value * 2^-8, its tensor scale and the 2^8 going into the
//      score scale,
//   3. masks positions past the split, the sequence and (T > 1) the causal limit, and updates
//      the running max and sum in base 2 (online softmax),
//   4. accumulates P.V in f32: for one query-row quarter as f16 pair dot products from the V
//      registers (int8 V: the scale is folded into the probabilities; fp8 V: the tensor scale
//      is applied to the output), otherwise on the MFMA from an LDS copy of V.
// It writes one partial (max, sum, f32 output) per query row, or o and lse directly when the
// plan has a single split.
//
// More than 16 query rows per KV head (G * T > 16: large groups, multi-token drafts): RT waves
// per workgroup serve the same KV head, 16 rows each (each wave reads the head's K/V rows; the
// reads of the other waves hit the caches), and row groups of 16 RT rows beyond 64 rows.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"

namespace skvd {

// ----------------------------------------------------------------------------- int8 -> f16
// K operand (feeds the score MFMA, so compiler-visible code only: the MFMA's operand hazards are
// tracked for the compiler's own instructions): flip the sign bit of each byte (x + 128 as an
// unsigned byte u), put u under the f16 exponent of 1024 with a byte permute (the f16 with bits
// 0x64uu is 1024 + u, exact) and subtract 1152 with one packed f16 add per pair.
constexpr unsigned kExp1024 = 0x64646464u;  // every byte 0x64: f16 high byte of 1024

template <int BIAS = 1152>
__device__ __forceinline__ half2v magic_pair(unsigned flipped, unsigned sel) {
  return __builtin_bit_cast(half2v, __builtin_amdgcn_perm(kExp1024, flipped, sel)) -
         (half2v)(_Float16)BIAS;
}

// 8 signed bytes (elements 0..7 in byte order) -> 8 f16.
__device__ __forceinline__ half8 i8x8_to_h8(uint2v w) {
  half8 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const unsigned x = w[k] ^ 0x80808080u;
    const half2v lo = magic_pair(x, 0x04010400u), hi = magic_pair(x, 0x04030402u);
    r[4 * k + 0] = lo[0];
    r[4 * k + 1] = lo[1];
    r[4 * k + 2] = hi[0];
    r[4 * k + 3] = hi[1];
  }
  return r;
}

// V pairs (feed v_dot2, vector ALU only): v_cvt_f16_i16 with SDWA operand selection takes byte
// k of a dword sign-extended and writes either the low half of the result (clearing the high
// half) or the high half (keeping the low half) -- a packed f16 pair in two instructions, one
// per element, with no shifts, permutes or packs.
template <int B>
__device__ __forceinline__ unsigned cvt_i8_lo(unsigned src);
template <int B>
__device__ __forceinline__ unsigned cvt_i8_hi(unsigned dst, unsigned src);
#define SKVD_CVT_I8(B)                                                                         \
  template <>                                                                                  \
  __device__ __forceinline__ unsigned cvt_i8_lo<B>(unsigned src) {                             \
    unsigned r;                                                                                \
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_" \
        #B : "=v"(r) : "v"(src));                                                              \
    return r;                                                                                  \
  }                                                                                            \
  template <>                                                                                  \
  __device__ __forceinline__ unsigned cvt_i8_hi<B>(unsigned dst, unsigned src) {               \
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE "           \
        "src0_sel:BYTE_" #B : "+v"(dst) : "v"(src));                                           \
    return dst;                                                                                \
  }
SKVD_CVT_I8(0)
SKVD_CVT_I8(1)
SKVD_CVT_I8(2)
SKVD_CVT_I8(3)
#undef SKVD_CVT_I8

// Two int8 rows a (token t) and b (token t + 16), 8 elements each -> the 8 f16 pairs
// (a_i, b_i).
__device__ __forceinline__ void i8_pairs(uint2v a, uint2v b, half2v *out) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const unsigned x = a[w], y = b[w];
    out[4 * w + 0] = __builtin_bit_cast(half2v, cvt_i8_hi<0>(cvt_i8_lo<0>(x), y));
    out[4 * w + 1] = __builtin_bit_cast(half2v, cvt_i8_hi<1>(cvt_i8_lo<1>(x), y));
    out[4 * w + 2] = __builtin_bit_cast(half2v, cvt_i8_hi<2>(cvt_i8_lo<2>(x), y));
    out[4 * w + 3] = __builtin_bit_cast(half2v, cvt_i8_hi<3>(cvt_i8_lo<3>(x), y));
  }
}

// Two f16 rows a (token t) and b (token t + 16) -> the 8 pairs (a_i, b_i).
__device__ __forceinline__ void h16_pairs(const half8 &a, const half8 &b, half2v *out) {
  const uint4v aw = __builtin_bit_cast(uint4v, a), bw = __builtin_bit_cast(uint4v, b);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(bw[k], aw[k], 0x05040100u));
    out[2 * k + 1] = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(bw[k], aw[k], 0x07060302u));
  }
}

// ----------------------------------------------------------------------------- q4_0 -> f16
// A q4_0 dword (four code bytes, byte k holding element k of a run in its low nibble and
// element k + 16 in its high nibble) gives 8 elements: the low nibbles (elements 0..3 of the
// run) and the high nibbles (16..19). Each nibble n goes under the f16 exponent of 1024 with a
// byte permute (1024 + n, exact) and one packed add of -1032 leaves n - 8, exact: the code's
// value before its scale.
constexpr unsigned kNib = 0x0F0F0F0Fu;

// One dword -> 8 f16 (c - 8): low nibbles of bytes 0..3, then high nibbles of bytes 0..3.
__device__ __forceinline__ half8 q4x8_to_h8(unsigned w) {
  const unsigned lo = w & kNib, hi = (w >> 4) & kNib;
  const half2v a = magic_pair<1032>(lo, 0x04010400u), b = magic_pair<1032>(lo, 0x04030402u);
  const half2v c = magic_pair<1032>(hi, 0x04010400u), d = magic_pair<1032>(hi, 0x04030402u);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Two q4_0 dwords a (token t) and b (token t + 16) -> the 8 f16 pairs (a_i - 8, b_i - 8) in
// q4x8_to_h8's element order: byte k of a and byte k of b side by side in the two halves, then
// their low nibbles, and (shifted down) their high nibbles, under the exponent of 1024.
__device__ __forceinline__ void q4_pairs(unsigned a, unsigned b, half2v *out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned t = __builtin_amdgcn_perm(b, a, 0x0C000C00u | ((4u + k) << 16) | (unsigned)k);
    out[k] = __builtin_bit_cast(half2v, (t & 0x000F000Fu) | 0x64006400u) - (half2v)(_Float16)1032;
    out[4 + k] =
        __builtin_bit_cast(half2v, ((t >> 4) & 0x000F000Fu) | 0x64006400u) - (half2v)(_Float16)1032;
  }
}

// ----------------------------------------------------------------------------- fp8 (E4M3) -> f16
// The conversion instruction turns two OCP E4M3 bytes (the low or the high half-word of a
// dword) into two f16 values times a power-of-two scale (only the scale's exponent is used):
// with 2^-8 every E4M3 value, subnormals included, is exact in f16 (|x| 2^-8 <= 1.75, the least
// subnormal 2^-17) and keeps the f16 products of the score MFMA and the P.V dot products far from
// overflow. The 2^8 comes back with the per-tensor scales, folded into the score scale (K) and
// the output (V). The NaN byte stays NaN.
constexpr float kF8Scale = 0.00390625f;  // 2^-8

template <bool HI>
__device__ __forceinline__ half2v f8x2_to_h2(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, kF8Scale, HI);
}

// 8 E4M3 bytes (elements 0..7 in byte order) -> 8 f16 (value * 2^-8).
__device__ __forceinline__ half8 f8x8_to_h8(uint2v w) {
  half8 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const half2v lo = f8x2_to_h2<false>(w[k]), hi = f8x2_to_h2<true>(w[k]);
    r[4 * k] = lo[0];
    r[4 * k + 1] = lo[1];
    r[4 * k + 2] = hi[0];
    r[4 * k + 3] = hi[1];
  }
  return r;
}

// Two E4M3 rows a (token t) and b (token t + 16), 8 elements each -> the 8 f16 pairs
// (a_i, b_i) (values * 2^-8): one byte permute gathers bytes i and i+1 of both rows as
// (a_i, b_i, a_i+1, b_i+1), the two half-words of which convert to two pairs.
__device__ __forceinline__ void f8_pairs(uint2v a, uint2v b, half2v *out) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      // perm selector bytes: 0-3 pick from the second operand (a), 4-7 from the first (b)
      const unsigned t = __builtin_amdgcn_perm(
          b[w], a[w], ((5u + i) << 24) | ((unsigned)(i + 1) << 16) | ((4u + i) << 8) | (unsigned)i);
      out[4 * w + i] = f8x2_to_h2<false>(t);
      out[4 * w + i + 1] = f8x2_to_h2<true>(t);
    }
  }
}


// ----------------------------------------------------------------------------- int8 K scale groups
// A score MFMA step contracts 32 head_dim elements, 8 from each of the four lane groups (lanes
// 16g .. 16g + 15). A lane loads the 32 bytes of one scale group of its token with two 16-byte
// loads: lane group g holds group g (of a run of four groups) as pieces 0..3 of 8 bytes. The
// 4 x 4 transpose of pieces across the lane groups -- two swap stages, lane groups {0,1} <->
// {2,3}, then {0,2} <-> {1,3} -- leaves piece g of group k in slot k of lane group g, so that
// MFMA step k contracts group k alone and its f32 result can take that group's scale exactly.
// lo holds slots 0, 1 (two dwords each), hi slots 2, 3; slot (c, d) = 2c + d.
__device__ __forceinline__ void group_transpose(uint4v &lo, uint4v &hi) {
  // lane groups (a, b) = (g / 2, g % 2): slot (1, d) of a = 0 <-> slot (0, d) of a = 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(lo[i], hi[i], false, false);
    lo[i] = r[0];
    hi[i] = r[1];
  }
  // slot (c, 1) of b = 0 <-> slot (c, 0) of b = 1
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto r0 = __builtin_amdgcn_permlane16_swap(lo[w], lo[2 + w], false, false);
    lo[w] = r0[0];
    lo[2 + w] = r0[1];
    const auto r1 = __builtin_amdgcn_permlane16_swap(hi[w], hi[2 + w], false, false);
    hi[w] = r1[0];
    hi[2 + w] = r1[1];
  }
}

// q4_0 K: a lane loads the 16 code bytes of group g4 (of a run of four groups) of its token as
// dwords 0..3. The same two-stage 4 x 4 transpose over dwords leaves dword g4 of group k in
// slot k of lane group g4: MFMA step k contracts group k alone (elements 4*g4 .. +3 and
// 16 + 4*g4 .. +3 of it from lane group g4), so its f32 result takes that group's scale.
__device__ __forceinline__ void nib_transpose(uint4v &x) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {  // slot (1, d) of lane groups {0,1} <-> slot (0, d) of {2,3}
    const auto r = __builtin_amdgcn_permlane32_swap(x[d], x[2 + d], false, false);
    x[d] = r[0];
    x[2 + d] = r[1];
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {  // slot (c, 1) of lane groups {0,2} <-> slot (c, 0) of {1,3}
    const auto r = __builtin_amdgcn_permlane16_swap(x[2 * c], x[2 * c + 1], false, false);
    x[2 * c] = r[0];
    x[2 * c + 1] = r[1];
  }
}

// ----------------------------------------------------------------------------- partial kernel
// K and V rows are read once: non-temporal loads (evict-first in L2, no Infinity Cache
// allocation) when each load instruction covers whole 128-byte lines between the lanes that
// share them (f16 K: half lines, consumed by the next instruction; f16 and int8 V: whole
// lines). int8 K instructions cover a quarter of each line, whose other quarters are read by
// the next three instructions: cached loads (measured: evict-first loses them).
template <bool STREAM, class T>
__device__ __forceinline__ T kv_load(const char *p) {
  if constexpr (STREAM) return __builtin_nontemporal_load((const T *)p);
  else return *(const T *)p;
}

// ----------------------------------------------------------------------------- partial kernel (body)
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v *lds_s4_ptr;

// Byte offset of 16-byte chunk c of row r in a row-major LDS tile with rows of ROWB bytes (a
// multiple of 128, so a row starts on bank 0 and a chunk's banks are set by c mod 8). The
// chunk index is XOR-swizzled by the row so that both read patterns are free of bank
// conflicts: (1) the transposed reads (ds_read_b64_tr_b16), where each 16-lane phase reads 32
// contiguous bytes (two chunks 2j, 2j+1) of 4 consecutive rows, need those rows' chunk pairs in
// 4 different 32-byte bank groups: swizzle bits 1-2 take the row's low 2 bits (bit 2 from row
// bit 0, so that two consecutive rows written 4 chunks at a time also fill all 8 chunk slots);
// (2) a 16-byte read of one chunk of 8 consecutive rows (8 lanes a phase) needs 8 different
// chunks mod 8: bit 0 takes row bit 2 (and bit 3 row bit 3 when a row holds 16 or more chunks in
// powers of two; rows of 24 chunks, head_dim 192, keep the chunk inside its aligned run of 8).
template <int ROWB>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int CPR = ROWB / 16;
  constexpr bool P2 = (CPR & (CPR - 1)) == 0;
  const int x = ((r & 1) << 2) | (r & 2) | ((r >> 2) & 1) | (P2 ? (r & 8) : 0);
  return r * ROWB + ((c ^ x) << 4);
}

// D: head_dim (128/256). RB: 4-row quarters of the 16 MFMA rows in use per wave (R = G*T
// query rows of a KV head; R <= 4*RB with one row tile, RB = 4 with more).
// KV: cache format, 0 f16, 1 int8 with f16 scales per 32 elements, 2 fp8 E4M3 with one f32
// scale per tensor, 3 q4_0 (two 4-bit codes per byte) with f16 scales per 32 elements; the
// two one-byte formats share the load layout (I8 below), int8 and q4_0 read per-row scales
// (SC), and q4_0 loads 16 code bytes per group and 4 per V lane (Q4). FAST: page_size >= 16, so each 16-token
// tile lies in one page and its page id is wave-uniform. CH: tokens per chunk (16, 32 or
// 64): the K and V registers of a chunk bound how many waves fit on a SIMD.
// PVM: P.V on the MFMA through an LDS copy of the chunk's V (dense when several query rows
// share the KV head); otherwise P.V on the vector ALU as f16 pair dot products
// (v_dot2_f32_f16) from the V registers, pairing token t with token t + 16.
// HW: KV heads per workgroup (one wave each). RT: row tiles per KV head (one wave each, 16
// query rows; HW = 1 when RT > 1). DBG: the gather-debug variant, which writes the raw K/V rows
// and int8 scales it holds at their point of use into LaunchArgs::dbg_* and nothing else.
// Minimum waves per SIMD the register allocator must leave room for. int8 at D=128 is vector-
// ALU heavy and runs several waves per SIMD (the plan launches 8 workgroups per CU): three,
// at the cost of three values spilled and reloaded once per segment. f16 single-quarter
// variants run one wave per SIMD under the balanced schedule and gain more from registers
// spent on instruction-level parallelism than from occupancy: no floor. The one-byte formats
// at D = 192 / 256 widen every element: two waves per SIMD (<= 256 registers; int8 spills 16
// values), so that one wave's widening overlaps the other's loads (the wide multi-token
// workload's shape: int8 408 -> 290-300 us, fp8 377 -> 244-255, q4_0 393 -> 240-254, with 8
// workgroups per CU); f16 there, a pure stream, keeps one wave per SIMD (no faster with two).
template <int D, int RB, bool I8>
constexpr int partial_waves() {
  return D == 128 ? (RB == 1 ? (I8 ? 3 : 1) : 2) : (D <= 256 && I8 ? 2 : 1);
}

template <int D, int RB, int KV, bool FAST, int CH, bool PVM, int HW, int RT, bool DBG>
__global__ __launch_bounds__(64 * HW * RT)
__attribute__((amdgpu_waves_per_eu(partial_waves<D, RB, KV != 0>()))) void partial_kernel(LaunchArgs a) {
  // The argument block's first two 64-byte lines (pointers and strides of q and the pools,
  // the page table) come in with the first batch of argument loads: left to the compiler,
  // they are loaded after the share arithmetic, one more memory round trip on the launch's
  // critical path.
  asm volatile("" ::"s"(a.q), "s"(a.table));
  constexpr bool I8 = KV != 0;  // elements of at most one byte
  constexpr bool SC = KV == 1 || KV == 3;  // int8, q4_0: f16 scales per 32 elements of a row
  constexpr bool F8 = KV == 2;  // fp8 E4M3: one f32 scale per tensor
  constexpr bool Q4 = KV == 3;  // q4_0: rows of D/2 bytes
  static_assert(RT == 1 || (HW == 1 && RB == 4 && PVM), "row tiles: one KV head per workgroup");
  static_assert(!SC || D % 128 == 0, "scale rows are read four groups at a time");
  constexpr int NW = HW * RT;        // waves per workgroup
  // row tiles re-read the same K/V rows: cached loads. q4_0 rows (64 bytes at D=128) are half
  // lines whose other half is the neighbouring KV head's, read by another wave: cached loads.
  constexpr bool STREAM = RT == 1 && !Q4;
  static_assert(CH == 16 || CH == 32 || (CH == 64 && !PVM), "chunk");
  static_assert(PVM || CH % 32 == 0, "the vector P.V pairs 16-token tiles 2h and 2h + 1");
  constexpr int NT = CH / 16;    // 16-token score tiles per chunk
  constexpr int KS = D / 32;     // 32-element head_dim groups (int8 scale groups)
  // one-byte K: a lane loads 32 bytes of group g4 + 4m for each block m of four groups (the
  // last block partly empty at head_dim 192: its missing groups hold zeros)
  constexpr int KB = (KS + 3) / 4;
  // score MFMA steps: one per group for f16 and int8 (after the int8 lane transpose); fp8 keeps
  // the load layout, four steps per block
  constexpr int KSTEPS = F8 ? 4 * KB : KS;
  constexpr int LPR = D / 8;     // lanes per V row in the load layout, 8 elements each
  constexpr int TPS = 64 / LPR;  // V rows per load step (lanes past TPS * LPR idle: D = 192)
  constexpr int NS = CH / TPS;   // V load steps per chunk
  static_assert(CH % TPS == 0, "V load steps");
  constexpr int NDT = D / 16;    // 16-wide head_dim tiles of the P.V MFMA
  constexpr int KPL = CH / 4;    // P.V contraction elements per lane (8: 16x16x32, 4: 16x16x16)
  constexpr int RM = 4 * RB;     // query rows held (padded)
  constexpr int PSTR = CH + 4;   // row stride of the probability tile, floats
  constexpr int ROWB = 2 * D;    // bytes per V row in LDS (f16)
  // one lane's 8 elements of a V row (q4_0: one dword, elements vq0 .. +3 and vq1 .. +3 below)
  using Vec = std::conditional_t<Q4, unsigned, std::conditional_t<I8, uint2v, half8>>;
  using PvOp = std::conditional_t<CH == 32, half8, half4>;

  // LDS, one slice per wave:
  constexpr int VL = PVM ? CH * ROWB : 16;          // chunk V rows, f16
  constexpr int PL = PVM ? RM * PSTR : 4;           // probabilities [row][token]
  // int8 at D=128 (32-token chunks): a chunk's K and V scales come in one 8-byte load per lane
  // (lanes 0..31: the K scales of chunk token lane; 32..63: the V scales of token lane - 32),
  // issued with the chunk's K rows and handed over through LDS, instead of a two-byte load per
  // token tile for K and an 8-byte load for V (one vector-memory instruction per chunk instead
  // of three).
  constexpr bool SCL = SC && D == 128 && CH == 32;
  constexpr int SL = SCL ? 64 : SC ? CH * (D / 128) : 1;  // int8 scales [token][group], f16
  constexpr int QL = PVM ? 4 : (CH / 2) * RM;       // vector P.V: f16 pairs (tp, tp+16) [tp][row]
  __shared__ __attribute__((aligned(16))) char v_lds_all[NW * VL];
  __shared__ __attribute__((aligned(16))) float p_lds_all[NW * PL];
  __shared__ __attribute__((aligned(16))) uint2v vsc_lds_all[NW * SL];
  __shared__ __attribute__((aligned(16))) unsigned p2_lds_all[NW * QL];
  // (readfirstlane: the wave index is uniform in the wave, and saying so keeps the KV head and
  // every row base derived from it in SGPRs, so loads take a scalar base + 32-bit lane offset)
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  const int head_w = RT > 1 ? 0 : wave;  // this wave's KV head within the workgroup's group
  const int tile_w = RT > 1 ? wave : 0;  // this wave's row tile within the row group
  char *const v_lds = v_lds_all + wave * VL;
  float *const p_lds = p_lds_all + wave * PL;
  uint2v *const vsc_lds = vsc_lds_all + wave * SL;
  const _Float16 *vsh = (const _Float16 *)(vsc_lds + (SCL ? CH : 0));  // V scales
  const _Float16 *ksl = (const _Float16 *)vsc_lds;                        // K scales (SCL)
  unsigned *const p2_lds = p2_lds_all + wave * QL;

  const int lane = threadIdx.x & 63;
  const int Hkv = a.Hkv;
  // schedule heads (Hkv / HW KV head groups times row groups): the rows of the schedule are
  // (sequence, schedule head)
  const int Hg = a.sched_heads;
  const int NRG = a.row_groups, RPG = a.rows_per_group;
  // fp8: the per-tensor scales (one f32 each in device memory) times the widening's 2^8, on
  // the scores' scale (K) and on the output (V); 1 for the other formats
  const float scale_log2 = F8 ? a.scale_log2 * (*(const float *)a.ks * 256.f) : a.scale_log2;
  const float vfac = F8 ? *(const float *)a.vs * 256.f : 1.f;
  const int T = a.T, G = a.G, R = G * T;
  const int P1 = (1 << a.page_shift) - 1;

  // ---- this workgroup's segments: (sequence, schedule head, block range, partial slot); wave
  // w of the workgroup serves KV head HW * group + w (or row tile w of the group's KV head)
  // over the same block range
  // Static: workgroup order split fastest, then KV head, then sequence, with an odd split
  // stride. Consecutive workgroups go to the eight XCDs in turn; with an even stride split s
  // of every (head, sequence) would land on the same XCD, and the live splits of a ragged
  // batch would pile onto the XCDs of the low split indices. The odd stride rotates each
  // row's start over all eight. Indices past splits_cap are padding. One segment.
  // Balanced: the batch's blocks in (sequence, KV head, block) order are cut into W equal
  // contiguous shares; workgroup w takes share w, which may cover the end of one row and the
  // start of the next ones: one segment per row, its partial in slot w - (first share of the
  // row). Sequence lengths, one per lane, come from kv_len on the device.
  int st_b = 0, st_grp = 0, st_split = 0;
  Shares sh{};
  int x_cur = 0, x_end = 0;  // balanced: this workgroup's share (blocks below 2^31)
  // Progress priority (int8, whose waves share SIMDs): waves of a SIMD are served oldest
  // first, so a co-resident workgroup started later falls behind and finishes alone, with fewer
  // loads in flight. Each wave instead sets its issue priority from the fraction of its work
  // done (3 in the first quarter down to 0 in the last), so the waves of a SIMD advance
  // together. Blocks done so far: done_base (earlier segments) + the segment's own; quarters
  // at pq1, pq2, pq3.
  int done_base = 0, pq1 = 0, pq2 = 0, pq3 = 0;
  const int share = blockIdx.x;
  if (a.balanced) {
    sh = balanced_shares(a, a.debug);
    if (share >= sh.n_shares) return;
    // floor(w N / W) = w q + floor(w r / W) with N = q W + r: 32-bit (N < 2^31, W^2 < 2^30)
    const unsigned N = (unsigned)sh.n_blocks, W = (unsigned)sh.n_shares;
    const unsigned q = N / W, r = N - q * W;
    x_cur = (int)(share * q + (share * r) / W);
    x_end = (int)((share + 1) * q + ((share + 1) * r) / W);
    const int total = (int)(x_end - x_cur);
    pq1 = total / 4;
    pq2 = total / 2;
    pq3 = 3 * total / 4;
  } else {
    const int wg = blockIdx.x;
    st_split = wg % a.split_stride;
    const int head_seq = wg / a.split_stride;
    st_grp = head_seq % Hg;
    st_b = head_seq / Hg;
    if (st_split >= a.splits_cap) return;
  }
  bool pending = true;
  for (;;) {
  int b, grp, slot, L, blk_lo, blk_hi;
  if (a.balanced) {
    if (x_cur >= x_end) break;
    // the sequence holding global block x_cur: Hg*pre <= x_cur < Hg*(pre + nb), that is
    // pre <= x_cur / Hg < pre + nb (one scalar division, 32-bit lane compares)
    const unsigned xq = (unsigned)x_cur / (unsigned)Hg;
    const SeqRef sr = seq_at(a, sh, xq);
    b = sr.b;
    const unsigned pre_b = sr.pre;
    const int nb_b = sr.nb;
    L = sr.L;
    const unsigned off = (unsigned)x_cur - (unsigned)Hg * pre_b;
    grp = (int)(off / (unsigned)nb_b);
    blk_lo = (int)(off - (unsigned)grp * (unsigned)nb_b);
    const int row0 = (int)((unsigned)Hg * pre_b + (unsigned)grp * (unsigned)nb_b);  // row's 1st block
    const int seg_end = min(x_end, row0 + nb_b);
    blk_hi = blk_lo + (seg_end - x_cur);
    // compact slot of (schedule row b*Hg + grp, share): unique, below rows + shares
    slot = b * Hg + grp + share;
    x_cur = seg_end;
  } else {
    if (!pending) break;
    pending = false;
    b = st_b;
    grp = st_grp;
    slot = st_split;
    L = clamp_len(a.kv_len[b], a.max_kv_len, a.status, a.debug);
    const int nblk = (L + 63) >> 6;
    blk_lo = st_split * a.bps;
    if (!a.single && blk_lo >= nblk) break;  // beyond this sequence: no partial is read
    blk_hi = min(blk_lo + a.bps, nblk);
    const int total = blk_hi - blk_lo;
    pq1 = total / 4;
    pq2 = total / 2;
    pq3 = 3 * total / 4;
  }
  const int kgrp = NRG == 1 ? grp : grp / NRG;  // KV head group
  const int rg = grp - kgrp * NRG;               // row group
  const int kvh = HW * kgrp + head_w;
  const int row0 = rg * RPG + kRowTile * tile_w;  // this wave's first query row of the KV head
  if (row0 >= R) continue;                        // a row tile past the last row
  const int tok0 = blk_lo * 64;
  const int tok_end = min(blk_hi * 64, L);

  const char *kbase = (const char *)a.k;
  const char *vbase = (const char *)a.v;
  constexpr int ES = I8 ? 1 : 2;  // element bytes
  const _Float16 *ksc = (const _Float16 *)a.ks;
  const _Float16 *vsc = (const _Float16 *)a.vs;

  // Query rows as the score MFMA A operand: lane holds row (lane & 15), elements
  // 8*(lane>>4)..+7 of each 32-element contraction step.
  const int g4 = lane >> 4, c16 = lane & 15;
  // head_dim element of step k's first lane element (the contraction order is free as long as
  // q and K agree): f16 and int8 (after the group transpose), 32k + 8*g4, so that step k
  // contracts the 32-element group k; fp8, group g4 + 4*(k/4) at offset 8*(k%4), each lane's
  // elements of a group being 32 contiguous bytes as loaded
  auto kelem = [&](int k) __attribute__((always_inline)) {
    return F8 ? 32 * (g4 + 4 * (k >> 2)) + 8 * (k & 3) : 32 * k + 8 * g4;
  };
  half8 qa[KSTEPS];
  {
    const int r = row0 + c16;
    if (r < R) {
      const int t = r / G, hg = r - (r / G) * G;
      const _Float16 *qp = (const _Float16 *)a.q + ((int64_t)b * T + t) * a.q_tok_stride +
                           (int64_t)(kvh * G + hg) * a.q_head_stride + 8 * g4;
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {  // (fp8 steps of a missing group: zeros)
        if constexpr (Q4) {
          // q4_0 step k: elements 4*g4 .. +3 and 16 + 4*g4 .. +3 of group k (the K dword's)
          const half4 lo = *(const half4 *)(qp - 4 * g4 + 32 * k);
          const half4 hi = *(const half4 *)(qp - 4 * g4 + 32 * k + 16);
          qa[k] = half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          qa[k] = kelem(k) < D ? *(const half8 *)(qp + kelem(k) - 8 * g4) : (half8)(_Float16)0;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) qa[k] = (half8)(_Float16)0;
    }
  }
  // This lane's MFMA output rows: row0 + 4*g4 + e. Row r sees positions j < L - T + t + 1.
  int nvis[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = row0 + 4 * g4 + e;
    const int n = r < R ? L - T + r / G + 1 : 0;
    nvis[e] = min(n, tok_end);
  }

  float m[4], lsum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { m[e] = kNegInf; lsum[e] = 0.f; }
  // MFMA P.V output: lane holds head_dim column 16*dt + c16 of rows 4*g4 + e.
  float4v acc[PVM ? NDT : 1];
#pragma unroll
  for (int dt = 0; dt < (PVM ? NDT : 1); ++dt) acc[dt] = (float4v)0.f;
  // Vector P.V output: lane holds elements vlane_el .. +7 of every row, summed over the
  // tokens of its load slot (reduced across slots at the end).
  float accv[PVM ? 1 : RM][8];
#pragma unroll
  for (int r = 0; r < (PVM ? 1 : RM); ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) accv[r][i] = 0.f;

  bool clamped_any = false;
  const int vlane_tok = lane / LPR, vlane_el = 8 * (lane % LPR);
  // head_dim elements of the lane's V slot as two runs of four: vq0 .. +3 and vq1 .. +3
  // (contiguous for f16 and one-byte elements; q4_0: the low and high nibbles of the lane's
  // dword, dword w of group g holding elements 32g + 4w .. +3 and 32g + 16 + 4w .. +3)
  const int vq0 = Q4 ? 32 * (vlane_el >> 5) + ((vlane_el & 31) >> 1) : vlane_el;
  const int vq1 = Q4 ? vq0 + 16 : vlane_el + 4;
  const bool vlane_ok = lane < TPS * LPR;  // (loads of the idle lanes re-read valid rows)
  // gather-debug variant: dense row (sequence b, position j, KV head kvh)
  auto dbg_row = [&](int j) __attribute__((always_inline)) -> int64_t {
    return ((int64_t)b * a.dbg_max_len + j) * Hkv + kvh;
  };
  _Float16 *const dbg_ks = (_Float16 *)a.dbg_ks, *const dbg_vs = (_Float16 *)a.dbg_vs;

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

  // Per-lane token offsets within a 16-token tile, hoisted: with a non-negative stride,
  // min(token, limit) * stride = min(token * stride, limit * stride), the limit being scalar.
  const unsigned c16_tok = (unsigned)(c16 * (int)a.tok_stride);
  const unsigned c16_stok = SC ? (unsigned)(c16 * (int)a.s_tok_stride) : 0u;
  const unsigned vt_tok = (unsigned)(vlane_tok * (int)a.tok_stride);

  Vec kb[NT][I8 ? 1 : KS];                   // f16 K: step k's 8 elements
  // one-byte K: the lane's 32 bytes of group g4 + 4m; q4_0: its 16 code bytes
  uint4v kq[NT][I8 ? KB : 1][Q4 ? 1 : 2];
  uint2v ksr[NT][SC && !SCL ? KS / 4 : 1];   // int8 K (no shared scale load): the D/32 scales
                                             // of the lane's token, four per 8-byte load
  Vec vb[NS];
  // int8 V scales: the D/32 scales of chunk token (lane % CH), one 8-byte load per lane (a
  // token-head's scales are contiguous), handed to the P.V lanes through LDS.
  uint2v vsr[D / 128];
  uint2v scr;  // SCL: this lane's K (lane < 32) or V scales of one chunk token

  // K rows of chunk c0 in the score MFMA B-operand layout: tile t, lane (g4, c16) holds
  // elements 32k + 8*g4 .. +7 of token 16t + c16.
  auto load_k = [&](int c0, const int *pgs) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int jt = c0 + 16 * t;
      if constexpr (FAST) {
        // wave-uniform base of the (clamped) tile on the scalar unit + 32-bit lane offset
        const int jte = min(jt, last_tile);
        const int64_t pg = clamp_page(pgs[t], a.num_k_pages);
        const char *base = kbase + row_offset(pg, jte & P1, kvh, a.page_stride, a.tok_stride,
                                              a.head_stride) * ES;
        const int lim = min(tok_end - 1 - jte, 15);  // last valid token of the tile
        if constexpr (Q4) {
          const unsigned off = min(c16_tok, (unsigned)(lim * (int)a.tok_stride)) + 16 * g4;
#pragma unroll
          for (int m = 0; m < KB; ++m) kq[t][m][0] = kv_load<STREAM, uint4v>(base + off + 64 * m);
        }
        if constexpr (I8 && !Q4) {
          const unsigned off = min(c16_tok, (unsigned)(lim * (int)a.tok_stride)) + 32 * g4;
#pragma unroll
          for (int m = 0; m < KB; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              kq[t][m][h] = KS % 4 == 0 || g4 + 4 * m < KS
                                ? kv_load<STREAM, uint4v>(base + off + 128 * m + 16 * h)
                                : (uint4v)0u;
        }
        if constexpr (I8) {
          if constexpr (SC && !SCL) {
            const _Float16 *sb = ksc + row_offset(pg, jte & P1, kvh, a.s_page_stride,
                                                  a.s_tok_stride, a.s_head_stride);
            const unsigned so = 2u * min(c16_stok, (unsigned)(lim * (int)a.s_tok_stride));
#pragma unroll
            for (int h = 0; h < KS / 4; ++h)
              ksr[t][h] = *(const uint2v *)((const char *)sb + so + 8 * h);
          }
        } else {
          const unsigned off = (min(c16_tok, (unsigned)(lim * (int)a.tok_stride)) + 8 * g4) * ES;
#pragma unroll
          for (int k = 0; k < KS; ++k) kb[t][k] = kv_load<STREAM, Vec>(base + off + 32 * k * ES);
        }
      } else {
        const int j = min(jt + c16, tok_end - 1);
        bool cl;
        const int64_t pg = lookup_page(a.table, a.table_stride, b, j, a.page_shift,
                                       a.num_k_pages, &cl);
        clamped_any |= cl;
        const int64_t off = row_offset(pg, j & P1, kvh, a.page_stride, a.tok_stride,
                                       a.head_stride);
        if constexpr (Q4) {
          const char *kp = kbase + off + 16 * g4;
#pragma unroll
          for (int m = 0; m < KB; ++m) kq[t][m][0] = kv_load<STREAM, uint4v>(kp + 64 * m);
        }
        if constexpr (I8 && !Q4) {
          const char *kp = kbase + off + 32 * g4;
#pragma unroll
          for (int m = 0; m < KB; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              kq[t][m][h] = KS % 4 == 0 || g4 + 4 * m < KS
                                ? kv_load<STREAM, uint4v>(kp + 128 * m + 16 * h)
                                : (uint4v)0u;
        }
        if constexpr (I8) {
          if constexpr (SC && !SCL) {
            const int64_t so = row_offset(pg, j & P1, kvh, a.s_page_stride, a.s_tok_stride,
                                          a.s_head_stride);
#pragma unroll
            for (int h = 0; h < KS / 4; ++h) ksr[t][h] = *(const uint2v *)(ksc + so + 4 * h);
          }
        } else {
          const char *kp = kbase + (off + 8 * g4) * ES;
#pragma unroll
          for (int k = 0; k < KS; ++k) kb[t][k] = kv_load<STREAM, Vec>(kp + 32 * k * ES);
        }
      }
    }
    if constexpr (SCL) {
      // K scales (lanes 0..31) or V scales (32..63) of chunk token lane % 32; a token past the
      // split reads the last one's
      const bool isk = lane < CH;
      const int jl = min(c0 + (lane & (CH - 1)), tok_end - 1);
      const int64_t np = isk ? a.num_k_pages : a.num_v_pages;
      int64_t pg;
      if constexpr (FAST) {
        const int tl = (jl - c0) >> 4;  // the token's 16-token tile (its page is wave-uniform)
        int pgl = pgs[0];
#pragma unroll
        for (int t = 1; t < NT; ++t) pgl = tl == t ? pgs[t] : pgl;
        pg = clamp_page(pgl, np);
      } else {
        bool cl;
        pg = lookup_page(a.table, a.table_stride, b, jl, a.page_shift, np, &cl);
        clamped_any |= cl;
      }
      const _Float16 *sp = (isk ? ksc : vsc) + row_offset(pg, jl & P1, kvh, a.s_page_stride,
                                                          a.s_tok_stride, a.s_head_stride);
      scr = *(const uint2v *)sp;
    }
  };
  // V rows of chunk c0 in the load layout: step s, lane holds elements vlane_el .. +7 of
  // token TPS*s + vlane_tok.
  auto load_v = [&](int c0, const int *pgs) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int js = c0 + TPS * s2;
      if constexpr (FAST) {
        const int jte = min(js & ~15, last_tile);
        const int64_t pg = clamp_page(pgs[(TPS * s2) >> 4], a.num_v_pages);
        const char *base = vbase + row_offset(pg, jte & P1, kvh, a.page_stride, a.tok_stride,
                                              a.head_stride) * ES;
        // token (js & 15) + vlane_tok of the tile, clamped to its last valid token
        const int ts = (int)a.tok_stride;
        const unsigned tko = min(vt_tok + (unsigned)((js & 15) * ts),
                                 (unsigned)(min(tok_end - 1 - jte, 15) * ts));
        const unsigned off = Q4 ? tko + vlane_el / 2 : (tko + vlane_el) * ES;
        vb[s2] = kv_load<STREAM, Vec>(base + off);
      } else {
        const int j = min(js + vlane_tok, tok_end - 1);
        bool cl;
        const int64_t pg = lookup_page(a.table, a.table_stride, b, j, a.page_shift,
                                       a.num_v_pages, &cl);
        clamped_any |= cl;
        const int64_t off = row_offset(pg, j & P1, kvh, a.page_stride, a.tok_stride,
                                       a.head_stride);
        vb[s2] = kv_load<STREAM, Vec>(vbase + (Q4 ? off + vlane_el / 2 : (off + vlane_el) * ES));
      }
    }
    if constexpr (SC && !SCL) {
      // scales of chunk token (lane % CH); a token past the split reads the last one's
      const int jl = min(c0 + lane % CH, tok_end - 1);
      int64_t pg;
      if constexpr (FAST) {
        const int tl = (jl - c0) >> 4;  // the lane's 16-token tile (its page is wave-uniform)
        int pgl = pgs[0];
#pragma unroll
        for (int t = 1; t < NT; ++t) pgl = tl == t ? pgs[t] : pgl;
        pg = clamp_page(pgl, a.num_v_pages);
      } else {
        bool cl;
        pg = lookup_page(a.table, a.table_stride, b, jl, a.page_shift, a.num_v_pages, &cl);
        clamped_any |= cl;
      }
      const _Float16 *sp = vsc + row_offset(pg, jl & P1, kvh, a.s_page_stride, a.s_tok_stride,
                                            a.s_head_stride);
#pragma unroll
      for (int k4 = 0; k4 < D / 128; ++k4) vsr[k4] = *(const uint2v *)(sp + 4 * k4);
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
  // softmax, P.V with the chunk's V, prefetch of the next V. The first call is peeled off the
  // loop so that the loop is entered with the same load order as its back edge (K before V):
  // the in-order load counter is then waited on for K alone at the loop top. A last call with
  // more = false prefetches nothing: loads of a chunk past the segment are waited on before the
  // epilogue reuses their registers, an HBM round trip at the end of a segment (measured: 0.7 us
  // per launch at B = 1).
  auto chunk = [&](int c0, auto more) __attribute__((always_inline)) {
    constexpr bool PF = decltype(more)::value;
    const int c1 = c0 + CH;
    if constexpr (SCL) {  // this chunk's K and V scales to LDS (the previous chunk's reads of
      vsc_lds[lane] = scr;  // them ended at its closing wave_sync)
      wave_sync();
    }
    if constexpr (FAST && PF) chunk_pages(c1, pg_next);
    // ---- scores: S[t] = rows x 16 tokens of tile t (lane: token c16, rows 4*g4 + e)
    // The MFMA chains run for every tile, also the ones past the split (their K is a clamped
    // re-read and their scores are masked): a branch between an MFMA and the reads of its
    // result let the compiler's wait-state insertion miss the taken path.
    float4v S[NT];
    if constexpr (Q4) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int m = 0; m < KB; ++m) nib_transpose(kq[t][m][0]);
    } else if constexpr (SC) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int m = 0; m < KB; ++m) group_transpose(kq[t][m][0], kq[t][m][1]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      S[t] = (float4v)0.f;
      const int jk = c0 + 16 * t + c16;  // this lane's token (its K column)
      if constexpr (SC) {
        // int8: step k contracts group k (piece g4 of it in each lane group, widened exactly);
        // the f32 step result times the token's f16 group scale is the exact int8 * scale
        // value's contribution
        // (bit_cast of a vector element would cast element 0: copy the element out first)
        _Float16 sk[KS];
        if constexpr (SCL) {
          const uint2v s4 = *(const uint2v *)(ksl + (16 * t + c16) * 4);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const unsigned w = s4[k >> 1];
            sk[k] = __builtin_bit_cast(half2v, w)[k & 1];
          }
        } else {
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            const unsigned w = ksr[t][k >> 2][(k >> 1) & 1];
            sk[k] = __builtin_bit_cast(half2v, w)[k & 1];
          }
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          float4v p;
          if constexpr (Q4) {
            // q4_0: dword g4 of group k, its codes widened to c - 8
            const unsigned w = kq[t][k >> 2][0][k & 3];
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], q4x8_to_h8(w), (float4v)0.f, 0, 0,
                                                       0);
            if constexpr (DBG) {
              if (jk < tok_end) *(unsigned *)(a.dbg_k + dbg_row(jk) * (D / 2) + 16 * k + 4 * g4) = w;
            }
          } else {
            const uint4v &q4 = kq[t][k >> 2][(k & 3) >> 1];
            const unsigned w0 = q4[2 * (k & 1)], w1 = q4[2 * (k & 1) + 1];
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], i8x8_to_h8(uint2v{w0, w1}),
                                                       (float4v)0.f, 0, 0, 0);
            if constexpr (DBG) {
              if (jk < tok_end) *(uint2v *)(a.dbg_k + dbg_row(jk) * D + kelem(k)) = uint2v{w0, w1};
            }
          }
          const float s = (float)sk[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) S[t][e] = __builtin_fmaf(s, p[e], S[t][e]);
          if constexpr (DBG) {
            if (jk < tok_end && g4 == 0) dbg_ks[dbg_row(jk) * (D / 32) + k] = sk[k];
          }
        }
      } else if constexpr (F8) {
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) {
          const uint4v &q4 = kq[t][k >> 2][(k & 3) >> 1];
          const unsigned w0 = q4[2 * (k & 1)], w1 = q4[2 * (k & 1) + 1];
          // fp8: k_scale * 2^8 is in the score scale
          S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], f8x8_to_h8(uint2v{w0, w1}), S[t],
                                                        0, 0, 0);
          if constexpr (DBG) {
            if (jk < tok_end && kelem(k) < D)
              *(uint2v *)(a.dbg_k + dbg_row(jk) * D + kelem(k)) = uint2v{w0, w1};
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          S[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k], kb[t][k], S[t], 0, 0, 0);
          if constexpr (DBG) {
            if (jk < tok_end) *(half8 *)(a.dbg_k + (dbg_row(jk) * D + kelem(k)) * 2) = kb[t][k];
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- prefetch the next chunk's K while this chunk's softmax and P.V run (past the end
    // of the split, in a partial last chunk, this re-reads the last token: never used)
    if constexpr (PF) load_k(c1, pg_next);
    __builtin_amdgcn_sched_barrier(0);

    // ---- mask, online softmax (base 2)
    float alpha[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float cmax = kNegInf;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int j = c0 + 16 * t + c16;
        const float sc = j < nvis[e] ? S[t][e] * scale_log2 : kNegInf;
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

    if constexpr (DBG) {  // the chunk's V rows as loaded
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int jv = c0 + TPS * s2 + vlane_tok;
        if (jv < tok_end && vlane_ok)
          *(Vec *)(a.dbg_v + (Q4 ? dbg_row(jv) * (D / 2) + vlane_el / 2
                                 : (dbg_row(jv) * D + vlane_el) * ES)) = vb[s2];
      }
    }
    if constexpr (PVM) {
      // ---- probabilities to LDS as [row][token]; the chunk's V rows to LDS (int8 widened
      // exactly to f16; int8 V scales to vsc_lds)
      if (g4 < RB) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) p_lds[(4 * g4 + e) * PSTR + 16 * t + c16] = S[t][e];
      }
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int row = TPS * s2 + vlane_tok;
        if constexpr (Q4) {
          // the two runs of four elements (half chunks) at their columns
          const half8 h = q4x8_to_h8(vb[s2]);
          if (vlane_ok) {
            *(half4 *)(v_lds + swz<ROWB>(row, vq0 >> 3) + ((vq0 & 7) << 1)) =
                half4{h[0], h[1], h[2], h[3]};
            *(half4 *)(v_lds + swz<ROWB>(row, vq1 >> 3) + ((vq1 & 7) << 1)) =
                half4{h[4], h[5], h[6], h[7]};
          }
        } else {
          half8 h;
          if constexpr (SC) {
            h = i8x8_to_h8(vb[s2]);
          } else if constexpr (F8) {
            h = f8x8_to_h8(vb[s2]);
          } else {
            h = vb[s2];
          }
          if (vlane_ok) *(half8 *)(v_lds + swz<ROWB>(row, lane % LPR)) = h;
        }
      }
      if constexpr (SC && !SCL) {
        if (lane < CH) {
#pragma unroll
          for (int k4 = 0; k4 < D / 128; ++k4) vsc_lds[lane * (D / 128) + k4] = vsr[k4];
        }
      }
      wave_sync();

      // ---- P.V on the MFMA: A = probabilities (row c16, tokens KPL*g4 ..), B = V^T tiles
      // read transposed from LDS (column 16*dt + c16, the same tokens)
      bool rescale = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) rescale |= alpha[e] != 1.f;
      if (__builtin_amdgcn_read_exec() && rescale) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[dt][e] *= alpha[e];
      }
      float pv[KPL];
#pragma unroll
      for (int i = 0; i < KPL; ++i) pv[i] = c16 < RM ? p_lds[c16 * PSTR + KPL * g4 + i] : 0.f;
      PvOp pa[SC ? D / 32 : 1];
      if constexpr (SC) {
#pragma unroll
        for (int gg = 0; gg < D / 32; ++gg)
#pragma unroll
          for (int i = 0; i < KPL; ++i)
            pa[gg][i] = (_Float16)(pv[i] * (float)vsh[(KPL * g4 + i) * (D / 32) + gg]);
        if constexpr (DBG) {  // the chunk's V scales as used
          if (c16 == 0) {
#pragma unroll
            for (int i = 0; i < KPL; ++i) {
              const int jv = c0 + KPL * g4 + i;
              if (jv < tok_end) {
#pragma unroll
                for (int gg = 0; gg < D / 32; ++gg)
                  dbg_vs[dbg_row(jv) * (D / 32) + gg] = vsh[(KPL * g4 + i) * (D / 32) + gg];
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) pa[0][i] = (_Float16)pv[i];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        // lane (g4, c16) of read h receives column 16*dt + c16 of tokens KPL*g4 + 4h + 0..3
        PvOp vt;
#pragma unroll
        for (int h = 0; h < KPL / 4; ++h) {
          const int row = KPL * g4 + 4 * h + (c16 >> 2);
          const int col = 16 * dt + 4 * (c16 & 3);
          const short4v r4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4_ptr)(v_lds + swz<ROWB>(row, col >> 3) + ((col & 7) << 1)));
          const half4 hv = __builtin_bit_cast(half4, r4);
#pragma unroll
          for (int i = 0; i < 4; ++i) vt[4 * h + i] = hv[i];
        }
        const PvOp &pop = pa[SC ? dt / 2 : 0];
        if constexpr (CH == 32)
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, vt, acc[dt], 0, 0, 0);
        else
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pop, vt, acc[dt], 0, 0, 0);
      }
    } else {
      // ---- probabilities to LDS as f16 pairs (token 32h + c16, token 32h + 16 + c16) per row
      if (g4 < RB) {
#pragma unroll
        for (int h = 0; h < NT / 2; ++h) {
          uint4v w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = __builtin_bit_cast(unsigned,
                                      half2v{(_Float16)S[2 * h][e], (_Float16)S[2 * h + 1][e]});
          *(uint4v *)&p2_lds[(16 * h + c16) * RM + 4 * g4] = w;
        }
      }
      // per-row rescale factors (row-uniform within the 16 lanes of a DPP row)
      float al[RM];
#pragma unroll
      for (int r = 0; r < RM; ++r) al[r] = readlane_f(alpha[r & 3], 16 * (r >> 2));
      if constexpr (SC && !SCL) {
        if (lane < CH) {
#pragma unroll
          for (int k4 = 0; k4 < D / 128; ++k4) vsc_lds[lane * (D / 128) + k4] = vsr[k4];
        }
      }
      wave_sync();
      bool rescale = false;
#pragma unroll
      for (int r = 0; r < RM; ++r) rescale |= al[r] != 1.f;
      if (rescale) {
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i) accv[r][i] *= al[r];
      }
      // ---- P.V: in the 32 tokens from 32h, load steps s and s + SPT hold tokens tp and
      // tp + 16 of the lane's slot (SPT load steps per 16-token tile)
      constexpr int SPT = 16 / TPS;
#pragma unroll
      for (int ps = 0; ps < NS / 2; ++ps) {
        const int h = ps / SPT, s2 = 2 * SPT * h + ps % SPT, s3 = s2 + SPT;
        const int tp = 16 * h + TPS * (ps % SPT) + vlane_tok;
        half2v pp[RM];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          const uint4v w = *(const uint4v *)&p2_lds[tp * RM + 4 * q];
          // (bit_cast of a vector element would cast element 0: copy the element out first)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned we = w[e];
            pp[4 * q + e] = __builtin_bit_cast(half2v, we);
          }
        }
        half2v vp[8];
        if constexpr (F8) {
          f8_pairs(vb[s2], vb[s3], vp);  // fp8: v_scale * 2^8 is applied to the output
        } else if constexpr (SC) {
          // int8 V: the pair's per-32 scales fold into the probabilities
          const int ta = TPS * s2 + vlane_tok, g = vlane_el / 32;
          const half2v sc = {vsh[ta * (D / 32) + g], vsh[(ta + 16) * (D / 32) + g]};
          if constexpr (DBG) {  // the two tokens' V scales as used
            if ((vlane_el & 31) == 0) {
              if (c0 + ta < tok_end) dbg_vs[dbg_row(c0 + ta) * (D / 32) + g] = sc[0];
              if (c0 + ta + 16 < tok_end) dbg_vs[dbg_row(c0 + ta + 16) * (D / 32) + g] = sc[1];
            }
          }
#pragma unroll
          for (int r = 0; r < RM; ++r) pp[r] *= sc;
          if constexpr (Q4) q4_pairs(vb[s2], vb[s3], vp);
          else i8_pairs(vb[s2], vb[s3], vp);
        } else {
          h16_pairs(vb[s2], vb[s3], vp);
        }
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            accv[r][i] = __builtin_amdgcn_fdot2(pp[r], vp[i], accv[r][i], false);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- prefetch the next chunk's V while the next chunk's scores run
    if constexpr (PF) load_v(c1, pg_next);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PF) {
#pragma unroll
      for (int t = 0; t < NT; ++t) pg_cur[t] = pg_next[t];
    }
    wave_sync();
  };
  auto set_priority = [&](int c0) __attribute__((always_inline)) {
    if constexpr (!I8) return;  // f16 runs one wave per SIMD: nothing to arbitrate
    const int done = done_base + ((c0 - tok0) >> 6);
    if (done < pq1) __builtin_amdgcn_s_setprio(3);
    else if (done < pq2) __builtin_amdgcn_s_setprio(2);
    else if (done < pq3) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  // The last chunk peeled off (a third copy of the chunk's code) where registers allow: at
  // D = 128, and for f16 at D = 256; elsewhere it would add spills.
  constexpr bool PEEL = D == 128 || (D == 256 && !I8);
  if (tok0 < tok_end) {
    int c0 = tok0;
    if constexpr (PEEL) {
      if (c0 + CH < tok_end) {
        set_priority(c0);
        chunk(c0, std::true_type{});
        for (c0 += CH; c0 + CH < tok_end; c0 += CH) {
          set_priority(c0);
          chunk(c0, std::true_type{});
        }
      }
      set_priority(c0);
      chunk(c0, std::false_type{});
    } else {
      set_priority(c0);
      chunk(c0, std::true_type{});
      for (c0 += CH; c0 < tok_end; c0 += CH) {
        set_priority(c0);
        chunk(c0, std::true_type{});
      }
    }
  }
  done_base += blk_hi - blk_lo;
  if (a.debug && clamped_any) atomicOr(a.status, (unsigned)SKVD_STATUS_PAGE_CLAMPED);
  if constexpr (DBG) continue;  // the gather-debug variant writes no partial or output

  // ---- per-row sum over the tokens of the lane's DPP row; max is already row-uniform
#pragma unroll
  for (int e = 0; e < 4; ++e) lsum[e] = row16_sum(lsum[e]);
  const int Hq = a.Hq;
  // Partial index of output row `orow` (query row rr of this wave's KV head): static, the
  // split slot of the row; balanced, the compact slot's entry for this head and row (a slot
  // holds the RPG rows of one row group of each of the workgroup's KV heads).
  auto part_index = [&](int64_t orow, int rr) __attribute__((always_inline)) -> int64_t {
    return a.balanced ? ((int64_t)slot * HW + head_w) * RPG + (rr - rg * RPG)
                      : orow * a.part_stride + slot;
  };

  if constexpr (PVM) {
    // ---- output: lanes of group g4 hold rows row0 + 4*g4 + e, column 16*dt + c16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + 4 * g4 + e;
      if (g4 >= RB || r >= R) continue;
      const int t = r / G, hg = r - (r / G) * G;
      const int64_t row = ((int64_t)b * T + t) * Hq + kvh * G + hg;
      if (a.single) {
        const float l = lsum[e];
        const float inv = (l > 0.f ? 1.f / l : 0.f) * vfac;
        _Float16 *o = (_Float16 *)a.o + row * D + c16;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[16 * dt] = (_Float16)(acc[dt][e] * inv);
        if (a.lse && c16 == 0) a.lse[row] = l > 0.f ? (m[e] + __log2f(l)) * kLn2 : kNegInf;
      } else {
        float *dst = a.ws_o + part_index(row, hg + G * t) * D + c16;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) dst[16 * dt] = acc[dt][e] * vfac;
        if (c16 == 0) {
          float *ml = a.ws_ml + part_index(row, hg + G * t) * 2;
          ml[0] = m[e];
          ml[1] = lsum[e];
        }
      }
    }
  } else {
    // ---- sum the four load slots (lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same head_dim
    // elements of every row) as a reduce-scatter on the lane swaps: the first step leaves rows
    // 0 and 1 in lanes 0..31 and rows 2 and 3 in lanes 32..63, the second row g = lane / 16 in
    // lane group g (24 swaps and adds, where a butterfly per value took 64 LDS shuffles)
    static_assert(LPR == 16 && RM == 4, "the vector P.V holds four rows at head_dim 128");
    float w[2][8], u[8];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) w[r][i] = swap_sum32(accv[r][i], accv[r + 2][i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = swap_sum16(w[0][i], w[1][i]);
    const int g = lane >> 4;  // this lane group's row
    float mr[RM], lr[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      mr[r] = readlane_f(m[r], 0);
      lr[r] = readlane_f(lsum[r], 0);
    }
    const float mg = g == 0 ? mr[0] : g == 1 ? mr[1] : g == 2 ? mr[2] : mr[3];
    const float lg = g == 0 ? lr[0] : g == 1 ? lr[1] : g == 2 ? lr[2] : lr[3];
    if (g < R) {
      const int t = g / G, hg = g - t * G;
      const int64_t row = ((int64_t)b * T + t) * Hq + kvh * G + hg;
      if (a.single) {
        const float inv = (lg > 0.f ? 1.f / lg : 0.f) * vfac;
        half8 out;
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (_Float16)(u[i] * inv);
        if constexpr (Q4) {
          *(half4 *)((_Float16 *)a.o + row * D + vq0) = half4{out[0], out[1], out[2], out[3]};
          *(half4 *)((_Float16 *)a.o + row * D + vq1) = half4{out[4], out[5], out[6], out[7]};
        } else {
          *(half8 *)((_Float16 *)a.o + row * D + vlane_el) = out;
        }
        if (a.lse && (lane & 15) == 0) a.lse[row] = lg > 0.f ? (mg + __log2f(lg)) * kLn2 : kNegInf;
      } else {
        float *dst = a.ws_o + part_index(row, hg + G * t) * D;
        *(float4v *)(dst + vq0) = float4v{u[0], u[1], u[2], u[3]} * vfac;
        *(float4v *)(dst + vq1) = float4v{u[4], u[5], u[6], u[7]} * vfac;
        if ((lane & 15) == 0) {
          float *ml = a.ws_ml + part_index(row, hg + G * t) * 2;
          ml[0] = mg;
          ml[1] = lg;
        }
      }
    }
  }
  }  // segments
}


// ----------------------------------------------------------------------------- launch dispatch
// Tokens per chunk and P.V unit per variant. D=128 chunks hold 32 tokens, D=256 chunks 16
// (register bound; 64 int8 tokens at D=128 measured slower: two waves per SIMD). One query
// row quarter at D=128 takes the vector P.V (pair dot products from registers, no LDS copy
// of V); more rows, or D=256, make P.V a dense tile for the MFMA.
template <int D, int RB>
constexpr bool pv_on_mfma() {
  return !(D == 128 && RB == 1);
}
template <int D>
constexpr int chunk_tokens() {
  return D == 128 ? 32 : 16;
}

template <typename K>
static void launch_one(K kernel, unsigned grid, unsigned threads, hipStream_t st,
                       const KernelEvents &ev, const LaunchArgs &la) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, st, (hipEvent_t)ev.start,
                          (hipEvent_t)ev.stop, 0, la);
  else
    kernel<<<grid, threads, 0, st>>>(la);
}

template <int D, int RB, int KV, int HW, int RT, bool DBG>
static void launch_variant(const LaunchArgs &la, unsigned grid, hipStream_t st, bool fast,
                           const KernelEvents &ev) {
  constexpr int CH = chunk_tokens<D>();
  constexpr bool PVM = pv_on_mfma<D, RB>();
  if (fast)
    launch_one(partial_kernel<D, RB, KV, true, CH, PVM, HW, RT, DBG>, grid, 64 * HW * RT, st, ev,
               la);
  else
    launch_one(partial_kernel<D, RB, KV, false, CH, PVM, HW, RT, DBG>, grid, 64 * HW * RT, st, ev,
               la);
}

// Variant by the plan: row tiles (more than 16 query rows per KV head), else row quarters and,
// for the D=128 single-quarter variants, KV heads per workgroup (one wave each: the waves of a
// CU read each token's rows of those heads together; int8: and share the token's scale line).
template <int D, int KV, bool DBG>
static void launch_by_plan(const Plan &p, const LaunchArgs &la, unsigned grid, hipStream_t st,
                           const KernelEvents &ev) {
  const bool fast = p.prm.page_size >= 16;
  if (p.row_tiles == 4) return launch_variant<D, 4, KV, 1, 4, DBG>(la, grid, st, fast, ev);
  if (p.row_tiles == 2) return launch_variant<D, 4, KV, 1, 2, DBG>(la, grid, st, fast, ev);
  switch (p.row_blocks) {
    case 1:
      if constexpr (D == 128) {
        if (la.heads_per_wg == 8) return launch_variant<D, 1, KV, 8, 1, DBG>(la, grid, st, fast, ev);
        if (la.heads_per_wg == 4) return launch_variant<D, 1, KV, 4, 1, DBG>(la, grid, st, fast, ev);
        if (la.heads_per_wg == 2) return launch_variant<D, 1, KV, 2, 1, DBG>(la, grid, st, fast, ev);
      }
      return launch_variant<D, 1, KV, 1, 1, DBG>(la, grid, st, fast, ev);
    case 2: return launch_variant<D, 2, KV, 1, 1, DBG>(la, grid, st, fast, ev);
    default: return launch_variant<D, 4, KV, 1, 1, DBG>(la, grid, st, fast, ev);
  }
}

template <int D, int KV>
int launch_partial_fmt(const Plan &p, const LaunchArgs &la, unsigned grid, void *stream,
                       const KernelEvents &ev, bool dbg) {
  hipStream_t st = (hipStream_t)stream;
  if (dbg) launch_by_plan<D, KV, true>(p, la, grid, st, ev);
  else launch_by_plan<D, KV, false>(p, la, grid, st, ev);
  return (int)hipGetLastError();
}

}  // namespace skvd
