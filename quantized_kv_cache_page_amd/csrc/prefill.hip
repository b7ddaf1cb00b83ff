// Prefill / multi-token route: T > 8 query tokens per sequence against the paged cache, as MFMA
// tiles with int8, fp8 and q4_0 caches widened on their way into LDS (no f16 temporary in memory).
//
// llama-cpp-turboquant PR #176 ("HIP: fix turbo KV decode crash under graph capture;
// batch-aware VEC/TILE FA routing", section "Changes") keeps the vector decode path for at most
// 8 query tokens and sends larger batches to the tiled matrix-core kernel; its tiled path
// dequantized the whole cache into K_f16/V_f16 buffers first. Here the tile kernel reads the
// pages itself and widens int8 and fp8 bytes in registers.
//
// Work unit: one workgroup of 4 waves per (sequence b, KV head, tile of query tokens). Its
// query rows (128 at head_dim 128, 64 at 256) are (token, head-of-group) pairs r = token * G +
// g, so every wave reads the same KV head: K and V tiles of KT tokens are gathered through the
// page table into LDS once and shared by the 4 waves (one or two sets of 16 rows each). Per KV
// tile a wave computes S^T = K Q^T with the 16x16x32 f16 MFMA (A = 16 K rows from LDS, B = the
// wave's 16 query rows, held in registers), so each lane holds one query row's scores (column
// lane % 16) for 4 tokens per 16-token sub-tile; the online softmax (base 2) needs only per-lane
// work plus two cross-row lane swaps (v_permlane32_swap, v_permlane16_swap) for the max, and the
// row sums come from one more MFMA with an all-ones operand; the probabilities are already the
// B operand of O^T = V^T P^T, whose A operand (16 head_dim rows x 32 tokens of V) comes from LDS
// through transposing reads (ds_read_b64_tr_b16). The token order inside the contraction is the
// one the score layout gives (tokens 4g..4g+3 and 16+4g..16+4g+3 for lane group g); both
// operands use it.
//
// Causal reading (the decode's): the T query tokens are the last T cached positions, token t
// sees positions j <= kv_len - T + t. A workgroup walks positions [0, kv_len - T + t_last] in
// tiles, two LDS tile buffers deep, one barrier per tile. Two workgroups share a CU (256
// registers per lane each). Workgroups run heaviest (latest query tiles) first.
//
// Two ways into LDS. f16 caches with pages of 16+ tokens: copies straight from HBM into LDS
// (global_load_lds_dwordx4, no registers held), the next tile's copies in flight while the
// current one is computed. int8, fp8 and q4_0 caches, and pages of fewer than 16 tokens: the
// next tile's rows are loaded into registers during the compute, widened (one-byte formats)
// and stored into the other buffer (a second register stage does not fit: the allocator then
// serializes the stages).
#include <hip/hip_runtime.h>

#include "skvd_internal.h"

namespace skvd {
namespace {

typedef _Float16 ph8 __attribute__((ext_vector_type(8)));
typedef _Float16 ph4 __attribute__((ext_vector_type(4)));
typedef float pf4 __attribute__((ext_vector_type(4)));
typedef short ps4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) ps4 *lds_ps4;
typedef unsigned pu4 __attribute__((ext_vector_type(4)));

constexpr float kPNegInf = -__builtin_huge_valf();
constexpr float kPLn2 = 0.6931471805599453f;
constexpr float kMFloor = -1e30f;  // running max before any visible score (keeps exp2 finite)
// s_waitcnt operand on gfx9: vector-memory count 0, export and LDS/scalar counts unchanged (at
// their maxima 7 and 15)
constexpr int kVmcntZero = 0x0F70;

// Byte offset of 16-byte chunk c of row r in an LDS tile with rows of ROWB bytes (256 or 512:
// a row starts on bank 0, a chunk's banks are set by c mod 8). The chunk is XOR-swizzled so that
// no access pattern is bank-conflicted:
//  - transposed V reads fetch 32 contiguous bytes (chunks 2j, 2j+1) of 4 consecutive rows per
//    16-lane phase: swizzle bits 1-2 take the row's low 2 bits (4 different 32-byte bank groups);
//  - K reads fetch one chunk of 8 consecutive rows per 8-lane phase: the row swizzle is a
//    bijection of the row's low 3 bits (8 different chunks mod 8);
//  - f16 tile stores (head_dim 128) write 4 consecutive chunks of each of two rows per phase:
//    the two rows' swizzles differ in bit 2 (row bit 0 goes to bit 2);
//  - one-byte tile stores write chunk 4q + c of a row from its q-th thread (each widened 16-byte
//    load fills 4 chunks): the column term moves chunk bit 3 to bit 1 and bit 4 to bit 0, so the
//    threads of a row land on different chunks mod 8, and the two rows of a phase differ in
//    swizzle bit 0 (row bit 0 goes to bit 0).
// The reads see a column term that is constant over a read (one chunk, or a 2j / 2j+1 pair).
template <int ROWB, bool ONEB>
__device__ __forceinline__ int pswz(int r, int c) {
  const int x = ONEB ? (((r & 1) ^ ((r >> 2) & 1)) | ((r & 3) << 1) | (r & 8))
                     : (((r & 1) << 2) | (r & 2) | ((r >> 2) & 1) | (r & 8));
  const int col = ONEB ? (((c >> 3) & 1) << 1) | ((c >> 4) & 1) : 0;
  return r * ROWB + ((c ^ x ^ col) << 4);
}

template <int D>
constexpr int kv_tile() { return D == 128 ? 64 : 32; }

// Max over the four lanes l, l^16, l^32, l^48 (the four lane groups holding one query row's
// scores) with the cross-row swaps of the vector ALU: each swap exchanges halves between two
// copies of x, so combining the two results combines lane pairs, whichever copy got which.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// One KV tile's rows held in registers between the global load and the LDS store. Each thread
// serves one token of the tile (TPT threads per token) and N 16-byte chunks of its K and V rows
// (f16: every TPT-th chunk from its own; one-byte formats: N consecutive chunks, one scale group),
// so it reads one page-table entry and forms one row address per tile. The loads
// are ordinary (cached): every query tile of the sequence reads the same K/V tiles, so they
// should stay in L2 and the Infinity Cache (non-temporal loads here cost 12-37 %).
template <int D, int KV, int NTH>
struct TileRegs {
  static constexpr bool I8 = KV != 0;  // one-byte layout (int8, fp8, q4_0)
  static constexpr int KT = kv_tile<D>();
  // 16-byte chunks of a row: f16 8 elements; int8 and fp8 16 elements (int8: + their scale);
  // q4_0 one 32-element group of codes (+ its scale)
  static constexpr int CPR = KV == 3 ? D / 32 : I8 ? D / 16 : D / 8;  // chunks per row
  static constexpr int TPT = NTH / KT;             // threads per token (NTH: the workgroup's)
  static constexpr int N = CPR / TPT;              // chunks per thread per tensor
  static_assert(N >= 1, "at least one chunk per thread");
  pu4 k[N], v[N];
  _Float16 ks[I8 ? N : 1], vs[I8 ? N : 1];
  // int8 and q4_0 with four threads per token (D = 128; thread q of the quad serves group q):
  // the token's K scales (thread 0 of the quad) or V scales (thread 1), all four groups in one
  // 8-byte load, shared over the quad by DPP
  static constexpr bool kQuadScales =
      TPT == 4 && ((KV == 1 && N == 2) || (KV == 3 && N == 1));
  unsigned sq[2];
};

// The page-table entry of this thread's token in the KV tile at kv0 (a tail token re-reads the
// tile's last one). Read one tile ahead of the tile's loads, so that its latency is not on the
// loop's path. PT (pages of at least 16 tokens): a wave's tokens of a tile (16 at head_dim 128,
// 8 at 256, aligned) lie in one page, so the entry is wave-uniform and read by a scalar load
// through the constant address space; the vector-memory count then holds tile loads only and
// the loop's waits for a page entry do not also wait for the tile loads issued after it.
template <int D, bool I8, int NTH, bool PT>
__device__ __forceinline__ int tile_page(const LaunchArgs &a, int b, int kv0, int kv_last) {
  using TR = TileRegs<D, I8 ? 1 : 0, NTH>;  // (threads per token: the same for every format)
  if constexpr (PT) {
    typedef const __attribute__((address_space(4))) int32_t *ctab_t;
    const int wave_tok = (int)(threadIdx.x & ~63u) / TR::TPT;  // the wave's first token
    const int tok = __builtin_amdgcn_readfirstlane(min(kv0 + wave_tok, kv_last));
    return ((ctab_t)a.table)[(int64_t)b * a.table_stride + (tok >> a.page_shift)];
  } else {
    const int tok = min(kv0 + (int)threadIdx.x / TR::TPT, kv_last);
    return a.table[(int64_t)b * a.table_stride + (tok >> a.page_shift)];
  }
}

// KV: 0 f16, 1 int8 with per-32 f16 scales, 2 fp8 E4M3 with one f32 scale per tensor, 3 q4_0
// (rows of D/2 code bytes, per-32 f16 scales; a thread loads whole groups). The one-byte
// formats share the int8 tile layout in LDS. pg: the thread's tile_page entry for this tile.
template <int D, int KV, int NTH>
__device__ __forceinline__ void load_tile(const LaunchArgs &a, int kvh, int kv0, int kv_last,
                                          int pg, TileRegs<D, KV, NTH> &r) {
  constexpr bool I8 = KV != 0;
  using TR = TileRegs<D, KV, NTH>;
  const int P1 = (1 << a.page_shift) - 1;
  const int tok = min(kv0 + (int)threadIdx.x / TR::TPT, kv_last);  // tail re-reads (masked)
  const int part0 = ((int)threadIdx.x % TR::TPT) * TR::N;  // one-byte: chunks part0 .. + N - 1
  const int q0 = (int)threadIdx.x % TR::TPT;                 // f16: chunks q0 + TPT * n
  const int64_t pk = pg < 0 ? 0 : (pg >= a.num_k_pages ? a.num_k_pages - 1 : pg);
  const int64_t pv = pg < 0 ? 0 : (pg >= a.num_v_pages ? a.num_v_pages - 1 : pg);
  const int64_t in_page = (int64_t)(tok & P1) * a.tok_stride + (int64_t)kvh * a.head_stride;
  const int64_t rk = pk * a.page_stride + in_page;
  const int64_t rv = pv * a.page_stride + in_page;
  if constexpr (!I8) {
    const pu4 *kp = (const pu4 *)((const _Float16 *)a.k + rk) + q0;
    const pu4 *vp = (const pu4 *)((const _Float16 *)a.v + rv) + q0;
#pragma unroll
    for (int n = 0; n < TR::N; ++n) {
      r.k[n] = kp[TR::TPT * n];
      r.v[n] = vp[TR::TPT * n];
    }
  } else {
    const pu4 *kp = (const pu4 *)((const int8_t *)a.k + rk) + part0;
    const pu4 *vp = (const pu4 *)((const int8_t *)a.v + rv) + part0;
    if constexpr (KV == 2) {
#pragma unroll
      for (int n = 0; n < TR::N; ++n) {
        r.k[n] = kp[n];
        r.v[n] = vp[n];
      }
      return;
    }
    const int64_t s_in_page = (int64_t)(tok & P1) * a.s_tok_stride + (int64_t)kvh * a.s_head_stride;
    const _Float16 *ksp = (const _Float16 *)a.ks + pk * a.s_page_stride + s_in_page;
    const _Float16 *vsp = (const _Float16 *)a.vs + pv * a.s_page_stride + s_in_page;
#pragma unroll
    for (int n = 0; n < TR::N; ++n) {
      r.k[n] = kp[n];
      r.v[n] = vp[n];
      if constexpr (!TR::kQuadScales) {
        // int8: a 16-element chunk lies in scale group chunk / 2; q4_0: chunk = group
        r.ks[n] = ksp[KV == 3 ? part0 + n : (part0 + n) >> 1];
        r.vs[n] = vsp[KV == 3 ? part0 + n : (part0 + n) >> 1];
      }
    }
    if constexpr (TR::kQuadScales) {
      const unsigned q = threadIdx.x & 3u;
      const _Float16 *sp = q == 0 ? ksp : vsp;  // threads 2 and 3 re-read V's line (unused)
      typedef unsigned su2 __attribute__((ext_vector_type(2)));
      const su2 sv = *(const su2 *)sp;
      r.sq[0] = sv[0];
      r.sq[1] = sv[1];
    }
  }
}

// 16 signed bytes -> two groups of 8 f16, each times the f16 scale (one rounding, as the
// decode's K path). Exact widening without per-element conversions: flipping each byte's sign
// bit gives u = x + 128 as an unsigned byte; a byte permute places u under the f16 exponent
// byte of 1024 (the f16 with bits 0x64uu is 1024 + u, exactly); one packed subtract of 1152
// leaves x exactly; one packed multiply applies the scale.
typedef _Float16 ph2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ ph2 magic_pair16(unsigned flipped, unsigned sel) {
  return __builtin_bit_cast(ph2, __builtin_amdgcn_perm(0x64646464u, flipped, sel)) -
         (ph2)(_Float16)1152;
}

__device__ __forceinline__ void widen16(pu4 w, _Float16 s, ph8 *lo, ph8 *hi) {
  const ph2 s2 = {s, s};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned x = w[k] ^ 0x80808080u;
    const ph2 a = magic_pair16(x, 0x04010400u) * s2;  // bytes 0, 1
    const ph2 b = magic_pair16(x, 0x04030402u) * s2;  // bytes 2, 3
    ph8 &dst = k < 2 ? *lo : *hi;
    const int e0 = 4 * (k & 1);
    dst[e0 + 0] = a[0];
    dst[e0 + 1] = a[1];
    dst[e0 + 2] = b[0];
    dst[e0 + 3] = b[1];
  }
}

// 16 E4M3 bytes -> two groups of 8 f16 holding value * 2^-8 exactly, two bytes per conversion
// instruction (power-of-two scale 2^-8: every E4M3 value, subnormals included, is exact in f16).
// The 2^8 and the tensor scales are applied to the score scale (K) and the output (V).
__device__ __forceinline__ void widen16_f8(pu4 w, ph8 *lo, ph8 *hi) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const ph2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 0.00390625f, false);  // bytes 0, 1
    const ph2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[k], 0.00390625f, true);   // bytes 2, 3
    ph8 &dst = k < 2 ? *lo : *hi;
    const int e0 = 4 * (k & 1);
    dst[e0] = a[0];
    dst[e0 + 1] = a[1];
    dst[e0 + 2] = b[0];
    dst[e0 + 3] = b[1];
  }
}

// One q4_0 group (16 code bytes: byte i holds element i in its low nibble and element 16 + i in
// its high nibble) -> four groups of 8 f16, (c - 8) times the f16 scale (one rounding, as the
// int8 path): a nibble c placed under the f16 exponent byte of 1024 is 1024 + c exactly; one
// packed subtract of 1032 leaves c - 8 exactly; one packed multiply applies the scale.
__device__ __forceinline__ void widen_q4(pu4 w, _Float16 s, ph8 *c) {
  const ph2 s2 = {s, s};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned lo = w[k] & 0x0F0F0F0Fu, hi = (w[k] >> 4) & 0x0F0F0F0Fu;
    const int e0 = 4 * (k & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned nib = h ? hi : lo;
      const ph2 a = (__builtin_bit_cast(ph2, __builtin_amdgcn_perm(0x64646464u, nib, 0x04010400u)) -
                     (ph2)(_Float16)1032) * s2;  // bytes 0, 1
      const ph2 b = (__builtin_bit_cast(ph2, __builtin_amdgcn_perm(0x64646464u, nib, 0x04030402u)) -
                     (ph2)(_Float16)1032) * s2;  // bytes 2, 3
      ph8 &dst = c[2 * h + (k >> 1)];  // elements 4k .. 4k+3 (low) or 16 + 4k .. (high)
      dst[e0] = a[0];
      dst[e0 + 1] = a[1];
      dst[e0 + 2] = b[0];
      dst[e0 + 3] = b[1];
    }
  }
}

// Broadcast of a quad's lane L (quad_perm [L, L, L, L]).
template <int L>
__device__ __forceinline__ unsigned quad_bcast(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, L * 0x55, 0xF, 0xF, false);
}

template <int D, int KV, int NTH>
__device__ __forceinline__ void store_tile(char *k_lds, char *v_lds,
                                           const TileRegs<D, KV, NTH> &r) {
  constexpr bool I8 = KV != 0;
  using TR = TileRegs<D, KV, NTH>;
  _Float16 qks = 0, qvs = 0;  // kQuadScales: this thread's group (its quad index) of K and V
  if constexpr (TR::kQuadScales) {
    const unsigned q = threadIdx.x & 3u;
    const unsigned k0 = quad_bcast<0>(r.sq[0]), k1 = quad_bcast<0>(r.sq[1]);
    const unsigned v0 = quad_bcast<1>(r.sq[0]), v1 = quad_bcast<1>(r.sq[1]);
    const unsigned kw = q < 2 ? k0 : k1, vw = q < 2 ? v0 : v1;
    const unsigned sh = (q & 1u) * 16u;
    qks = __builtin_bit_cast(_Float16, (unsigned short)(kw >> sh));
    qvs = __builtin_bit_cast(_Float16, (unsigned short)(vw >> sh));
  }
  constexpr int ROWB = D * 2;
  const int tok = (int)threadIdx.x / TR::TPT;
#pragma unroll
  for (int n = 0; n < TR::N; ++n) {
    // (f16: chunk q0 + TPT * n, so that the 4 threads of a token store 4 consecutive chunks)
    const int part = I8 ? ((int)threadIdx.x % TR::TPT) * TR::N + n
                        : (int)threadIdx.x % TR::TPT + TR::TPT * n;
    if constexpr (!I8) {
      *(pu4 *)(k_lds + pswz<ROWB, false>(tok, part)) = r.k[n];
      *(pu4 *)(v_lds + pswz<ROWB, false>(tok, part)) = r.v[n];
    } else if constexpr (KV == 3) {
      // one group: f16 chunks 4 part .. + 3 of the row (the int8 layout's chunks of this thread)
      ph8 c4[4];
      widen_q4(r.k[n], TR::kQuadScales ? qks : r.ks[n], c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) *(ph8 *)(k_lds + pswz<ROWB, true>(tok, 4 * part + j)) = c4[j];
      widen_q4(r.v[n], TR::kQuadScales ? qvs : r.vs[n], c4);
#pragma unroll
      for (int j = 0; j < 4; ++j) *(ph8 *)(v_lds + pswz<ROWB, true>(tok, 4 * part + j)) = c4[j];
    } else {
      ph8 lo, hi;
      if constexpr (KV == 2) widen16_f8(r.k[n], &lo, &hi);
      else widen16(r.k[n], TR::kQuadScales ? qks : r.ks[n], &lo, &hi);
      *(ph8 *)(k_lds + pswz<ROWB, true>(tok, 2 * part)) = lo;
      *(ph8 *)(k_lds + pswz<ROWB, true>(tok, 2 * part + 1)) = hi;
      if constexpr (KV == 2) widen16_f8(r.v[n], &lo, &hi);
      else widen16(r.v[n], TR::kQuadScales ? qvs : r.vs[n], &lo, &hi);
      *(ph8 *)(v_lds + pswz<ROWB, true>(tok, 2 * part)) = lo;
      *(ph8 *)(v_lds + pswz<ROWB, true>(tok, 2 * part + 1)) = hi;
    }
  }
}

// Row sets per wave: each wave serves RS sets of 16 query rows, so every K fragment and every
// transposed V fragment it reads from LDS feeds RS MFMAs (LDS traffic per FLOP / RS).
template <int D>
constexpr int row_sets() { return D == 128 ? 2 : 1; }

// Waves per workgroup: 4, two workgroups per CU (8 waves sharing each tile, one workgroup per
// CU, measured no faster for f16 and slower for the one-byte formats).
template <int D>
constexpr int prefill_waves() { return 4; }

template <int D, int KV, int NW, bool PT>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void prefill_kernel(LaunchArgs a, int tpw,
                                                                         int qtiles) {
  constexpr int NTH = 64 * NW;  // threads per workgroup
  constexpr bool I8 = KV != 0;
  constexpr int KT = kv_tile<D>();
  constexpr int RS = row_sets<D>();
  constexpr int NST = KT / 16;   // 16-token score sub-tiles per KV tile
  constexpr int NCH = KT / 32;   // 32-token P.V chunks per KV tile
  constexpr int NKS = D / 32;    // contraction steps over head_dim
  constexpr int NDT = D / 16;    // 16-wide head_dim tiles of the output
  constexpr int ROWB = D * 2;
  // two K/V tile buffers: tile i+1 is stored into one while tile i is read from the other
  __shared__ __attribute__((aligned(16))) char kv_lds[2][2][KT * ROWB];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  // Work item of this workgroup: (sequence b, KV head, query tile). Workgroups are handed to
  // the 8 XCDs in turn (linear id mod 8), and every query tile of one (sequence, KV head) pair
  // re-reads that pair's K/V tiles, so the items of a pair go to one XCD: their tiles then stay
  // in one L2 instead of being fetched into all eight. When the pairs divide evenly, pairs
  // x, x+8, ... go to XCD x, latest (heaviest) query tiles of all of them first. Otherwise XCD x
  // takes a contiguous run of the (pair, query tile) list -- as many items as ids = x mod 8 --
  // heaviest tile of each pair first; only the pairs cut at a run's ends span two XCDs.
  const int pairs = a.Hkv * a.batch;
  const int id = blockIdx.x;
  const int x = id % 8, k = id / 8;
  int pair, qt;
  if (pairs % 8 == 0) {
    const int per_xcd = pairs / 8;
    qt = qtiles - 1 - k / per_xcd;
    pair = x + 8 * (k % per_xcd);
  } else {
    const int n = qtiles * pairs;  // the grid: ids with id % 8 == y number ceil((n - y) / 8)
    const int base = n / 8, extra = n % 8;
    const int item = x * base + min(x, extra) + k;  // runs of XCDs 0..x-1 come first
    pair = item / qtiles;
    qt = qtiles - 1 - item % qtiles;
  }
  const int kvh = pair % a.Hkv, b = pair / a.Hkv;
  const int G = a.G, T = a.T;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
  const int t0 = qt * tpw;
  const int t_last = min(t0 + tpw, T) - 1;
  const int kv_end = min(L, L - T + t_last + 1);  // positions [0, kv_end) are visited

  // this lane's query rows: column c16 of each of the wave's row sets (r = token * G + head)
  bool row_ok[RS];
  int trow[RS], hrow[RS], limit[RS];
  ph8 qv[RS][NKS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int r = 16 * (RS * w + rs) + c16;
    const int tl = r / G;
    const int gh = r - tl * G;
    row_ok[rs] = tl < tpw && t0 + tl < T;
    trow[rs] = row_ok[rs] ? t0 + tl : t_last;
    hrow[rs] = kvh * G + gh;
    limit[rs] = L - T + trow[rs];  // last visible position of the row
    const _Float16 *qp = (const _Float16 *)a.q + ((int64_t)b * T + trow[rs]) * a.q_tok_stride +
                         (int64_t)hrow[rs] * a.q_head_stride + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qv[rs][ks] = *(const ph8 *)(qp + 32 * ks);
  }

  // Scores are scaled inside the exponent, p = 2^(s c - m) with c = sm_scale * log2(e) > 0,
  // so the max is taken on unscaled scores and scaled once. A negative scale is carried by q
  // (negating f16 is exact); a zero scale by a tiny c (masked scores stay -inf, others ~0).
  float c = a.scale_log2;
  if constexpr (KV == 2) c *= *(const float *)a.ks * 256.0f;  // fp8: k_scale and the 2^8
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qv[rs][ks] = -qv[rs][ks];
  }
  c = fmaxf(c, 1e-30f);

  // acc: O^T tiles; lacc: the row sums, as one more MFMA tile whose A operand is all ones (every
  // lane then holds its row's sum of the f16 probabilities that the P.V tiles also use, with no
  // vector adds or cross-lane sums)
  pf4 acc[RS][NDT], lacc[RS];
  float m[RS];
  const ph8 ones = (ph8)(_Float16)1;
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[rs][dt] = pf4{0.f, 0.f, 0.f, 0.f};
    lacc[rs] = pf4{0.f, 0.f, 0.f, 0.f};
    m[rs] = kMFloor;
  }

  const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;
  // The next tile's loads run one step ahead of its use, its page-table entries one more.
  TileRegs<D, KV, NTH> regs;
  int pg_ahead = 0;           // the page entry of the next tile to be loaded
  if (ntiles > 0) {
    load_tile<D, KV, NTH>(a, kvh, 0, kv_end - 1, tile_page<D, I8, NTH, PT>(a, b, 0, kv_end - 1),
                          regs);
    if (ntiles > 1) pg_ahead = tile_page<D, I8, NTH, PT>(a, b, KT, kv_end - 1);
    store_tile<D, KV, NTH>(kv_lds[0][0], kv_lds[0][1], regs);
  }
  // Every load issued so far (q rows, the first tiles, page entries) is complete here. Stated
  // explicitly: the loop's first use of the q registers otherwise inherits, through the merge
  // of the loop entry with the back edge, a wait for the vector loads the loop itself issues,
  // i.e. a wait for the next tile right after its loads are issued.
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int kv0 = it * KT;
    const char *k_lds = kv_lds[it & 1][0];
    const char *v_lds = kv_lds[it & 1][1];
    // the next tile's loads; its successor's page entry first (requested before the tile loads,
    // so that the next step waits for the entry alone)
    const int pg_use = pg_ahead;
    if (it + 2 < ntiles) pg_ahead = tile_page<D, I8, NTH, PT>(a, b, (it + 2) * KT, kv_end - 1);
    if (it + 1 < ntiles) load_tile<D, KV, NTH>(a, kvh, (it + 1) * KT, kv_end - 1, pg_use, regs);

    // ---- S^T = K Q^T: lane holds row c16's scores for tokens 16 st + 4 g4 + e
    pf4 s[RS][NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) s[rs][st] = pf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const ph8 kf = *(const ph8 *)(k_lds + pswz<ROWB, I8>(16 * st + c16, 4 * ks + g4));
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
          s[rs][st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qv[rs][ks], s[rs][st], 0, 0, 0);
      }
    }
    // ---- mask (only tiles that reach past the first row's limit), scale (base 2), online
    // softmax per row set. The reference max m is raised only when a score exceeds it by more
    // than 2^8 in weight (then the accumulators are rescaled); otherwise probabilities up to 2^8
    // are taken against the old reference, which the final o = acc / l and lse = m + log2 l
    // absorb exactly.
    const bool need_mask = kv0 + KT - 1 > L - T + t0;  // workgroup-uniform
    ph8 pb[RS][NCH];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      // the max of the unscaled scores (c > 0), scaled once per row
      float mx = kPNegInf;
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = kv0 + 16 * st + 4 * g4 + e;
            const float v = pos <= limit[rs] ? s[rs][st][e] : kPNegInf;
            s[rs][st][e] = v;
            mx = fmaxf(mx, v);
          }
      } else {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[rs][st][e]);
      }
      mx = rows4_max(mx) * c;
      const bool raise = mx > m[rs] + 8.f;
      if (__any(raise)) {
        const float m_new = raise ? mx : m[rs];
        const float alpha = __builtin_amdgcn_exp2f(m[rs] - m_new);
        m[rs] = m_new;
#pragma unroll
        for (int e = 0; e < 4; ++e) lacc[rs][e] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rs][dt][e] *= alpha;
      }
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[rs][st][e] = __builtin_amdgcn_exp2f(fmaf(s[rs][st][e], c, -m[rs]));
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[rs][c][e] = (_Float16)s[rs][2 * c][e];
          pb[rs][c][4 + e] = (_Float16)s[rs][2 * c + 1][e];
        }
    }
    // ---- O^T += V^T P^T, 32 tokens per MFMA
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        ph8 va;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // lane (g4, c16) receives column 16 dt + c16 of tokens 32 c + 16 hh + 4 g4 + 0..3
          const int row = 32 * c + 16 * hh + 4 * g4 + (c16 >> 2);
          const int col = 16 * dt + 4 * (c16 & 3);
          const ps4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_ps4)(const_cast<char *>(v_lds) + pswz<ROWB, I8>(row, col >> 3) +
                        ((col & 7) << 1)));
          const ph4 hv = __builtin_bit_cast(ph4, r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) va[4 * hh + e] = hv[e];
        }
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
          acc[rs][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[rs][c], acc[rs][dt], 0, 0, 0);
      }
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
        lacc[rs] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[rs][c], lacc[rs], 0, 0, 0);
    }
    // the other buffer was last read in the previous iteration, which every wave has left
    if (it + 1 < ntiles)
      store_tile<D, KV, NTH>(kv_lds[(it + 1) & 1][0], kv_lds[(it + 1) & 1][1], regs);
    __syncthreads();  // tile it+1 is in LDS, and every wave is done reading tile it
  }

  // ---- epilogue: row sums across the four lane groups, normalize, write o and lse
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const float lt = lacc[rs][0];
    if (!row_ok[rs]) continue;
    const int64_t orow = ((int64_t)b * T + trow[rs]) * a.Hq + hrow[rs];
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (KV == 2) inv *= *(const float *)a.vs * 256.0f;  // fp8: v_scale and the 2^8
    _Float16 *op = (_Float16 *)a.o + orow * D + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      ph4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (_Float16)(acc[rs][dt][e] * inv);
      *(ph4 *)(op + 16 * dt) = ov;
    }
    if (g4 == 0 && a.lse) a.lse[orow] = lt > 0.f ? (m[rs] + __log2f(lt)) * kPLn2 : kPNegInf;
  }
}

// ---- f16 caches with pages of 16+ tokens: K/V tiles copied from HBM straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base + 16 * lane, no
// registers held), NSTG tile buffers deep, so that a tile's loads are issued NSTG - 1 tiles
// before its use. Each lane loads the global chunk that the tile's swizzle puts at its LDS
// slot. A wave waits for its own copies of a tile explicitly (vector-memory count, the copies of
// the later tiles still in flight) before the barrier that publishes the tile; the loop holds no
// other vector-memory operation, so the count is exact.

// s_waitcnt operand: vector-memory count n (0..63), export and LDS/scalar counts at their maxima
template <int N>
constexpr int vmcnt_imm() { return (N & 15) | ((N >> 4) << 14) | 0x0F70; }

template <int D, int KT, int NW>
struct DmaTile {
  static constexpr int ROWB = D * 2;             // bytes per K or V row in LDS
  static constexpr int RPS = 1024 / ROWB;        // rows per wave copy (64 lanes x 16 bytes)
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int SPW = KT * ROWB / 1024 / NW;  // copies per wave per tensor and tile
  static constexpr int RPW = SPW * RPS;          // rows (tokens) per wave: 8 or 16, one page
  static constexpr int BYTES = KT * ROWB;        // one tensor's tile
  static_assert(SPW >= 1 && KT * ROWB == 1024 * NW * SPW, "tile not a whole number of copies");
  static_assert(RPW <= 16, "a wave's tokens must lie in one 16-token group");
};

// The page-table entry of wave w's tokens of the tile at kv0 (wave-uniform for pages of 16+
// tokens, scalar load; a tail token is clamped to the last visited position).
template <int D, int KT, int NW>
__device__ __forceinline__ int dma_page(const LaunchArgs &a, int b, int w, int kv0, int kv_last) {
  using DT = DmaTile<D, KT, NW>;
  typedef const __attribute__((address_space(4))) int32_t *ctab_t;
  const int tok = __builtin_amdgcn_readfirstlane(min(kv0 + DT::RPW * w, kv_last));
  return ((ctab_t)a.table)[(int64_t)b * a.table_stride + (tok >> a.page_shift)];
}

// Issue the copies of wave w's rows of the K and V tile at kv0 into k_lds / v_lds. The wave's
// rows lie in one page (pg, the entry of its first visited token tw): a scalar base at token tw
// of that page plus a 32-bit lane offset (fewer than 16 rows further, within the 32-bit in-tile
// range the host checks).
template <int D, int KT, int NW>
__device__ __forceinline__ void dma_tile(const LaunchArgs &a, int kvh, int w, int kv0,
                                         int kv_last, int pg, char *k_lds, char *v_lds) {
  using DT = DmaTile<D, KT, NW>;
  typedef __attribute__((address_space(3))) void *lds_t;
  const int lane = threadIdx.x & 63;
  const int P1 = (1 << a.page_shift) - 1;
  const int tw = __builtin_amdgcn_readfirstlane(min(kv0 + DT::RPW * w, kv_last));
  const int64_t pk = pg < 0 ? 0 : (pg >= a.num_k_pages ? a.num_k_pages - 1 : pg);
  const int64_t pv = pg < 0 ? 0 : (pg >= a.num_v_pages ? a.num_v_pages - 1 : pg);
  const int64_t in_page = (int64_t)(tw & P1) * a.tok_stride + (int64_t)kvh * a.head_stride;
  const char *kb = (const char *)((const _Float16 *)a.k + pk * a.page_stride + in_page);
  const char *vb = (const char *)((const _Float16 *)a.v + pv * a.page_stride + in_page);
  const unsigned ts = (unsigned)a.tok_stride * 2u;     // bytes per token
  const int rl = lane / DT::CPR, pc = lane % DT::CPR;  // row within the copy, LDS chunk
#pragma unroll
  for (int j = 0; j < DT::SPW; ++j) {
    const int seg = w * DT::SPW + j;
    const int row = seg * DT::RPS + rl;
    const int tok = min(kv0 + row, kv_last);
    // the chunk whose swizzled place is LDS chunk pc of this row (the swizzle is an XOR)
    const int c = (pswz<DT::ROWB, false>(row, pc) - row * DT::ROWB) >> 4;
    const unsigned off = (unsigned)(tok - tw) * ts + 16u * (unsigned)c;
    __builtin_amdgcn_global_load_lds((const void *)(kb + off), (lds_t)(k_lds + seg * 1024), 16, 0,
                                     0);
    __builtin_amdgcn_global_load_lds((const void *)(vb + off), (lds_t)(v_lds + seg * 1024), 16, 0,
                                     0);
  }
}

template <int D, int NW, int KT, int NSTG>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void prefill_dma_kernel(LaunchArgs a,
                                                                             int tpw, int qtiles) {
  using DT = DmaTile<D, KT, NW>;
  static_assert(NSTG >= 2 && NSTG <= 4, "two to four tile buffers");
  constexpr int RS = row_sets<D>();
  constexpr int NST = KT / 16;
  constexpr int NCH = KT / 32;
  constexpr int NKS = D / 32;
  constexpr int NDT = D / 16;
  constexpr int ROWB = D * 2;
  // NSTG tile buffers (K then V in each)
  __shared__ __attribute__((aligned(1024))) char stg[NSTG][2 * DT::BYTES];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  // work item: as in prefill_kernel (the query tiles of one (sequence, KV head) pair on one XCD,
  // heaviest first)
  const int pairs = a.Hkv * a.batch;
  const int id = blockIdx.x;
  const int x = id % 8, k = id / 8;
  int pair, qt;
  if (pairs % 8 == 0) {
    const int per_xcd = pairs / 8;
    qt = qtiles - 1 - k / per_xcd;
    pair = x + 8 * (k % per_xcd);
  } else {
    const int n = qtiles * pairs;
    const int base = n / 8, extra = n % 8;
    const int item = x * base + min(x, extra) + k;
    pair = item / qtiles;
    qt = qtiles - 1 - item % qtiles;
  }
  const int kvh = pair % a.Hkv, b = pair / a.Hkv;
  const int G = a.G, T = a.T;
  int L = a.kv_len[b];
  L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
  const int t0 = qt * tpw;
  const int t_last = min(t0 + tpw, T) - 1;
  const int kv_end = min(L, L - T + t_last + 1);
  const int kv_last = kv_end - 1;

  bool row_ok[RS];
  int trow[RS], hrow[RS], limit[RS];
  ph8 qv[RS][NKS];
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const int r = 16 * (RS * w + rs) + c16;
    const int tl = r / G;
    const int gh = r - tl * G;
    row_ok[rs] = tl < tpw && t0 + tl < T;
    trow[rs] = row_ok[rs] ? t0 + tl : t_last;
    hrow[rs] = kvh * G + gh;
    limit[rs] = L - T + trow[rs];
    const _Float16 *qp = (const _Float16 *)a.q + ((int64_t)b * T + trow[rs]) * a.q_tok_stride +
                         (int64_t)hrow[rs] * a.q_head_stride + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qv[rs][ks] = *(const ph8 *)(qp + 32 * ks);
  }
  float c = a.scale_log2;
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qv[rs][ks] = -qv[rs][ks];
  }
  c = fmaxf(c, 1e-30f);

  pf4 acc[RS][NDT], lacc[RS];
  float m[RS];
  const ph8 ones = (ph8)(_Float16)1;
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[rs][dt] = pf4{0.f, 0.f, 0.f, 0.f};
    lacc[rs] = pf4{0.f, 0.f, 0.f, 0.f};
    m[rs] = kMFloor;
  }

  const int ntiles = kv_end > 0 ? (kv_end + KT - 1) / KT : 0;

  // Per-lane LDS read offsets within a buffer, the same for every buffer: K fragment of step
  // ks (16-row sub-tile st adds 16 rows), V fragment of head_dim tile dt (the 32-token chunk and
  // its 16-token half add whole rows). The swizzle depends on the row's low 4 bits only.
  int koff[NKS], voff[NDT];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = pswz<ROWB, false>(c16, 4 * ks + g4);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int row = 4 * g4 + (c16 >> 2), col = 16 * dt + 4 * (c16 & 3);
    voff[dt] = pswz<ROWB, false>(row, col >> 3) + ((col & 7) << 1);
  }

  // Scores of one tile, S^T = K Q^T: lane holds row c16's scores for tokens 16 st + 4 g4 + e.
  auto scores = [&](const char *k_lds, pf4 (&sc)[RS][NST]) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) sc[rs][st] = pf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const ph8 kf = *(const ph8 *)(k_lds + koff[ks] + 16 * st * ROWB);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
          sc[rs][st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qv[rs][ks], sc[rs][st], 0, 0, 0);
      }
    }
  };
  // Wait until at most n tiles' copies issued after the one needed are outstanding (n <= 2).
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    if (n >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm<4 * DT::SPW>());
    else if (n == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * DT::SPW>());
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  };

  // Mask (tiles that reach past the first row's limit) and online softmax statistics of tile
  // it: the running max m is raised only when a score exceeds it by more than 2^8 in weight
  // (then the accumulators are rescaled); otherwise probabilities up to 2^8 are taken against
  // the old reference, which o = acc / l and lse = m + log2 l absorb exactly.
  auto mask_max = [&](pf4 (&sc)[RS][NST], int it) __attribute__((always_inline)) {
    const int kv0 = it * KT;
    const bool need_mask = kv0 + KT - 1 > L - T + t0;  // workgroup-uniform
    float mrow[RS];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      float mx = kPNegInf;
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = kv0 + 16 * st + 4 * g4 + e;
            const float v = pos <= limit[rs] ? sc[rs][st][e] : kPNegInf;
            sc[rs][st][e] = v;
            mx = fmaxf(mx, v);
          }
      } else {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[rs][st][e]);
      }
      mrow[rs] = rows4_max(mx) * c;
    }
    // one rescale branch for both row sets (one fewer basic-block boundary in the tile)
    bool any_raise = false;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) any_raise |= mrow[rs] > m[rs] + 8.f;
    if (__any(any_raise)) {
#pragma unroll
      for (int rs = 0; rs < RS; ++rs) {
        const bool raise = mrow[rs] > m[rs] + 8.f;
        const float m_new = raise ? mrow[rs] : m[rs];
        const float alpha = __builtin_amdgcn_exp2f(m[rs] - m_new);
        m[rs] = m_new;
#pragma unroll
        for (int e = 0; e < 4; ++e) lacc[rs][e] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rs][dt][e] *= alpha;
      }
    }
  };
  // Probabilities of tile it (base 2, f16) and O^T += V^T P^T over its V rows, 32 tokens per
  // MFMA; the row sums by the all-ones MFMA.
  auto exp_pv = [&](const char *buf, pf4 (&sc)[RS][NST]) __attribute__((always_inline)) {
    ph8 pb[RS][NCH];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[rs][st][e] = __builtin_amdgcn_exp2f(fmaf(sc[rs][st][e], c, -m[rs]));
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[rs][ch][e] = (_Float16)sc[rs][2 * ch][e];
          pb[rs][ch][4 + e] = (_Float16)sc[rs][2 * ch + 1][e];
        }
    }
    const char *v_lds = buf + DT::BYTES;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        ph8 va;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const ps4 r4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_ps4)(const_cast<char *>(v_lds) + voff[dt] + (32 * ch + 16 * hh) * ROWB));
          const ph4 hv = __builtin_bit_cast(ph4, r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) va[4 * hh + e] = hv[e];
        }
#pragma unroll
        for (int rs = 0; rs < RS; ++rs)
          acc[rs][dt] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[rs][ch], acc[rs][dt], 0, 0, 0);
      }
#pragma unroll
      for (int rs = 0; rs < RS; ++rs)
        lacc[rs] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[rs][ch], lacc[rs], 0, 0, 0);
    }
  };

  // One tile per step: wait for its copies (those of up to NSTG - 2 later tiles may stay in
  // flight), publish it with a barrier (which also says that every wave is done with the
  // previous tile's buffer), issue the copies of tile it + NSTG - 1 into that buffer, compute.
  int pg_next = 0;
#pragma unroll
  for (int t = 0; t < NSTG - 1; ++t)
    if (t < ntiles)
      dma_tile<D, KT, NW>(a, kvh, w, t * KT, kv_last,
                          dma_page<D, KT, NW>(a, b, w, t * KT, kv_last), stg[t],
                          stg[t] + DT::BYTES);
  if (NSTG - 1 < ntiles) pg_next = dma_page<D, KT, NW>(a, b, w, (NSTG - 1) * KT, kv_last);
  for (int it = 0, bi = 0; it < ntiles; ++it) {
    const int bn = bi == 0 ? NSTG - 1 : bi - 1;  // buffer of tile it + NSTG - 1
    wait_tiles(min(NSTG - 2, ntiles - 1 - it));
    __builtin_amdgcn_s_barrier();
    if (it + NSTG - 1 < ntiles) {
      const int pg = pg_next;
      if (it + NSTG < ntiles) pg_next = dma_page<D, KT, NW>(a, b, w, (it + NSTG) * KT, kv_last);
      dma_tile<D, KT, NW>(a, kvh, w, (it + NSTG - 1) * KT, kv_last, pg, stg[bn],
                          stg[bn] + DT::BYTES);
    }
    pf4 s[RS][NST];
    // raised issue priority over the MFMA phases: when the other workgroup's wave on this SIMD
    // is in its softmax, this wave's MFMAs go first (measured 1 % faster; the softmax raised
    // instead: 0.5 % slower)
    __builtin_amdgcn_s_setprio(1);
    scores(stg[bi], s);
    __builtin_amdgcn_s_setprio(0);
    mask_max(s, it);
    __builtin_amdgcn_s_setprio(1);
    exp_pv(stg[bi], s);
    __builtin_amdgcn_s_setprio(0);
    bi = bi == NSTG - 1 ? 0 : bi + 1;
  }

  // ---- epilogue: normalize, write o and lse
#pragma unroll
  for (int rs = 0; rs < RS; ++rs) {
    const float lt = lacc[rs][0];
    if (!row_ok[rs]) continue;
    const int64_t orow = ((int64_t)b * T + trow[rs]) * a.Hq + hrow[rs];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    _Float16 *op = (_Float16 *)a.o + orow * D + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      ph4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = (_Float16)(acc[rs][dt][e] * inv);
      *(ph4 *)(op + 16 * dt) = ov;
    }
    if (g4 == 0 && a.lse) a.lse[orow] = lt > 0.f ? (m[rs] + __log2f(lt)) * kPLn2 : kPNegInf;
  }
}

// The copy-staged kernel's shape: 4 waves per workgroup (two workgroups per CU, so that the two
// waves on a SIMD belong to different workgroups and do not meet at the same barriers), two
// tile buffers of the register-staged kernel's tile size. Measured alternatives: 8 waves per
// workgroup with two or three buffers (as fast, or 1 % slower), 32-token tiles with three to
// five buffers (7-20 % slower), one workgroup of 4 waves per CU (70 % slower), and a pipeline
// inside each wave that issues the next tile's score MFMAs among this tile's exponentials
// (10 % slower: both waves of a SIMD then reach their LDS reads together).
constexpr int kDmaWaves = 4;
constexpr int kDmaStages = 2;

template <int D>
void launch_pd(const LaunchArgs &a, hipStream_t st) {
  constexpr int NW = prefill_waves<D>();
  const int tpw = 16 * NW * row_sets<D>() / a.G;  // query tokens per workgroup: its rows / G
  const int qtiles = (a.T + tpw - 1) / tpw;
  const unsigned grid = (unsigned)qtiles * a.Hkv * a.batch;
  if (a.page_shift >= 4 && !a.int8 && !a.fp8) {  // f16, pages of 16+ tokens: copies into LDS
    constexpr int DNW = kDmaWaves, DKT = kv_tile<D>();
    const int dtpw = 16 * DNW * row_sets<D>() / a.G;
    const int dq = (a.T + dtpw - 1) / dtpw;
    prefill_dma_kernel<D, DNW, DKT, kDmaStages>
        <<<(unsigned)dq * a.Hkv * a.batch, 64 * DNW, 0, st>>>(a, dtpw, dq);
    return;
  }
  if (a.page_shift >= 4) {  // pages of 16 tokens or more: wave-uniform page entries
    if (a.q4) prefill_kernel<D, 3, NW, true><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else if (a.fp8) prefill_kernel<D, 2, NW, true><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else if (a.int8) prefill_kernel<D, 1, NW, true><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else prefill_kernel<D, 0, NW, true><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
  } else {
    if (a.q4) prefill_kernel<D, 3, NW, false><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else if (a.fp8) prefill_kernel<D, 2, NW, false><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else if (a.int8) prefill_kernel<D, 1, NW, false><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
    else prefill_kernel<D, 0, NW, false><<<grid, 64 * NW, 0, st>>>(a, tpw, qtiles);
  }
}

}  // namespace

int launch_prefill(const LaunchArgs &a, void *stream) {
  if (a.batch == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  if (a.D == 128) launch_pd<128>(a, st);
  else launch_pd<256>(a, st);
  return (int)hipGetLastError();
}

}  // namespace skvd
