/*
 * oracle.c - plain fp64 CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The HIP library never calls it, and the two share no code:
 * no headers, no helpers, no tables, no constants.
 *
 * What it computes
 * ----------------
 * The split-KV decode of the pages computes exactly (up to rounding order) plain softmax
 * attention over the cached positions of each sequence: cutting the KV length into 64-token
 * partial blocks and merging the per-block partials with a log-sum-exp reduction is an
 * algebraic identity (1bit-MONSTER/engine issue #115, "HRX: flash-attention decode-split
 * template resolution fails", comments "Root-caused" and "Closing the remaining half of this
 * issue": the producer writes one partial per 64-token block and reduce_fused merges them).
 * So this oracle is that plain definition, written out in fp64, step by step:
 *
 *   O1 gather  For sequence b and logical position j, the page is table[b][j / P] and the
 *              slot j % P; the K row of KV head g is read at
 *              page*page_stride + slot*tok_stride + g*head_stride (elements). V is read with
 *              the same page shape and strides as K, and only pages named by the table are
 *              read (AMD-Ecosystem/flashinfer PR #397, "Stop declaring the paged KV cache
 *              mutated on read-only attention ops", section "What changed": K and V share page
 *              shape and strides; page counts may differ; only indexed pages are read).
 *              An f16 element widens to f64 exactly. An int8 element is value = int8 * scale
 *              with one f16 scale per 32 contiguous head_dim elements; the product is exact
 *              in f64. An fp8 element is an OCP E4M3 byte (the AMD-Ecosystem/flashinfer PR
 *              #397 commit messages name fp8 caches read with per-tensor k_scale and v_scale
 *              values) times the tensor's f32 scale: value = e4m3(byte) * k_scale for K and
 *              * v_scale for V, exact in f64.
 *              A q4_0 element (the 4-bit cache type that 1bit-MONSTER/engine issue #115,
 *              comment "Closing the remaining half of this issue", names beside q8_0 among the
 *              KV cache types not yet exercised; the pages do not define it, so it is read here
 *              as the published ggml q4_0 block) is a 4-bit code c in 0..15 with one f16 scale
 *              per 32 contiguous head_dim elements: value = (c - 8) * scale, exact in f64. The
 *              codes of a row are D/2 bytes: group k (elements 32k .. 32k+31) in bytes
 *              16k .. 16k+15, byte i of a group holding element i of the group in its low nibble
 *              and element i + 16 in its high nibble. Scales are laid out as int8's.
 *   O2 heads   Query head h reads KV head floor(h / G), G = Hq / Hkv (consecutive grouping;
 *              the pages give only the head counts).
 *   O3 length  Query token t of a sequence with T query tokens and kv_len L sees positions
 *              j < L - T + t + 1 (the T query tokens are the last T cached positions: the
 *              multi-token decode that the routing threshold of llama-cpp-turboquant PR #176,
 *              section "Changes", keeps on the decode path for MTP spec-decode). T = 1 sees L.
 *   O4 logits  s_j = sm_scale * sum_d q[d] * K[j][d], all in fp64.
 *   O5 result  m = max_j s_j, w_j = exp(s_j - m), S = sum_j w_j,
 *              o[d] = sum_j w_j V[j][d] / S, lse = m + ln S (natural log, scale included).
 *              A row that sees no position gets o = 0 and lse = -inf.
 *   O6         (self-check only) the same result in split form: blocks of a given number of
 *              tokens, each with its own (m_i, S_i, o_i), merged with M = max m_i,
 *              S = sum S_i e^(m_i - M), o = sum e^(m_i - M) o_i / S, lse = M + ln S.
 *
 * Layouts: q is [B*T, Hq, D] f16 (row b*T + t; token and head strides in elements, D dense);
 * K and V pools are [pages, P, Hkv, D] with the given element strides; int8 scales are
 * [pages, P, Hkv, D/32] f16 with their own strides; table is [B, table_stride] int32;
 * kv_len is [B] int32. Outputs are fp64 [nrows, D] and [nrows].
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* A mutant build plants one deliberate mistake so that the tests can show a pin catches
 * it. The default build (ORACLE_MUTANT undefined or 0) is the oracle. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

typedef struct {
  int32_t batch;        /* B */
  int32_t q_per_seq;    /* T */
  int32_t num_qo_heads; /* Hq */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* D */
  int32_t page_size;    /* P */
  int32_t kv_int8;      /* 0: f16 K/V; 1: int8 K/V with f16 scales per 32 elements;
                           2: fp8 E4M3 K/V with one f32 scale per tensor (k_fp8_scale,
                           v_fp8_scale); 3: q4_0 codes (D/2 bytes per row) with f16 scales
                           per 32 elements */
  int32_t pad0;
  double sm_scale;      /* the f32 scale the caller passes, widened */
  const uint16_t *q;    /* f16 bits */
  int64_t q_tok_stride, q_head_stride;
  const void *k, *v;    /* f16 bits or int8 */
  const uint16_t *k_scale, *v_scale;
  int64_t page_stride, tok_stride, head_stride;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  const int32_t *kv_len;
  double k_fp8_scale, v_fp8_scale; /* fp8 cache: the per-tensor f32 scales, widened */
} oracle_problem;

/* IEEE-754 binary16 -> binary64, exact. */
double oracle_half_to_double(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25); /* (1024 + m) * 2^(e - 15 - 10) */
  return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3 (exponent bias 7, 3 mantissa bits, no infinities):
 * byte s.eeee.mmm is (-1)^s * 2^(e - 7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * (m/8) for
 * e = 0, and NaN for eeee.mmm = 1111.111. Exact in f64. */
double oracle_e4m3_to_double(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
#if ORACLE_MUTANT == 17
  if (e == 0)
    v = ldexp((double)m, -10); /* planted: subnormal exponent off by one */
#else
  if (e == 0)
    v = ldexp((double)m, -9); /* 2^-6 * m / 8 */
#endif
  else
    v = ldexp((double)(8 + m), e - 10); /* 2^(e - 7) * (8 + m) / 8 */
  return sign ? -v : v;
}

/* O1: element offset of position j's row for KV head g, and of its scale row. */
static int64_t row_offset(const oracle_problem *p, int b, int64_t j, int g, int64_t *scale_off) {
  int64_t page_idx = j / p->page_size;
  int64_t slot = j % p->page_size;
#if ORACLE_MUTANT == 4
  slot = (j + 1) % p->page_size; /* planted: wrong slot */
#endif
  int64_t page = p->table[(int64_t)b * p->table_stride + page_idx];
  if (scale_off)
    *scale_off = page * p->s_page_stride + slot * p->s_tok_stride + (int64_t)g * p->s_head_stride;
  return page * p->page_stride + slot * p->tok_stride + (int64_t)g * p->head_stride;
}

/* O1: dequantized element d of a gathered row, in fp64 (tscale: the fp8 tensor scale). */
static double kv_elem(const oracle_problem *p, const void *base, const uint16_t *scales,
                      double tscale, int64_t off, int64_t soff, int d) {
  if (!p->kv_int8) return oracle_half_to_double(((const uint16_t *)base)[off + d]);
  if (p->kv_int8 == 2) {
#if ORACLE_MUTANT == 18
    tscale = 1.0; /* planted: tensor scale dropped */
#endif
    return oracle_e4m3_to_double(((const uint8_t *)base)[off + d]) * tscale;
  }
  if (p->kv_int8 == 3) {
    int grp = d / 32, i = d % 32;
    uint8_t byte = ((const uint8_t *)base)[off + 16 * grp + (i % 16)];
    int c = i < 16 ? (byte & 15) : (byte >> 4);
#if ORACLE_MUTANT == 20
    c = i < 16 ? (byte >> 4) : (byte & 15); /* planted: nibble order swapped */
#endif
#if ORACLE_MUTANT == 21
    return (double)(c - 7) * oracle_half_to_double(scales[soff + grp]); /* planted: offset 7 */
#endif
    return (double)(c - 8) * oracle_half_to_double(scales[soff + grp]);
  }
  int group = d / 32;
#if ORACLE_MUTANT == 5
  group = d / 16; /* planted: wrong scale group */
  if (group >= p->head_dim / 32) group = p->head_dim / 32 - 1;
#endif
  double s = oracle_half_to_double(scales[soff + group]);
  return (double)((const int8_t *)base)[off + d] * s;
}

/* O3: number of positions row (b, t) sees. */
static int64_t visible_len(const oracle_problem *p, int b, int t) {
  int64_t L = p->kv_len[b];
  int64_t n = L - p->q_per_seq + t + 1;
#if ORACLE_MUTANT == 3
  n = L - p->q_per_seq + t; /* planted: causal off by one */
#endif
  if (n > L) n = L;
  return n < 0 ? 0 : n;
}

/* O2 */
static int kv_head_of(const oracle_problem *p, int h) {
#if ORACLE_MUTANT == 1
  return h % p->num_kv_heads; /* planted: interleaved head map */
#else
  return h / (p->num_qo_heads / p->num_kv_heads);
#endif
}

/* O4 for one (row, position). */
static double logit(const oracle_problem *p, const uint16_t *qrow, int b, int64_t j, int g) {
  int64_t soff = 0;
  int64_t off = row_offset(p, b, j, g, &soff);
#if ORACLE_MUTANT == 8
  const void *kb = p->v; const uint16_t *ks = p->v_scale; /* planted: V used as K */
  double ts = p->v_fp8_scale;
#else
  const void *kb = p->k; const uint16_t *ks = p->k_scale;
  double ts = p->k_fp8_scale;
#endif
  double dot = 0.0;
  for (int d = 0; d < p->head_dim; ++d)
    dot += oracle_half_to_double(qrow[d]) * kv_elem(p, kb, ks, ts, off, soff, d);
#if ORACLE_MUTANT == 2
  return dot; /* planted: scale dropped */
#else
  return p->sm_scale * dot;
#endif
}

static void row_coords(const oracle_problem *p, int64_t r, int *b, int *t, int *h) {
  int64_t Hq = p->num_qo_heads, T = p->q_per_seq;
  *h = (int)(r % Hq);
  int64_t bt = r / Hq;
  *t = (int)(bt % T);
  *b = (int)(bt / T);
}

static const uint16_t *q_row(const oracle_problem *p, int b, int t, int h) {
  int tt = t;
#if ORACLE_MUTANT == 10
  tt = 0; /* planted: every query token reads token 0's q */
#endif
  return p->q + ((int64_t)b * p->q_per_seq + tt) * p->q_tok_stride + (int64_t)h * p->q_head_stride;
}

/* O1-O5 for one row; s is scratch of at least n doubles. */
static void decode_row(const oracle_problem *p, int64_t r, double *o, double *lse, double *s) {
  int b, t, h;
  row_coords(p, r, &b, &t, &h);
  int D = p->head_dim, g = kv_head_of(p, h);
  int64_t n = visible_len(p, b, t);
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (n <= 0) { *lse = -INFINITY; return; }
  const uint16_t *qrow = q_row(p, b, t, h);
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    s[j] = logit(p, qrow, b, j, g);
    if (s[j] > m) m = s[j];
  }
  double S = 0.0;
  for (int64_t j = 0; j < n; ++j) {
#if ORACLE_MUTANT == 9
    double w = exp(m - s[j]); /* planted: sign flipped */
#else
    double w = exp(s[j] - m);
#endif
    S += w;
    int64_t soff = 0;
    int64_t off = row_offset(p, b, j, g, &soff);
    for (int d = 0; d < D; ++d) o[d] += w * kv_elem(p, p->v, p->v_scale, p->v_fp8_scale, off, soff, d);
  }
#if ORACLE_MUTANT != 7
  for (int d = 0; d < D; ++d) o[d] /= S;
#endif
#if ORACLE_MUTANT == 6
  *lse = log(S); /* planted: max dropped from lse */
#else
  *lse = m + log(S);
#endif
}

static int64_t max_visible(const oracle_problem *p) {
  int64_t mx = 1;
  for (int b = 0; b < p->batch; ++b)
    if (p->kv_len[b] > mx) mx = p->kv_len[b];
  return mx;
}

/* Decode the given rows (r = (b*T + t)*Hq + h), or all B*T*Hq rows when rows is NULL.
 * o is [nrows, D] and lse [nrows], fp64. nthreads <= 0 uses the OpenMP default. */
int oracle_decode(const oracle_problem *p, const int64_t *rows, int64_t nrows, double *o,
                  double *lse, int nthreads) {
  int64_t total = (int64_t)p->batch * p->q_per_seq * p->num_qo_heads;
  if (!rows) nrows = total;
  int64_t smax = max_visible(p);
  int D = p->head_dim;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)smax);
    if (!s) bad = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t i = 0; i < nrows; ++i) {
      int64_t r = rows ? rows[i] : i;
      if (!s || r < 0 || r >= total) { bad = 1; continue; }
      decode_row(p, r, o + i * D, lse + i, s);
    }
    free(s);
  }
  return bad ? -1 : 0;
}

/* O6 (self-check): the same rows in split form over blocks of `block` tokens. */
int oracle_decode_blocked(const oracle_problem *p, const int64_t *rows, int64_t nrows,
                          int64_t block, double *o, double *lse) {
  int64_t total = (int64_t)p->batch * p->q_per_seq * p->num_qo_heads;
  if (!rows) nrows = total;
  if (block <= 0) return -1;
  int D = p->head_dim;
  double *oi = (double *)malloc(sizeof(double) * (size_t)D);
  if (!oi) return -1;
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (r < 0 || r >= total) { free(oi); return -1; }
    int b, t, h;
    row_coords(p, r, &b, &t, &h);
    int g = kv_head_of(p, h);
    int64_t n = visible_len(p, b, t);
    const uint16_t *qrow = q_row(p, b, t, h);
    double *orow = o + i * D;
    double M = -INFINITY, S = 0.0;
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    for (int64_t j0 = 0; j0 < n; j0 += block) {
      int64_t j1 = j0 + block < n ? j0 + block : n;
      double mi = -INFINITY, Si = 0.0;
      for (int64_t j = j0; j < j1; ++j) {
        double s = logit(p, qrow, b, j, g);
        if (s > mi) mi = s;
      }
      for (int d = 0; d < D; ++d) oi[d] = 0.0;
      for (int64_t j = j0; j < j1; ++j) {
        double w = exp(logit(p, qrow, b, j, g) - mi);
        Si += w;
        int64_t soff = 0;
        int64_t off = row_offset(p, b, j, g, &soff);
        for (int d = 0; d < D; ++d) oi[d] += w * kv_elem(p, p->v, p->v_scale, p->v_fp8_scale, off, soff, d);
      }
      /* merge block i into the running state */
      double Mn = mi > M ? mi : M;
      double a = (M == -INFINITY) ? 0.0 : exp(M - Mn), c = exp(mi - Mn);
      S = S * a + Si * c;
      for (int d = 0; d < D; ++d) orow[d] = orow[d] * a + oi[d] * c;
      M = Mn;
    }
    if (n <= 0) { lse[i] = -INFINITY; continue; }
    for (int d = 0; d < D; ++d) orow[d] /= S;
    lse[i] = M + log(S);
  }
  free(oi);
  return 0;
}

/* O1 alone: copy the raw elements (and, for int8 and q4_0, the raw f16 scale bits; fp8 has
 * none per row) of every visible position j < kv_len[b] into dense [B, max_len, Hkv, RB]
 * (and [B, max_len, Hkv, D/32]) arrays, RB the bytes of a row over the element size (D, or
 * D/2 bytes for q4_0). Positions at or beyond kv_len are left untouched. */
int oracle_gather(const oracle_problem *p, int64_t max_len, void *dense_k, void *dense_v,
                  uint16_t *dense_ks, uint16_t *dense_vs) {
  int Hkv = p->num_kv_heads, es = p->kv_int8 ? 1 : 2, ng = p->head_dim / 32;
  int D = p->kv_int8 == 3 ? p->head_dim / 2 : p->head_dim; /* row length in pool elements */
  for (int b = 0; b < p->batch; ++b) {
    int64_t L = p->kv_len[b];
    if (L > max_len) return -1;
    for (int64_t j = 0; j < L; ++j)
      for (int g = 0; g < Hkv; ++g) {
        int64_t soff = 0;
        int64_t off = row_offset(p, b, j, g, &soff);
        int64_t dst = (((int64_t)b * max_len + j) * Hkv + g);
        memcpy((char *)dense_k + dst * D * es, (const char *)p->k + off * es, (size_t)D * es);
        memcpy((char *)dense_v + dst * D * es, (const char *)p->v + off * es, (size_t)D * es);
        if (p->kv_int8 == 1 || p->kv_int8 == 3) {
          memcpy(dense_ks + dst * ng, p->k_scale + soff, sizeof(uint16_t) * ng);
          memcpy(dense_vs + dst * ng, p->v_scale + soff, sizeof(uint16_t) * ng);
        }
      }
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ============================================================================ append
 * Writing new tokens into the paged cache: the step before a decode, and the one operation
 * that writes the cache (AMD-Ecosystem/flashinfer PR #397, section "What changed": append
 * genuinely writes the cache and keeps declaring it written, unlike the read-only decode).
 * The pages give no further definition, so this is the plainest reading, stated in the
 * library's own terms:
 *
 *   W1 place   New token i belongs to sequence b = batch_idx[i] at logical position
 *              j = positions[i]. Its K row of KV head g goes to slot j % P of page
 *              table[b][j / P], at page*page_stride + slot*tok_stride + g*head_stride
 *              (elements) - the address O1 reads - and its V row to the same place in V.
 *              A token whose b is outside [0, batch) or j outside [0, max_len) is skipped;
 *              a page id outside a pool skips that pool's write. Nothing else is written.
 *   W2 f16     An f16 cache receives the f16 elements verbatim.
 *   W3 int8    An int8 cache (value = int8 * scale, one f16 scale per 32 contiguous head_dim
 *              elements: the q8_0-style KV type that the pages name, 1bit-MONSTER/engine issue
 *              #115 "Fixed" and llama-cpp-turboquant PR #176 "Results") quantizes each group
 *              of 32 on write, symmetric, with the largest magnitude mapped to 127:
 *                a = max |x| over the group (exact),
 *                s = f16(a / 127): the quotient in f32, rounded once to f16 (nearest even),
 *                c = clip(rint(x / s), -127, 127), x / s in f32, rint to nearest even;
 *                s = 0 (an all-zero group, or a below f16's range) gives c = 0.
 *              The pages fix no precision for these decisions; f32 is the kernel's.
 *              Non-finite inputs (the pages do not cover them; the plainest reading of the
 *              formulas): a NaN element is not larger than any magnitude, so it leaves the
 *              maximum alone, and its quotient is NaN, stored as code 0; an infinite element
 *              makes a infinite, s = f16(inf) = inf, and every code 0 (finite / inf = 0,
 *              inf / inf = NaN).
 *   W4 fp8     An fp8 cache (OCP E4M3 bytes times a per-tensor f32 scale s: k_scale for K,
 *              v_scale for V) stores for each element the E4M3 value nearest to
 *              clip(x / s, -448, 448), x / s the f32 quotient, ties to the even mantissa;
 *              a NaN quotient (0 / 0, or a NaN element) stores 0; an infinite one saturates
 *              at +-448. 448 is E4M3's largest finite value, so the clip saturates rather
 *              than overflowing. The pages name the format and its
 *              per-tensor scales only; the rule is the plainest one with the kernel's f32.
 *   W5 q4_0    A q4_0 cache (O1's 4-bit codes, value = (c - 8) * d, one f16 d per group of
 *              32) quantizes each group on write by the published ggml q4_0 rule, all in f32:
 *                m = the group's element of largest magnitude (the first one in element
 *                    order on a tie; m = +0 when every magnitude is 0),
 *                d = m / -8 (so that m itself gets code 0 and value -8d = m),
 *                r = 1 / d (correctly rounded; r = 0 when d = 0),
 *                c = min(15, trunc(x * r + 8.5)), the product and the sum each rounded to
 *                    f32 (x * r lies in [-8, 8] up to rounding, so the sum is positive),
 *              and the stored scale is f16(d) (nearest even): the codes come from the f32 d,
 *              not from the rounded scale. Non-finite inputs: a NaN element does not take
 *              part in the maximum and stores code 8 (value 0); an infinite m makes
 *              d = -+inf, r = -+0 and every code 8 (an infinite element's x * r is NaN, a
 *              finite one's 0), with the scale f16(d) = -+inf.
 * ============================================================================ */

typedef struct {
  int32_t num_tokens;   /* N */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* D */
  int32_t page_size;    /* P */
  int32_t kv_int8;      /* 0: f16 cache; 1: int8 cache with f16 scales per 32 elements;
                           2: fp8 E4M3 cache with per-tensor f32 scales; 3: q4_0 codes with
                           f16 scales per 32 elements */
  int32_t batch;        /* rows of the page table */
  int32_t max_len;      /* positions are < max_len */
  int32_t pad0;
  const uint16_t *k_new, *v_new; /* f16 bits [N, Hkv, D] */
  int64_t new_tok_stride, new_head_stride;
  const int32_t *batch_idx, *positions;
  void *k, *v;                   /* written: f16 bits or int8 */
  uint16_t *k_scale, *v_scale;   /* written: f16 bits (int8 cache only) */
  int64_t page_stride, tok_stride, head_stride;
  int64_t num_k_pages, num_v_pages;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  float k_fp8_scale, v_fp8_scale; /* fp8 cache: the per-tensor scales */
} oracle_append_problem;

/* IEEE-754 binary32 -> binary16, rounded to nearest, ties to even (the default IEEE rounding).
 * Written from the format's definition: the result is the f16 value nearest to x, so scale x
 * to the integer significand grid of its binade and round that once. */
uint16_t oracle_float_to_half(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs((double)x);
  if (isnan(x)) return (uint16_t)(sign | 0x7e00);
  if (isinf(x)) return (uint16_t)(sign | 0x7c00);
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1): the binade is [2^(e2-1), 2^e2) */
  int e = e2 - 1;         /* unbiased exponent of a */
  if (e < -14) e = -14;   /* subnormal range: the grid step stays 2^-24 */
  double q = rint(ldexp(a, 10 - e)); /* significand with 10 fraction bits, nearest even */
  if (q >= 2048.0) { q /= 2.0; e += 1; } /* rounded up into the next binade (exact) */
  if (e > 15) return (uint16_t)(sign | 0x7c00); /* overflow: infinity */
  if (q < 1024.0) return (uint16_t)(sign | (uint16_t)q); /* subnormal (exponent field 0) */
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* W3 for one group of n (= 32) f16 elements. */
void oracle_quantize_group(const uint16_t *x, int n, int8_t *codes, uint16_t *scale_bits) {
  float a = 0.0f;
  for (int d = 0; d < n; ++d) {
    float v = fabsf((float)oracle_half_to_double(x[d]));
    if (v > a) a = v;
  }
#if ORACLE_MUTANT == 11
  float sq = a / 128.0f; /* planted: wrong divisor */
#else
  float sq = a / 127.0f;
#endif
  uint16_t sb = oracle_float_to_half(sq);
  float s = (float)oracle_half_to_double(sb);
  *scale_bits = sb;
  for (int d = 0; d < n; ++d) {
    float v = (float)oracle_half_to_double(x[d]);
    float c = 0.0f;
    if (s > 0.0f) {
#if ORACLE_MUTANT == 12
      c = truncf(v / s); /* planted: truncation instead of rounding */
#else
      c = rintf(v / s);
#endif
      if (c > 127.0f) c = 127.0f;
      if (c < -127.0f) c = -127.0f;
      if (isnan(c)) c = 0.0f; /* NaN element, or an infinite one over an infinite scale */
    }
    codes[d] = (int8_t)c;
  }
}

/* W4 for one f32 value: the byte of the nearest E4M3 value to clip(q, -448, 448), ties to
 * the even mantissa, found by comparing against every finite non-negative E4M3 magnitude
 * (bytes 0x00 .. 0x7E, in increasing order of value). */
uint8_t oracle_e4m3_from_float(float q) {
  if (isnan(q)) return 0;
  uint8_t sign = signbit(q) ? 0x80 : 0;
  double a = fabs((double)q);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(oracle_e4m3_to_double((uint8_t)c) - a);
#if ORACLE_MUTANT == 19
    if (d < best_d) { /* planted: ties go to the smaller magnitude */
#else
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
#endif
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* W5 for one group of 32 f16 elements: 16 code bytes (element i in the low nibble of byte i,
 * element i + 16 in its high nibble) and the f16 scale. */
void oracle_quantize_q4_group(const uint16_t *x, uint8_t *codes, uint16_t *scale_bits) {
  float m = 0.0f, amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float v = (float)oracle_half_to_double(x[i]);
#if ORACLE_MUTANT == 22
    if (amax <= fabsf(v)) { /* planted: the last element of largest magnitude wins a tie */
#else
    if (amax < fabsf(v)) { /* false for NaN: a NaN never becomes the maximum */
#endif
      amax = fabsf(v);
      m = v;
    }
  }
  float d = m / -8.0f;
#if ORACLE_MUTANT == 23
  d = amax / 8.0f; /* planted: the magnitude instead of the signed extreme */
#endif
  float r = d != 0.0f ? 1.0f / d : 0.0f;
  uint8_t c[32];
  for (int i = 0; i < 32; ++i) {
    float v = (float)oracle_half_to_double(x[i]);
    float xr = v * r;
    float t = xr + 8.5f;
#if ORACLE_MUTANT == 24
    t = rintf(xr) + 8.0f; /* planted: nearest-even rounding instead of the +8.5 truncation */
#endif
    int q = isnan(t) ? 8 : (int)t;
    c[i] = (uint8_t)(q > 15 ? 15 : q);
  }
  for (int i = 0; i < 16; ++i) codes[i] = (uint8_t)(c[i] | (c[i + 16] << 4));
  *scale_bits = oracle_float_to_half(d);
}

/* W1-W5 for one row of one pool. */
static void append_row(const oracle_append_problem *p, const uint16_t *src, void *pool,
                       uint16_t *scales, float tscale, int64_t page, int64_t slot, int g) {
  int D = p->head_dim;
  int64_t off = page * p->page_stride + slot * p->tok_stride + (int64_t)g * p->head_stride;
  if (!p->kv_int8) {
    memcpy((uint16_t *)pool + off, src, sizeof(uint16_t) * (size_t)D);
    return;
  }
  if (p->kv_int8 == 2) {
    for (int d = 0; d < D; ++d) {
      float x = (float)oracle_half_to_double(src[d]);
      ((uint8_t *)pool)[off + d] = oracle_e4m3_from_float(x / tscale);
    }
    return;
  }
  int64_t soff = page * p->s_page_stride + slot * p->s_tok_stride + (int64_t)g * p->s_head_stride;
  if (p->kv_int8 == 3) {
    for (int grp = 0; grp < D / 32; ++grp)
      oracle_quantize_q4_group(src + grp * 32, (uint8_t *)pool + off + grp * 16,
                               scales + soff + grp);
    return;
  }
  for (int grp = 0; grp < D / 32; ++grp) {
    int sg = grp;
#if ORACLE_MUTANT == 13
    sg = (grp + 1) % (D / 32); /* planted: scale stored in the wrong group's slot */
#endif
    oracle_quantize_group(src + grp * 32, 32, (int8_t *)pool + off + grp * 32, scales + soff + sg);
  }
}

/* Append every new token (W1-W3), in token order. Returns the number of tokens skipped. */
int64_t oracle_append(const oracle_append_problem *p) {
  int64_t skipped = 0;
  int P = p->page_size;
  for (int64_t i = 0; i < p->num_tokens; ++i) {
    int b = p->batch_idx[i];
    int64_t j = p->positions[i];
    if (b < 0 || b >= p->batch || j < 0 || j >= p->max_len) { ++skipped; continue; }
    int64_t page = p->table[(int64_t)b * p->table_stride + j / P];
    int64_t slot = j % P;
    for (int g = 0; g < p->num_kv_heads; ++g) {
      int gg = g;
#if ORACLE_MUTANT == 14
      gg = (g + 1) % p->num_kv_heads; /* planted: row written under the next KV head */
#endif
      const uint16_t *kr = p->k_new + i * p->new_tok_stride + (int64_t)g * p->new_head_stride;
      const uint16_t *vr = p->v_new + i * p->new_tok_stride + (int64_t)g * p->new_head_stride;
      if (page >= 0 && page < p->num_k_pages)
        append_row(p, kr, p->k, p->k_scale, p->k_fp8_scale, page, slot, gg);
      if (page >= 0 && page < p->num_v_pages)
        append_row(p, vr, p->v, p->v_scale, p->v_fp8_scale, page, slot, gg);
    }
  }
  return skipped;
}

/* ============================================================================ merge states
 * Merging attention states: the shared-prefix (cascade) use of the log-sum-exp reduction that
 * merges the split-KV partials (1bit-MONSTER/engine issue #115, comments "Root-caused" and
 * "Closing the remaining half of this issue": partials merged by reduce_fused; AMD-Ecosystem/
 * flashinfer PR #397 names a cascade test under "Test plan"). A state of one row over a set of
 * keys is (o, lse) with o the softmax-weighted mean of V over the set and lse = ln sum exp of
 * the set's scaled logits. States over disjoint key sets merge to the state over their union:
 *   M = max_s lse_s, w_s = exp(lse_s - M), W = sum_s w_s,
 *   o = sum_s w_s o_s / W, lse = M + ln W;
 * a state with lse = -inf (an empty key set) contributes nothing; if every state is empty,
 * o = 0 and lse = -inf. fp64 throughout.
 * ============================================================================ */

/* o_states: fp64 [S][rows][D]; lse_states: fp64 [S][rows]; outputs fp64 o [rows][D], lse [rows]. */
int oracle_merge_states(int32_t num_states, int64_t rows, int32_t head_dim,
                        const double *o_states, const double *lse_states, double *o,
                        double *lse) {
  if (num_states < 1 || rows < 0 || head_dim < 1) return -1;
  int D = head_dim;
  for (int64_t r = 0; r < rows; ++r) {
    double M = -INFINITY;
    for (int s = 0; s < num_states; ++s) {
      double x = lse_states[(int64_t)s * rows + r];
      if (x > M) M = x;
    }
    double *orow = o + r * D;
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
    double W = 0.0;
    for (int s = 0; s < num_states; ++s) {
      double x = lse_states[(int64_t)s * rows + r];
      if (x == -INFINITY) continue;
#if ORACLE_MUTANT == 15
      double w = exp(M - x); /* planted: weight sign flipped */
#else
      double w = exp(x - M);
#endif
      W += w;
      const double *os = o_states + ((int64_t)s * rows + r) * D;
      for (int d = 0; d < D; ++d) orow[d] += w * os[d];
    }
    for (int d = 0; d < D; ++d) orow[d] /= W;
#if ORACLE_MUTANT == 16
    lse[r] = log(W); /* planted: max dropped */
#else
    lse[r] = M + log(W);
#endif
  }
  return 0;
}
