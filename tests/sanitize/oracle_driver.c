/* Host-only driver that runs every oracle entry point on small problems held in exactly sized
 * heap buffers, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py: an out-of-range read or write, or undefined arithmetic, in the
 * oracle aborts the run. Edge cases: an empty sequence, causal multi-token rows, int8 pools,
 * appends with skipped tokens, merges with empty states. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t batch, q_per_seq, num_qo_heads, num_kv_heads, head_dim, page_size, kv_int8, pad0;
  double sm_scale;
  const uint16_t *q;
  int64_t q_tok_stride, q_head_stride;
  const void *k, *v;
  const uint16_t *k_scale, *v_scale;
  int64_t page_stride, tok_stride, head_stride;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  const int32_t *kv_len;
  double k_fp8_scale, v_fp8_scale;
} oracle_problem;

typedef struct {
  int32_t num_tokens, num_kv_heads, head_dim, page_size, kv_int8, batch, max_len, pad0;
  const uint16_t *k_new, *v_new;
  int64_t new_tok_stride, new_head_stride;
  const int32_t *batch_idx, *positions;
  void *k, *v;
  uint16_t *k_scale, *v_scale;
  int64_t page_stride, tok_stride, head_stride, num_k_pages, num_v_pages;
  int64_t s_page_stride, s_tok_stride, s_head_stride;
  const int32_t *table;
  int64_t table_stride;
  float k_fp8_scale, v_fp8_scale;
} oracle_append_problem;

int oracle_decode(const oracle_problem *, const int64_t *, int64_t, double *, double *, int);
int oracle_decode_blocked(const oracle_problem *, const int64_t *, int64_t, int64_t, double *,
                          double *);
int oracle_gather(const oracle_problem *, int64_t, void *, void *, uint16_t *, uint16_t *);
int64_t oracle_append(const oracle_append_problem *);
uint16_t oracle_float_to_half(float);
int oracle_merge_states(int32_t, int64_t, int32_t, const double *, const double *, double *,
                        double *);

static uint32_t rng_state = 12345u;
static float frand(void) { /* xorshift32 in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)(rng_state >> 8) / 8388608.0f - 1.0f;
}

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) exit(3);
  return p;
}

static int run(int int8, int T) {
  const int B = 3, Hq = 4, Hkv = 2, D = 64, P = 4;
  const int32_t lens[3] = {0, 5, 37};
  int32_t npages[3], max_pages = 0, total_pages = 0;
  for (int b = 0; b < B; ++b) {
    npages[b] = (lens[b] + P - 1) / P;
    if (npages[b] > max_pages) max_pages = npages[b];
    total_pages += npages[b];
  }
  int32_t *table = xmalloc(sizeof(int32_t) * B * max_pages);
  for (int i = 0; i < B * max_pages; ++i) table[i] = -1;
  for (int b = 0, pg = total_pages - 1; b < B; ++b)
    for (int i = 0; i < npages[b]; ++i) table[b * max_pages + i] = pg--; /* reversed pages */
  const size_t elems = (size_t)total_pages * P * Hkv * D, es = int8 ? 1 : 2;
  void *k = xmalloc(elems * es), *v = xmalloc(elems * es);
  uint16_t *ks = NULL, *vs = NULL;
  const size_t sel = (size_t)total_pages * P * Hkv * (D / 32);
  if (int8 == 2) { /* fp8 E4M3 bytes, no NaN byte; per-tensor scales in the problem */
    for (size_t i = 0; i < elems; ++i) {
      uint8_t a = (uint8_t)((frand() + 1.0f) * 127.5f), c = (uint8_t)((frand() + 1.0f) * 127.5f);
      ((uint8_t *)k)[i] = (a & 0x7F) == 0x7F ? a ^ 1 : a;
      ((uint8_t *)v)[i] = (c & 0x7F) == 0x7F ? c ^ 1 : c;
    }
  } else if (int8) {
    ks = xmalloc(sizeof(uint16_t) * sel);
    vs = xmalloc(sizeof(uint16_t) * sel);
    for (size_t i = 0; i < elems; ++i) {
      ((int8_t *)k)[i] = (int8_t)(frand() * 127);
      ((int8_t *)v)[i] = (int8_t)(frand() * 127);
    }
    for (size_t i = 0; i < sel; ++i) {
      ks[i] = oracle_float_to_half(0.01f + 0.005f * frand());
      vs[i] = oracle_float_to_half(0.01f + 0.005f * frand());
    }
  } else {
    for (size_t i = 0; i < elems; ++i) {
      ((uint16_t *)k)[i] = oracle_float_to_half(frand());
      ((uint16_t *)v)[i] = oracle_float_to_half(frand());
    }
  }
  const size_t qe = (size_t)B * T * Hq * D;
  uint16_t *q = xmalloc(sizeof(uint16_t) * qe);
  for (size_t i = 0; i < qe; ++i) q[i] = oracle_float_to_half(frand());
  int32_t *kv_len = xmalloc(sizeof(int32_t) * B);
  memcpy(kv_len, lens, sizeof lens);
  oracle_problem p = {B, T, Hq, Hkv, D, P, int8, 0, 0.125, q, (int64_t)Hq * D, D, k, v, ks, vs,
                      (int64_t)P * Hkv * D, (int64_t)Hkv * D, D,
                      (int64_t)P * Hkv * (D / 32), (int64_t)Hkv * (D / 32), D / 32,
                      table, max_pages, kv_len, 0.05, 0.07};
  const int64_t rows = (int64_t)B * T * Hq;
  double *o = xmalloc(sizeof(double) * rows * D), *lse = xmalloc(sizeof(double) * rows);
  double *o2 = xmalloc(sizeof(double) * rows * D), *lse2 = xmalloc(sizeof(double) * rows);
  int bad = oracle_decode(&p, NULL, rows, o, lse, 2) != 0;
  bad |= oracle_decode_blocked(&p, NULL, rows, 7, o2, lse2) != 0;
  for (int64_t i = 0; i < rows * D; ++i) bad |= fabs(o[i] - o2[i]) > 1e-12;
  /* gather */
  const int max_len = 37;
  void *dk = xmalloc((size_t)B * max_len * Hkv * D * es), *dv = xmalloc((size_t)B * max_len * Hkv * D * es);
  uint16_t *dks = int8 == 1 ? xmalloc(sizeof(uint16_t) * B * max_len * Hkv * (D / 32)) : NULL;
  uint16_t *dvs = int8 == 1 ? xmalloc(sizeof(uint16_t) * B * max_len * Hkv * (D / 32)) : NULL;
  bad |= oracle_gather(&p, max_len, dk, dv, dks, dvs) != 0;
  /* append: tokens of sequences 1 and 2, plus skipped ones (bad sequence, bad position) */
  const int N = 8;
  uint16_t *kn = xmalloc(sizeof(uint16_t) * N * Hkv * D), *vn = xmalloc(sizeof(uint16_t) * N * Hkv * D);
  for (int i = 0; i < N * Hkv * D; ++i) {
    kn[i] = oracle_float_to_half(3 * frand());
    vn[i] = oracle_float_to_half(3 * frand());
  }
  /* skipped: sequence -1, sequence 3 (= batch), position 40 (= max_len); sequence 0 has no
   * pages (table entry -1): its write is dropped without counting as a skip */
  int32_t bi[8] = {1, 2, 2, -1, 3, 1, 2, 0}, pos[8] = {4, 0, 36, 0, 0, 5, 40, 0};
  oracle_append_problem ap = {N, Hkv, D, P, int8, B, max_pages * P, 0, kn, vn, (int64_t)Hkv * D, D,
                              bi, pos, k, v, ks, vs, (int64_t)P * Hkv * D, (int64_t)Hkv * D, D,
                              total_pages, total_pages, (int64_t)P * Hkv * (D / 32),
                              (int64_t)Hkv * (D / 32), D / 32, table, max_pages, 0.05f, 0.07f};
  const int64_t skipped = oracle_append(&ap);
  bad |= skipped != 3;
  /* merge two states of every row, one of them empty for the first rows */
  double *os = xmalloc(sizeof(double) * 2 * rows * D), *ls = xmalloc(sizeof(double) * 2 * rows);
  memcpy(os, o, sizeof(double) * rows * D);
  memcpy(os + rows * D, o2, sizeof(double) * rows * D);
  memcpy(ls, lse, sizeof(double) * rows);
  memcpy(ls + rows, lse2, sizeof(double) * rows);
  bad |= oracle_merge_states(2, rows, D, os, ls, o2, lse2) != 0;
  free(os); free(ls); free(kn); free(vn); free(dk); free(dv); free(dks); free(dvs);
  free(o); free(lse); free(o2); free(lse2); free(q); free(kv_len); free(table);
  free(k); free(v); free(ks); free(vs);
  return bad;
}

int main(void) {
  int bad = 0;
  for (int int8 = 0; int8 < 3; ++int8) /* f16, int8, fp8 */
    for (int T = 1; T <= 3; T += 2) bad |= run(int8, T);
  printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
  return bad;
}
