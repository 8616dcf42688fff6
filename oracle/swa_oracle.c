/*
 * fp64 reference for sliding-window attention (forward + backward).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and
 * the benchmark's CPU-baseline leg, never by the GPU library.  It shares no
 * code with the GPU path.  See swa_oracle.h for the sources and addressing.
 *
 * Everything here is the plain definition written out, one query row at a
 * time, in double precision; inputs stored as bf16 / f16 are widened
 * exactly.  No tiling, no fusion, no reordering.
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one known mistake; the test
 * suite builds such variants to show that its pins catch each of them.
 */
#include "swa_oracle.h"

#include <math.h>
#include <omp.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* ---- element access ---------------------------------------------------- */

/* IEEE binary16: sign, 5 exponent bits (bias 15), 10 fraction bits. */
static double f16_to_double(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
#if ORACLE_MUTANT == 11
    v = ldexp((double)m, -25);
#else
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
#endif
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
#if ORACLE_MUTANT == 10
    v = ldexp((double)(m | 0x400), e - 24);
#else
    v = ldexp((double)(m | 0x400), e - 25); /* (1024 + m) * 2^(e - 25) */
#endif
  return s ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double bf16_to_double(uint16_t h) {
#if ORACLE_MUTANT == 13
  if (((h >> 7) & 0xff) == 0) h &= 0x8000; /* subnormals flushed to zero */
#endif
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* f16_to_double of every bit pattern, filled once before any parallel
 * region (widening through ldexp per element dominated the oracle's time on
 * f16 inputs). */
static double f16_table[1 << 16];
static pthread_once_t f16_once = PTHREAD_ONCE_INIT;
static void fill_f16_table(void) {
  for (int h = 0; h < (1 << 16); ++h) f16_table[h] = f16_to_double((uint16_t)h);
}
static void widen_init(void) { pthread_once(&f16_once, fill_f16_table); }

static double ld(const void* base, int dtype, int64_t idx) {
#if ORACLE_MUTANT == 12
  if (dtype != ORACLE_F64) dtype = dtype == ORACLE_BF16 ? ORACLE_F16 : ORACLE_BF16;
#endif
  switch (dtype) {
    case ORACLE_BF16: return bf16_to_double(((const uint16_t*)base)[idx]);
    case ORACLE_F16: return f16_table[((const uint16_t*)base)[idx]];
    default: return ((const double*)base)[idx];
  }
}

static int64_t q_at(const oracle_problem* p, int b, int h, int i) {
  return (p->row0_q[b] + i) * p->q_stride_r + (int64_t)h * p->q_stride_h;
}
static int64_t kv_at(const oracle_problem* p, int b, int hk, int j) {
  return (p->row0_kv[b] + j) * p->kv_stride_r + (int64_t)hk * p->kv_stride_h;
}

/* GQA / MQA: query heads are split into heads_kv contiguous groups, group g
 * reads kv head g ([PR557] Summary: H_q a multiple of H_kv). */
static int kv_head_of(const oracle_problem* p, int h) {
#if ORACLE_MUTANT == 8
  return h % p->heads_kv;
#else
  return h / (p->heads_q / p->heads_kv);
#endif
}

/* ---- the mask ([PR866] commit message and Change section) ---------------
 * anchor(i) = i (top-left) or i + len_kv - len_q (bottom-right), with the
 * in-sequence indices of the row's own sequence.  Key j is visible from row
 * i when both lie inside their sequences' valid lengths, j <= anchor(i) if
 * causal, and anchor(i) - j <= window_left if a window is set (inclusive:
 * window_left + 1 keys including the diagonal).  Right-band widening
 * ([PR557] Summary names it, without a formula) moves the causal bound to
 * j <= anchor(i) + window_right, read as inclusive like the left window. */
static long anchor_of(const oracle_problem* p, int b, int i) {
#if ORACLE_MUTANT == 6
  return p->bottom_right ? (long)i + p->len_q[b] - p->len_kv[b] : (long)i;
#else
  return p->bottom_right ? (long)i + p->len_kv[b] - p->len_q[b] : (long)i;
#endif
}

static int visible(const oracle_problem* p, int b, int i, int j) {
  if (i < 0 || i >= p->len_q[b] || j < 0 || j >= p->len_kv[b]) return 0;
  long a = anchor_of(p, b, i);
#if ORACLE_MUTANT == 9
  if (p->causal && j - a >= (p->window_right > 0 ? p->window_right : 1)) return 0;
#else
  if (p->causal && j > a + p->window_right) return 0;
#endif
#if ORACLE_MUTANT == 2
  if (p->window_left >= 0 && a - j >= p->window_left) return 0;
#else
  if (p->window_left >= 0 && a - j > p->window_left) return 0;
#endif
  return 1;
}

/* Keys a row can see form one interval [lo, hi]; the loops below walk it
 * (O(S*W) work) unless p->dense asks to scan every key through visible(). */
static void key_range(const oracle_problem* p, int b, int i, int* lo, int* hi) {
  if (p->dense) {
    *lo = 0;
    *hi = p->len_kv[b] - 1;
    return;
  }
  long a = anchor_of(p, b, i);
  long l = 0, r = p->len_kv[b] - 1;
  if (p->window_left >= 0 && a - p->window_left > l) l = a - p->window_left;
  if (p->causal && a + p->window_right < r) r = a + p->window_right;
  *lo = (int)l;
  *hi = (int)r;
}

static double dot_qk(const oracle_problem* p, const void* x, int64_t xo, const void* y,
                     int64_t yo) {
  double s = 0.0;
  for (int d = 0; d < p->head_dim; ++d) s += ld(x, p->dtype, xo + d) * ld(y, p->dtype, yo + d);
  return s;
}

/* ---- one row of the forward ----------------------------------------------
 * s_j = scale * <Q_i, K_j> over visible keys; with a sink the logit sink[h]
 * joins the softmax denominator only ([PR557] Summary).  m = max(s_j, sink),
 * LSE = m + log(sum_j exp(s_j - m) + exp(sink - m)), P_j = exp(s_j - LSE),
 * O_i = sum_j P_j V_j.  No visible key and no sink: LSE = -inf, O_i = 0.
 * s (scratch, >= len_kv doubles) receives the logits; returns LSE. */
static double row_forward(const oracle_problem* p, int b, int h, int i, const void* q,
                          const void* k, const void* v, const double* sink, double* s,
                          double* o_row) {
  const int D = p->head_dim, hk = kv_head_of(p, h);
  int lo, hi;
  key_range(p, b, i, &lo, &hi);
  const int64_t qo = q_at(p, b, h, i);
  double m = -INFINITY;
  int any = 0;
  for (int j = lo; j <= hi; ++j) {
    if (!visible(p, b, i, j)) continue;
    s[j] = p->scale * dot_qk(p, q, qo, k, kv_at(p, b, hk, j));
    if (s[j] > m) m = s[j];
    any = 1;
  }
  for (int d = 0; d < D; ++d) o_row[d] = 0.0;
  int use_sink = p->has_sink && sink;
#if ORACLE_MUTANT == 4
  use_sink = 0;
#endif
  if (use_sink && sink[h] > m) m = sink[h];
  if (!any && !use_sink) return -INFINITY;
  double l = use_sink ? exp(sink[h] - m) : 0.0;
  for (int j = lo; j <= hi; ++j)
    if (visible(p, b, i, j)) l += exp(s[j] - m);
  const double lse = m + log(l);
  for (int j = lo; j <= hi; ++j) {
    if (!visible(p, b, i, j)) continue;
    const double pj = exp(s[j] - lse);
    const int64_t vo = kv_at(p, b, hk, j);
    for (int d = 0; d < D; ++d) o_row[d] += pj * ld(v, p->dtype, vo + d);
  }
  return lse;
}

static int check(const oracle_problem* p) {
  if (!p || p->batch < 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->head_dim <= 0) return -1;
  if (p->heads_q % p->heads_kv) return -1;
  if (p->dtype < 0 || p->dtype > 2 || !p->len_q || !p->len_kv || !p->row0_q || !p->row0_kv)
    return -1;
  return 0;
}

static int max_len_kv(const oracle_problem* p) {
  int m = 1;
  for (int b = 0; b < p->batch; ++b)
    if (p->len_kv[b] > m) m = p->len_kv[b];
  return m;
}

int oracle_forward(const oracle_problem* p, const void* q, const void* k, const void* v,
                   const double* sink, double* o, double* lse) {
  if (check(p)) return -1;
  widen_init();
  const int nkv = max_len_kv(p);
  const int units = p->batch * p->heads_q;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * nkv);
    double* orow = (double*)malloc(sizeof(double) * p->head_dim);
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
      const int b = u / p->heads_q, h = u % p->heads_q;
      for (int i = 0; i < p->len_q[b]; ++i) {
        const double l = row_forward(p, b, h, i, q, k, v, sink, s, orow);
        if (lse) lse[((int64_t)b * p->heads_q + h) * p->stat_ld + i] = l;
        if (o) {
          const int64_t oo = q_at(p, b, h, i);
          for (int d = 0; d < p->head_dim; ++d) o[oo + d] = orow[d];
        }
      }
    }
    free(s);
    free(orow);
  }
  return 0;
}

/* ---- one row of the backward ---------------------------------------------
 * Gradient of L = sum(dO * O) for fixed dO (textbook softmax-attention
 * backward):
 *   delta_i = <dO_i, O_i>,   dP_ij = <dO_i, V_j>,   dS_ij = P_ij (dP_ij - delta_i)
 *   dQ_i += scale dS_ij K_j,  dK_j += scale dS_ij Q_i,  dV_j += P_ij dO_i
 *   dsink_h -= exp(sink_h - LSE_i) delta_i   (valid rows only; [PR557] Summary
 *                                             and the review on padded rows)
 * Any of dq_row / dk / dv may be NULL.  With only_j < 0, dk and dv use kv
 * addressing; with only_j >= 0 just key only_j is visited and dk / dv point
 * at that key's single output row. */
static void row_backward(const oracle_problem* p, int b, int h, int i, const void* q,
                         const void* k, const void* v, const void* dO, const double* s,
                         double lse, double delta, double* dq_row, double* dk, double* dv,
                         int only_j) {
  const int D = p->head_dim, hk = kv_head_of(p, h);
  int lo, hi;
  key_range(p, b, i, &lo, &hi);
  if (only_j >= 0) {
    if (only_j < lo || only_j > hi) return;
    lo = hi = only_j;
  }
  const int64_t qo = q_at(p, b, h, i);
  for (int j = lo; j <= hi; ++j) {
    if (!visible(p, b, i, j)) continue;
    const int64_t ko = kv_at(p, b, hk, j);
    const int64_t go = only_j >= 0 ? 0 : ko; /* output row offset */
    const double pij = exp(s[j] - lse);
    const double dp = dot_qk(p, dO, qo, v, ko);
#if ORACLE_MUTANT == 3
    const double ds = pij * (delta - dp);
#else
    const double ds = pij * (dp - delta);
#endif
    for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 1
      if (dq_row) dq_row[d] += ds * ld(k, p->dtype, ko + d);
#else
      if (dq_row) dq_row[d] += p->scale * ds * ld(k, p->dtype, ko + d);
#endif
#if ORACLE_MUTANT == 5
      if (dk) dk[go + d] += p->scale * ds * ld(dO, p->dtype, qo + d);
#else
      if (dk) dk[go + d] += p->scale * ds * ld(q, p->dtype, qo + d);
#endif
      if (dv) dv[go + d] += pij * ld(dO, p->dtype, qo + d);
    }
  }
}

static double row_delta(const oracle_problem* p, int b, int h, int i, const void* dO,
                        const double* o_row) {
  const int64_t qo = q_at(p, b, h, i);
  double dl = 0.0;
  for (int d = 0; d < p->head_dim; ++d) dl += ld(dO, p->dtype, qo + d) * o_row[d];
  return dl;
}

static double sink_term(const oracle_problem* p, int h, const double* sink, double lse,
                        double delta) {
  if (!p->has_sink || !sink) return 0.0;
#if ORACLE_MUTANT == 7
  return exp(sink[h] - lse) * delta;
#else
  return -exp(sink[h] - lse) * delta;
#endif
}

int oracle_backward(const oracle_problem* p, const void* q, const void* k, const void* v,
                    const void* dO, const double* sink, double* dq, double* dk, double* dv,
                    double* dsink, double* o, double* lse, double* delta) {
  if (check(p)) return -1;
  widen_init();
  const int G = p->heads_q / p->heads_kv, D = p->head_dim;
  const int nkv = max_len_kv(p);
  /* One unit = (sequence, kv head): it owns that kv head's dK / dV rows and
   * its query heads' dQ rows, so units never write the same element. */
  const int units = p->batch * p->heads_kv;
  double* sink_part = (double*)calloc((size_t)units * p->heads_q + 1, sizeof(double));
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * nkv);
    double* orow = (double*)malloc(sizeof(double) * D);
    double* dqrow = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
      const int b = u / p->heads_kv, hk = u % p->heads_kv;
      for (int h = 0; h < p->heads_q; ++h) {
        if (kv_head_of(p, h) != hk) continue;
        for (int i = 0; i < p->len_q[b]; ++i) {
          const double l = row_forward(p, b, h, i, q, k, v, sink, s, orow);
          const double dl = row_delta(p, b, h, i, dO, orow);
          const int64_t qo = q_at(p, b, h, i);
          const int64_t si = ((int64_t)b * p->heads_q + h) * p->stat_ld + i;
          if (o)
            for (int d = 0; d < D; ++d) o[qo + d] = orow[d];
          if (lse) lse[si] = l;
          if (delta) delta[si] = dl;
          if (l == -INFINITY) continue; /* no visible key, no sink: P = 0 */
          for (int d = 0; d < D; ++d) dqrow[d] = 0.0;
          row_backward(p, b, h, i, q, k, v, dO, s, l, dl, dqrow, dk, dv, -1);
          if (dq)
            for (int d = 0; d < D; ++d) dq[qo + d] = dqrow[d];
          sink_part[(size_t)u * p->heads_q + h] += sink_term(p, h, sink, l, dl);
        }
      }
    }
    free(s);
    free(orow);
    free(dqrow);
  }
  (void)G;
  if (dsink)
    for (int h = 0; h < p->heads_q; ++h) {
      double acc = 0.0;
      for (int u = 0; u < units; ++u) acc += sink_part[(size_t)u * p->heads_q + h];
      dsink[h] = acc;
    }
  free(sink_part);
  return 0;
}

int oracle_dq_rows(const oracle_problem* p, const void* q, const void* k, const void* v,
                   const void* dO, const double* sink, int n, const int32_t* bs,
                   const int32_t* hs, const int32_t* is, double* out) {
  if (check(p) || n < 0) return -1;
  widen_init();
  const int D = p->head_dim, nkv = max_len_kv(p);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * nkv);
    double* orow = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 4)
    for (int t = 0; t < n; ++t) {
      double* row = out + (int64_t)t * D;
      for (int d = 0; d < D; ++d) row[d] = 0.0;
      const int b = bs[t], h = hs[t], i = is[t];
      if (b < 0 || b >= p->batch || h < 0 || h >= p->heads_q || i < 0 || i >= p->len_q[b])
        continue;
      const double l = row_forward(p, b, h, i, q, k, v, sink, s, orow);
      if (l == -INFINITY) continue;
      const double dl = row_delta(p, b, h, i, dO, orow);
      row_backward(p, b, h, i, q, k, v, dO, s, l, dl, row, NULL, NULL, -1);
    }
    free(s);
    free(orow);
  }
  return 0;
}

int oracle_dkdv_rows(const oracle_problem* p, const void* q, const void* k, const void* v,
                     const void* dO, const double* sink, int n, const int32_t* bs,
                     const int32_t* hks, const int32_t* js, double* dk_out, double* dv_out) {
  if (check(p) || n < 0) return -1;
  widen_init();
  const int D = p->head_dim, nkv = max_len_kv(p);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * nkv);
    double* orow = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < n; ++t) {
      double* dkr = dk_out + (int64_t)t * D;
      double* dvr = dv_out + (int64_t)t * D;
      for (int d = 0; d < D; ++d) dkr[d] = dvr[d] = 0.0;
      const int b = bs[t], hk = hks[t], j = js[t];
      if (b < 0 || b >= p->batch || hk < 0 || hk >= p->heads_kv || j < 0 || j >= p->len_kv[b])
        continue;
      for (int h = 0; h < p->heads_q; ++h) {
        if (kv_head_of(p, h) != hk) continue;
        for (int i = 0; i < p->len_q[b]; ++i) {
          if (!visible(p, b, i, j)) continue;
          const double l = row_forward(p, b, h, i, q, k, v, sink, s, orow);
          const double dl = row_delta(p, b, h, i, dO, orow);
          row_backward(p, b, h, i, q, k, v, dO, s, l, dl, NULL, dkr, dvr, j);
        }
      }
    }
    free(s);
    free(orow);
  }
  return 0;
}

int64_t oracle_attended_pairs(const oracle_problem* p) {
  if (check(p)) return -1;
  int64_t total = 0;
  for (int b = 0; b < p->batch; ++b)
    for (int i = 0; i < p->len_q[b]; ++i) {
      int lo, hi;
      key_range(p, b, i, &lo, &hi);
      for (int j = lo; j <= hi; ++j) total += visible(p, b, i, j);
    }
  return total;
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
