/* Drives every entry point of the fp64 oracle on small problems whose
 * buffers are allocated at exactly their required sizes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
 * Cases: dense GQA with a sink, a left window and a right band (bf16 and
 * fp64 storage), and a packed batch with padded slots, an empty query
 * sequence and an empty key sequence.  Exit status 0 when every call
 * succeeds and every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/swa_oracle.h"

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double unit(void) { /* splitmix64, mapped to [-1, 1) */
  uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}

static void* fill(int dtype, int64_t n) {
  if (dtype == ORACLE_F64) {
    double* x = malloc(sizeof(double) * (size_t)(n ? n : 1));
    for (int64_t i = 0; i < n; ++i) x[i] = unit();
    return x;
  }
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(n ? n : 1));
  for (int64_t i = 0; i < n; ++i) { /* a finite 16-bit pattern: sign, small exponent, mantissa */
    const uint16_t m = (uint16_t)((uint64_t)(unit() * 1e6) & 0x7f);
    x[i] = (uint16_t)((dtype == ORACLE_BF16 ? 0x3e00u : 0x3400u) | m | (unit() < 0 ? 0x8000u : 0u));
  }
  return x;
}

static int finite_all(const double* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

static int run_case(const char* name, oracle_problem* p, int64_t q_elems, int64_t kv_elems) {
  const int Hq = p->heads_q, D = p->head_dim;
  void* q = fill(p->dtype, q_elems);
  void* k = fill(p->dtype, kv_elems);
  void* v = fill(p->dtype, kv_elems);
  void* dO = fill(p->dtype, q_elems);
  double* sink = NULL;
  if (p->has_sink) {
    sink = malloc(sizeof(double) * (size_t)Hq);
    for (int h = 0; h < Hq; ++h) sink[h] = unit();
  }
  const int64_t nstat = (int64_t)p->batch * Hq * p->stat_ld;
  double* o = calloc((size_t)(q_elems ? q_elems : 1), sizeof(double));
  double* lse = calloc((size_t)(nstat ? nstat : 1), sizeof(double));
  double* delta = calloc((size_t)(nstat ? nstat : 1), sizeof(double));
  double* dq = calloc((size_t)(q_elems ? q_elems : 1), sizeof(double));
  double* dk = calloc((size_t)(kv_elems ? kv_elems : 1), sizeof(double));
  double* dv = calloc((size_t)(kv_elems ? kv_elems : 1), sizeof(double));
  double* dsink = p->has_sink ? calloc((size_t)Hq, sizeof(double)) : NULL;
  int ok = 1;
  ok &= oracle_forward(p, q, k, v, sink, o, lse) == 0;
  ok &= oracle_backward(p, q, k, v, dO, sink, dq, dk, dv, dsink, o, lse, delta) == 0;
  ok &= finite_all(o, q_elems) && finite_all(dq, q_elems) && finite_all(dk, kv_elems) && finite_all(dv, kv_elems);
  if (dsink) ok &= finite_all(dsink, Hq);
  /* sampled rows, including samples outside the valid rows (zero rows) */
  enum { NS = 6 };
  int32_t b[NS], h[NS], r[NS];
  for (int s = 0; s < NS; ++s) {
    b[s] = s % p->batch;
    h[s] = s % Hq;
    r[s] = s * 5 - 2 * (s == NS - 1);
  }
  double* rows = malloc(sizeof(double) * NS * D);
  double* rows2 = malloc(sizeof(double) * NS * D);
  ok &= oracle_dq_rows(p, q, k, v, dO, sink, NS, b, h, r, rows) == 0;
  for (int s = 0; s < NS; ++s) h[s] = s % p->heads_kv;
  ok &= oracle_dkdv_rows(p, q, k, v, dO, sink, NS, b, h, r, rows, rows2) == 0;
  ok &= finite_all(rows, NS * D) && finite_all(rows2, NS * D);
  ok &= oracle_attended_pairs(p) >= 0;
  p->dense = 1;
  ok &= oracle_backward(p, q, k, v, dO, sink, dq, dk, dv, dsink, NULL, NULL, NULL) == 0;
  p->dense = 0;
  printf("%-34s %s\n", name, ok ? "ok" : "FAILED");
  free(q); free(k); free(v); free(dO); free(sink); free(o); free(lse); free(delta);
  free(dq); free(dk); free(dv); free(dsink); free(rows); free(rows2);
  return ok;
}

int main(void) {
  int ok = 1;
  for (int dt = 0; dt < 3; dt += 2) { /* bf16, fp64 storage */
    /* dense [B, H, S, D], GQA 4/2, bottom-right, W = 3, right band 2, sink */
    const int B = 2, Hq = 4, Hkv = 2, Sq = 9, Skv = 13, D = 8;
    int32_t lq[2] = {9, 6}, lk[2] = {13, 10};
    int64_t r0q[2] = {0, (int64_t)Hq * Sq}, r0k[2] = {0, (int64_t)Hkv * Skv};
    oracle_problem p;
    memset(&p, 0, sizeof p);
    p.dtype = dt; p.batch = B; p.heads_q = Hq; p.heads_kv = Hkv; p.head_dim = D;
    p.causal = 1; p.bottom_right = 1; p.window_left = 3; p.window_right = 2; p.has_sink = 1;
    p.scale = 0.35; p.len_q = lq; p.len_kv = lk; p.row0_q = r0q; p.row0_kv = r0k;
    p.q_stride_h = (int64_t)Sq * D; p.q_stride_r = D; p.kv_stride_h = (int64_t)Skv * D; p.kv_stride_r = D;
    p.stat_ld = Sq;
    ok &= run_case(dt == 0 ? "dense gqa band sink bf16" : "dense gqa band sink f64", &p,
                   (int64_t)B * Hq * Sq * D, (int64_t)B * Hkv * Skv * D);
  }
  {
    /* packed [T, H, D]: padded slots, an empty query and an empty key sequence */
    const int Hq = 4, Hkv = 1, D = 8;
    int32_t lq[4] = {5, 0, 7, 3}, lk[4] = {9, 4, 0, 6};
    int64_t cq[5] = {0, 8, 8, 16, 20}, ck[5] = {0, 9, 14, 14, 22};
    oracle_problem p;
    memset(&p, 0, sizeof p);
    p.dtype = ORACLE_F16; p.batch = 4; p.heads_q = Hq; p.heads_kv = Hkv; p.head_dim = D;
    p.causal = 1; p.bottom_right = 1; p.window_left = 4; p.has_sink = 1; p.scale = 0.5;
    p.len_q = lq; p.len_kv = lk; p.row0_q = cq; p.row0_kv = ck;
    p.q_stride_h = D; p.q_stride_r = (int64_t)Hq * D; p.kv_stride_h = D; p.kv_stride_r = (int64_t)Hkv * D;
    p.stat_ld = 8;
    ok &= run_case("packed thd empty sequences f16", &p, cq[4] * Hq * D, ck[4] * Hkv * D);
  }
  return ok ? 0 : 1;
}
