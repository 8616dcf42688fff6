/*
 * Reference (oracle) for sliding-window scaled-dot-product attention,
 * forward and backward, in plain fp64 C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links it, and the two share no code.
 *
 * Sources (web pages; cited by title and section):
 *   [PR866] cudnn-frontend PR #866, "frost(sdpa): bound the SM80 backward
 *           q-loop by the sliding window ... + window-aware deterministic
 *           relay" -- commit message and "Change" section: the anchor
 *           (q, or q + causal_diag under bottom-right), the per-element
 *           causal + left-window mask, per-sequence indices for THD.
 *   [PR557] cudnn-frontend PR #557, "frost(sdpa): GQA/MQA, padding mask,
 *           right-band widening, and sink-token gradients for the SM120 f16
 *           backward" -- "Summary" section: H_q a multiple of H_kv, per-batch
 *           sequence lengths, sink logit in the softmax denominator and the
 *           dSink formula; review comments: padded query rows skipped in
 *           dSink.
 *
 * Addressing.  Element (b, h, i, d) of Q / O / dO (and of the dQ output) is at
 *   (row0_q[b] + i) * q_stride_r + h * q_stride_h + d
 * and of K / V (dK / dV outputs) at
 *   (row0_kv[b] + j) * kv_stride_r + h_kv * kv_stride_h + d.
 * Dense [B,H,S,D] uses row0 = b*H*S, stride_r = D, stride_h = S*D; packed
 * [T,H,D] uses row0 = cu_seqlens[b], stride_r = H*D, stride_h = D.
 * Row statistics (LSE, delta) use index (b*heads_q + h)*stat_ld + i.
 *
 * Output arrays must be zero-filled by the caller; rows at or beyond a
 * sequence's valid length are never written (so they stay exactly zero).
 */
#ifndef SWA_ORACLE_H
#define SWA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_BF16 = 0, ORACLE_F16 = 1, ORACLE_F64 = 2 };

typedef struct oracle_problem {
  int dtype;            /* storage type of q, k, v, dO (ORACLE_*)            */
  int batch, heads_q, heads_kv, head_dim;
  int causal;           /* 1: keys right of the anchor are masked            */
  int bottom_right;     /* 1: anchor(i) = i + len_kv - len_q, else i         */
  int window_left;      /* < 0: no window; else keep anchor - j <= window    */
  int window_right;     /* causal only, >= 0: keep j - anchor <= window_right
                           (right-band widening; 0 is plain causal)          */
  int dense;            /* 1: scan every key and test the mask (slow check)  */
  int has_sink;         /* sink[h_q]: an extra logit in each row's softmax   */
  double scale;         /* multiplies <Q_i, K_j>; the sink is not scaled     */
  const int32_t* len_q;  /* [batch] valid query rows of each sequence        */
  const int32_t* len_kv; /* [batch] valid key rows                           */
  const int64_t* row0_q; /* [batch] first row of each sequence               */
  const int64_t* row0_kv;
  int64_t q_stride_h, q_stride_r;
  int64_t kv_stride_h, kv_stride_r;
  int64_t stat_ld;       /* leading dimension of LSE / delta outputs         */
} oracle_problem;

/* Forward: O (fp64, q addressing) and LSE (natural log; -inf for a row with
 * no visible key and no sink).  Returns 0, or -1 on a bad argument. */
int oracle_forward(const oracle_problem* p, const void* q, const void* k,
                   const void* v, const double* sink, double* o, double* lse);

/* Backward of L = sum(dO * O) with dO held fixed: dq (q addressing),
 * dk / dv (kv addressing), dsink[heads_q] (may be NULL without a sink).
 * o / lse / delta may be NULL; when given they receive the forward output,
 * the row LSE and delta_i = <dO_i, O_i>. */
int oracle_backward(const oracle_problem* p, const void* q, const void* k,
                    const void* v, const void* dO, const double* sink,
                    double* dq, double* dk, double* dv, double* dsink,
                    double* o, double* lse, double* delta);

/* Sampled backward: gradient rows computed one at a time.
 * dq rows for n samples (b[s], h_q[s], i[s]) -> out[s*head_dim + d];
 * dk / dv rows for n samples (b[s], h_kv[s], j[s]).
 * A sample outside the valid rows yields a zero row. */
int oracle_dq_rows(const oracle_problem* p, const void* q, const void* k,
                   const void* v, const void* dO, const double* sink, int n,
                   const int32_t* b, const int32_t* h, const int32_t* i,
                   double* out);
int oracle_dkdv_rows(const oracle_problem* p, const void* q, const void* k,
                     const void* v, const void* dO, const double* sink, int n,
                     const int32_t* b, const int32_t* hk, const int32_t* j,
                     double* dk_out, double* dv_out);

/* Number of (query, key) pairs the mask keeps for one query head, summed
 * over sequences: the attended-pair count used for FLOP accounting. */
int64_t oracle_attended_pairs(const oracle_problem* p);

/* Threads the oracle uses (OpenMP). */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
