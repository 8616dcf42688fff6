/*
 * swa_sdpa -- sliding-window scaled-dot-product attention for MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels: a window-trimmed forward that
 * produces O and the row log-sum-exp, and the window-bounded backward that
 * produces dQ, dK, dV (and dSink) from Q, K, V, O, dO and LSE.
 *
 * Sources (web pages; cited by title and section):
 *   [PR866] cudnn-frontend PR #866 "frost(sdpa): bound the SM80 backward
 *           q-loop by the sliding window (6-12x on gpt_oss-style SWA) +
 *           window-aware deterministic relay": commit message, Change.
 *   [PR557] cudnn-frontend PR #557 "frost(sdpa): GQA/MQA, padding mask,
 *           right-band widening, and sink-token gradients for the SM120 f16
 *           backward": Summary, review comments.
 *   [PR2352] cudnn-frontend PR #2352 "sdpa bwd: lead square A100 backward
 *           window graphs from a measured study": Measurement, Not measured.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller allocates and frees every device buffer
 *     (inputs, outputs and the workspace).  The library never allocates
 *     device memory and never synchronizes the stream.  Plans are host
 *     objects owned by the caller (destroy them with *_plan_destroy).
 *   - Pointers named as device pointers must be device memory of the
 *     current HIP device; host pointers are plain host memory.
 *   - Errors are returned as sdpa_status; nothing is thrown across the ABI.
 *     sdpa_last_error() returns a thread-local message naming the field or
 *     tensor at fault.  A failed call leaves outputs unspecified.
 *   - Runs are stream-ordered and asynchronous.  A plan is immutable (but
 *     for the test hook sdpa_bwd_plan_set_relay_watchdog) and may be used by
 *     concurrent runs that use distinct workspaces.
 */
#ifndef SWA_SDPA_H
#define SWA_SDPA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_INVALID_ARG = 1, /* a descriptor field or a pointer is invalid   */
  SDPA_ERR_UNSUPPORTED = 2, /* valid, but not provided (e.g. head_dim 96)  */
  SDPA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned  */
  SDPA_ERR_HIP = 4,         /* a HIP runtime call (e.g. a launch) failed   */
  SDPA_ERR_RELAY_TIMEOUT = 5 /* an ordered-relay wait of a run gave up:
                               that run's dQ is invalid (see
                               sdpa_bwd_relay_expiries)                     */
} sdpa_status;

typedef enum sdpa_dtype { SDPA_BF16 = 0, SDPA_F16 = 1 } sdpa_dtype;

/* BHSD: dense [B, H, S, D] (any batch / head / row strides, D contiguous).
 * THD : packed [T, H, D]; sequence b owns the row slots
 *       [cu_seqlens[b], cu_seqlens[b+1]) of which the first seq_lens[b] are
 *       valid (the rest is padding). */
typedef enum sdpa_layout { SDPA_LAYOUT_BHSD = 0, SDPA_LAYOUT_THD = 1 } sdpa_layout;

/*
 * Problem descriptor, shared by the forward and the backward.
 *
 * Mask ([PR866] commit message): query row i of a sequence has the anchor
 * a(i) = i (top-left) or i + s_kv - s_q (bottom-right), in-sequence indices.
 * Key j is visible when j < s_kv, i < s_q, j <= a(i) + window_right if
 * causal, and a(i) - j <= window_left if window_left >= 0 (an inclusive left
 * window of window_left + 1 keys).  window_right is the right-band widening
 * of [PR557] (Summary), which names it without a formula; it is read here
 * as an inclusive right bound, 0 giving the plain causal mask.  With a sink ([PR557] Summary) the per-query-head
 * logit sink[h] (not multiplied by scale) joins each row's softmax
 * denominator.  GQA / MQA ([PR557] Summary): query head h reads kv head
 * h / (heads_q / heads_kv).
 */
typedef struct sdpa_attn_desc {
  int32_t dtype;        /* sdpa_dtype of Q, K, V, O, dO, dQ, dK, dV          */
  int32_t layout;       /* sdpa_layout                                       */
  int32_t batch;        /* B: batches (BHSD) or packed sequences (THD), >= 1 */
  int32_t heads_q;      /* query heads, a multiple of heads_kv               */
  int32_t heads_kv;     /* key / value heads (1 = MQA)                       */
  int32_t head_dim;     /* 64 or 128                                         */
  int32_t seq_q;        /* BHSD: S_q.  THD: >= every slot capacity           */
  int32_t seq_kv;       /* BHSD: S_kv. THD: >= every slot capacity           */
  int64_t total_q;      /* THD: rows of the packed Q buffer; BHSD: ignored   */
  int64_t total_kv;     /* THD: rows of the packed K / V buffers             */
  int32_t causal;       /* 1: mask keys after the anchor                     */
  int32_t bottom_right; /* 1: anchor i + s_kv - s_q; 0: anchor i             */
  int32_t window_left;  /* -1: none; >= 0: inclusive left window W           */
  int32_t window_right; /* >= 0, causal only: keys up to a(i) + window_right
                           are visible (0: plain causal)                      */
  float scale;          /* softmax scale on Q.K (> 0), e.g. 1/sqrt(D)        */
  int32_t deterministic; /* backward: 0 unordered (fp32 atomics where
                            blocks share a dQ tile); 1 bitwise repeatable,
                            by the fastest ordered method (the streaming
                            kernel's chunk relay, or the relay-free q-major
                            dQ pass of the per-tile path); 2 the per-kv-tile
                            ordered relay of [PR866] on the per-tile path,
                            for every shape                                 */
  int32_t has_sink;     /* 1: sink logits given (fp32 [heads_q])             */
  int32_t has_seq_lens; /* 1: seq_lens_q / seq_lens_kv given (THD requires)  */
  int32_t q_run_tiles;  /* 0: the measured default; 1..16: consecutive 64-row
                           q-tiles one block of the q-major passes (forward,
                           unordered dQ of the per-tile path) walks; for
                           tuning studies                                     */
  int32_t engine;       /* backward kernels and dQ mechanism.  0: chosen by
                           the plan from a measured table, among those the
                           deterministic option allows.  For tuning studies,
                           1..5 force one: 1 streaming kernel with fp32
                           atomics at chunk boundaries, 2 streaming kernel
                           with the chunk relay, 3 per-tile kernels with the
                           q-major dQ pass, 4 per-tile kernel with the
                           per-kv-tile relay, 5 q-major streaming kernel
                           (one pass; repeatable).  1 and 2 need heads_q ==
                           heads_kv, causal, window_right 0, window_left
                           0..128, head_dim 64; 5 needs head_dim 128,
                           causal, window_right 0, window_left 0..96, BHSD
                           without seq_lens, seq_kv - seq_q a multiple of 32
                           if bottom-right, at most 64 query heads per kv
                           head with a sink (SDPA_ERR_UNSUPPORTED
                           otherwise); 1 needs deterministic 0, and
                           deterministic 2 admits only 4
                           (SDPA_ERR_INVALID_ARG otherwise).  The forward:
                           0 takes the q-major forward where it applies,
                           5 forces it (engine 5's shapes, with heads_q /
                           heads_kv a multiple of 8, at most 512, and
                           seq_kv > 0; SDPA_ERR_UNSUPPORTED otherwise),
                           1..4 run the per-tile forward.                     */
  /* Element strides (batch, head, row) of each tensor; the head_dim axis is
   * contiguous.  THD ignores the batch entry (rows are tokens).  Rows and
   * base pointers must be 16-byte aligned; row strides below 2^32 elements
   * (SDPA_ERR_UNSUPPORTED otherwise). */
  int64_t stride_q[3], stride_k[3], stride_v[3], stride_o[3], stride_do[3];
  int64_t stride_dq[3], stride_dk[3], stride_dv[3];
} sdpa_attn_desc;

/* Row statistics (LSE) layout: BHSD [B, heads_q, seq_q]; THD
 * [heads_q, total_q] (head-major, indexed by packed row).  fp32, natural
 * log; -inf for a row with no visible key and no sink, and for padding. */

typedef struct sdpa_fwd_tensors {
  const void* q;                /* device, dtype, Q                           */
  const void* k;                /* device, dtype, K                           */
  const void* v;                /* device, dtype, V                           */
  const float* sink;            /* device fp32 [heads_q] or NULL              */
  const int32_t* cu_seqlens_q;  /* device int32 [B+1] (THD) or NULL           */
  const int32_t* cu_seqlens_kv; /* device int32 [B+1] (THD) or NULL           */
  const int32_t* seq_lens_q;    /* device int32 [B] valid rows, or NULL       */
  const int32_t* seq_lens_kv;   /* device int32 [B] valid rows, or NULL       */
  void* o;                      /* device output, dtype, O (padding -> 0)     */
  float* lse;                   /* device output fp32, layout above           */
} sdpa_fwd_tensors;

typedef struct sdpa_bwd_tensors {
  const void* q;                /* device inputs, dtype                       */
  const void* k;
  const void* v;
  const void* o;                /* forward output O                           */
  const void* dO;               /* gradient of the loss with respect to O     */
  const float* lse;             /* forward row LSE (layout above)             */
  const float* sink;            /* device fp32 [heads_q] or NULL              */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  const int32_t* seq_lens_q;
  const int32_t* seq_lens_kv;
  void* dq;                     /* device outputs, dtype; padding rows -> 0   */
  void* dk;
  void* dv;
  float* dsink;                 /* device fp32 [heads_q] output, or NULL      */
} sdpa_bwd_tensors;

typedef struct sdpa_bwd_plan sdpa_bwd_plan_t;
typedef struct sdpa_fwd_plan sdpa_fwd_plan_t;

/*
 * sdpa_bwd_plan -- validate a descriptor and build a backward plan.
 * Host only: no device call.  *workspace_bytes receives the size of the
 * device workspace sdpa_bwd_run needs (256-byte aligned).  Rejects, among
 * others: head_dim other than 64/128, heads_q % heads_kv != 0, a dense
 * bottom-right mask with seq_q > seq_kv (every early row would see no key;
 * [PR2352] Not measured), THD without seq lens.
 */
sdpa_status sdpa_bwd_plan(const sdpa_attn_desc* desc, sdpa_bwd_plan_t** plan,
                          size_t* workspace_bytes);

/*
 * sdpa_bwd_run -- enqueue the backward on `stream`:
 *   1. dot  : delta_i = <dO_i, O_i> per row, per-row dSink terms, and
 *             clearing of the relay counters / dQ accumulator;
 *   2. main : per kv-tile, the window-bounded q-tile loop ([PR866] Change):
 *             recompute P, dS = P (dP - delta), accumulate dK / dV over the
 *             kv head's query-head group ([PR557] Summary), add dS K into
 *             dQ through the ordered relay whose turns count from kv_first
 *             ([PR866] commit message) or, unordered, through fp32 atomics
 *             (multi-head windows up to 128 keys: only at the boundaries of
 *             the streaming kernel's chunks, converted by the last chunk);
 *             a kv-tile with no q-tile stores dK = dV = 0;
 *   3. dq   : (unordered mode, other shapes) a q-major pass that writes
 *             dQ = scale * sum_j dS_ij K_j once per row;
 *   4. dsink: fixed-order reduction dSink[h] = -sum exp(sink_h - LSE) delta
 *             over valid rows ([PR557] Summary and review).
 * `workspace` is a device buffer of at least the planned size.
 */
sdpa_status sdpa_bwd_run(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* tensors,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* As sdpa_bwd_run, also recording `main_start` / `main_stop` (created by the
 * caller, may be NULL) on `stream` right around the main kernel, so its
 * duration can be read with hipEventElapsedTime. */
sdpa_status sdpa_bwd_run_events(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* tensors,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                hipEvent_t main_start, hipEvent_t main_stop);

void sdpa_bwd_plan_destroy(sdpa_bwd_plan_t* plan);

/*
 * sdpa_bwd_run_noalloc -- sdpa_bwd_run for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same kernels and results as
 * sdpa_bwd_run (bitwise in the ordered modes), but the workspace is the
 * library's own 64 MiB scratch array: each GPU the library runs on holds
 * one until the process ends.  The caller still passes (and owns) the
 * inputs and outputs.  No allocation and no synchronization happen here.
 * Errors: SDPA_ERR_WORKSPACE (with a message naming both sizes) when the
 * plan's workspace (the size sdpa_bwd_plan reported) exceeds 64 MiB;
 * SDPA_ERR_HIP if the scratch address cannot be looked up; otherwise those
 * of sdpa_bwd_run.  Every call on one GPU shares that GPU's array and it
 * keeps the last call's contents (the kernels clear what must start at
 * zero): calls that overlap on one GPU, on any streams, race.
 */
sdpa_status sdpa_bwd_run_noalloc(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* tensors,
                                 hipStream_t stream);

/*
 * sdpa_fwd_plan / sdpa_fwd_run -- the window-trimmed forward
 * ([PR866] Problem: the forward already trims its kv range by the window):
 * each q-tile walks only the kv-tiles [kv_first, kv_last] its rows can see
 * and writes O (dtype) and LSE (fp32).  For head_dim 128, short windows and
 * query-head groups of a multiple of 8 (see `engine`), a q-major kernel
 * walks 32-row q-steps of a (sequence, kv head) with the window's kv-tiles
 * resident and every head of the group reading them.  Workspace is 0 bytes
 * today; pass the planned size anyway.
 */
sdpa_status sdpa_fwd_plan(const sdpa_attn_desc* desc, sdpa_fwd_plan_t** plan,
                          size_t* workspace_bytes);
sdpa_status sdpa_fwd_run(const sdpa_fwd_plan_t* plan, const sdpa_fwd_tensors* tensors,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);
void sdpa_fwd_plan_destroy(sdpa_fwd_plan_t* plan);

/*
 * sdpa_bwd_schedule -- host-side view of a plan's tile schedule for one
 * sequence of valid lengths (len_q, len_kv).  Writes the tile sizes, then
 * for each kv-tile j < n_kv (n_kv <= kv_cap) q_lo[j], q_hi[j] (q_hi <= q_lo
 * means the tile stores zeros), and for each q-tile i < n_q (<= q_cap)
 * kv_first[i], kv_last[i] (the relay visitor range).  Any array may be
 * NULL.  Host only.
 */
sdpa_status sdpa_bwd_schedule(const sdpa_bwd_plan_t* plan, int32_t len_q, int32_t len_kv,
                              int32_t* tile_q, int32_t* tile_kv, int32_t* n_q, int32_t* n_kv,
                              int32_t kv_cap, int32_t* q_lo, int32_t* q_hi, int32_t q_cap,
                              int32_t* kv_first, int32_t* kv_last);

/*
 * sdpa_bwd_relay_expiries -- outcome of the ordered dQ relay of the last run
 * on `workspace` (deterministic = 1 or 2).  Each relay wait ([PR866] commit
 * message: a visitor waits for its turn, counted from the q-tile's first
 * visitor; its tests note that a wrong first visitor would hang or
 * mis-order) is bounded by a watchdog of 2^20 spins (~55 ms) so that the
 * device never hangs.  A wait that gives up counts an expiry and adds NaN
 * instead of its partial, so the q-tile's dQ rows come out NaN, never
 * plausible but out of order (a late predecessor may still overwrite a
 * poisoned partial: treat the whole dQ of such a run as invalid).
 * Copies to *count (host) the number of waits that gave up, synchronizing
 * `stream`, and returns SDPA_ERR_RELAY_TIMEOUT when it is > 0, SDPA_OK
 * when every turn arrived in order.  sdpa_bwd_run cannot report this
 * itself: it returns before the kernels run.
 */
sdpa_status sdpa_bwd_relay_expiries(const sdpa_bwd_plan_t* plan, const void* workspace,
                                    hipStream_t stream, int32_t* count);

/*
 * sdpa_bwd_plan_set_relay_watchdog -- test hook for the watchdog path.
 * spin_limit > 0 sets the spins before a relay wait gives up (0 restores
 * the default 2^20).  unreachable = 1 makes every wait target a turn no
 * visitor ever releases, so each non-first turn gives up after spin_limit
 * spins and every kernel still runs to its end: a host-forced timeout for
 * tests.  Host only; changes the plan, so call it before runs that use the
 * plan, not concurrently with them.
 */
sdpa_status sdpa_bwd_plan_set_relay_watchdog(sdpa_bwd_plan_t* plan, int32_t spin_limit, int32_t unreachable);

const char* sdpa_status_string(sdpa_status status);
const char* sdpa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SWA_SDPA_H */
