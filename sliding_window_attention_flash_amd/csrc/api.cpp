// C ABI of swa_sdpa: descriptor validation, plans, workspace layout and the
// launch sequence of the forward and the backward.  Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "api_internal.h"
#include "kernels.h"
#include "swa_sdpa.h"

using swa::kTile;

struct sdpa_bwd_plan {
  sdpa_attn_desc desc;
  swa::Problem prob;
  int64_t stat_rows;  // rows of the delta / dQ-accumulator workspace
  size_t off_delta, off_acc, off_stash, off_sem, off_ctl, off_sink, ws_bytes;
  int spin_limit;  // relay watchdog: spins before a wait gives up
  int relay_bias;  // 0, or (test hook) a wait target no visitor releases
};

struct sdpa_fwd_plan {
  sdpa_attn_desc desc;
  swa::Problem prob;
};

namespace {

thread_local char g_err[512] = "";

sdpa_status fail(sdpa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A window (left) or band (right) of at least s_q + s_kv keys masks nothing
// that a shorter one of that length would not; negative stays negative.
int clamp_band(int w, int64_t sq, int64_t skv) {
  return w < 0 ? w : (int)std::min<int64_t>(w, sq + skv);
}

sdpa_status check_strides(const char* name, const int64_t* st, const sdpa_attn_desc* d) {
  const int first = d->layout == SDPA_LAYOUT_THD ? 1 : 0;
  for (int k = first; k < 3; ++k) {
    if (st[k] < 0) return fail(SDPA_ERR_INVALID_ARG, "stride_%s[%d] = %lld is negative", name, k, (long long)st[k]);
    if (st[k] % 8)
      return fail(SDPA_ERR_INVALID_ARG, "stride_%s[%d] = %lld is not a multiple of 8 elements (16-byte rows)",
                  name, k, (long long)st[k]);
  }
  if (st[2] < d->head_dim)
    return fail(SDPA_ERR_INVALID_ARG, "stride_%s row stride %lld is smaller than head_dim %d", name,
                (long long)st[2], d->head_dim);
  if (st[2] > (int64_t)UINT32_MAX)  // the kernels form row offsets with 32 x 32-bit products
    return fail(SDPA_ERR_UNSUPPORTED, "stride_%s row stride %lld exceeds 2^32 - 1 elements", name,
                (long long)st[2]);
  return SDPA_OK;
}

sdpa_status check_desc(const sdpa_attn_desc* d, bool backward) {
  if (!d) return fail(SDPA_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != SDPA_BF16 && d->dtype != SDPA_F16)
    return fail(SDPA_ERR_INVALID_ARG, "dtype %d is not SDPA_BF16 or SDPA_F16", d->dtype);
  if (d->layout != SDPA_LAYOUT_BHSD && d->layout != SDPA_LAYOUT_THD)
    return fail(SDPA_ERR_INVALID_ARG, "layout %d is not BHSD or THD", d->layout);
  if (d->batch < 1) return fail(SDPA_ERR_INVALID_ARG, "batch %d < 1", d->batch);
  if (d->heads_q < 1 || d->heads_kv < 1)
    return fail(SDPA_ERR_INVALID_ARG, "heads_q %d / heads_kv %d must be >= 1", d->heads_q, d->heads_kv);
  if (d->heads_q % d->heads_kv)
    return fail(SDPA_ERR_INVALID_ARG, "heads_q %d is not a multiple of heads_kv %d", d->heads_q, d->heads_kv);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SDPA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are provided", d->head_dim);
  if (d->seq_q < 0 || d->seq_kv < 0)
    return fail(SDPA_ERR_INVALID_ARG, "seq_q %d / seq_kv %d must be >= 0", d->seq_q, d->seq_kv);
  if (d->causal != 0 && d->causal != 1) return fail(SDPA_ERR_INVALID_ARG, "causal %d is not 0/1", d->causal);
  if (d->bottom_right != 0 && d->bottom_right != 1)
    return fail(SDPA_ERR_INVALID_ARG, "bottom_right %d is not 0/1", d->bottom_right);
  if (d->window_left < -1) return fail(SDPA_ERR_INVALID_ARG, "window_left %d < -1", d->window_left);
  if (d->window_right < 0) return fail(SDPA_ERR_INVALID_ARG, "window_right %d < 0", d->window_right);
  if (d->window_right > 0 && !d->causal)
    return fail(SDPA_ERR_INVALID_ARG, "window_right %d widens the causal band and needs causal = 1", d->window_right);
  if (!(d->scale > 0.f) || !std::isfinite(d->scale))
    return fail(SDPA_ERR_INVALID_ARG, "scale %g must be finite and > 0", (double)d->scale);
  if (d->deterministic < 0 || d->deterministic > 2)
    return fail(SDPA_ERR_INVALID_ARG, "deterministic %d is not 0/1/2", d->deterministic);
  if (d->has_sink != 0 && d->has_sink != 1) return fail(SDPA_ERR_INVALID_ARG, "has_sink %d is not 0/1", d->has_sink);
  if (d->has_seq_lens != 0 && d->has_seq_lens != 1)
    return fail(SDPA_ERR_INVALID_ARG, "has_seq_lens %d is not 0/1", d->has_seq_lens);
  if (d->q_run_tiles < 0 || d->q_run_tiles > 16)
    return fail(SDPA_ERR_INVALID_ARG, "q_run_tiles %d is not in 0..16", d->q_run_tiles);
  if (d->layout == SDPA_LAYOUT_THD) {
    if (!d->has_seq_lens) return fail(SDPA_ERR_INVALID_ARG, "THD layout needs seq_lens_q / seq_lens_kv (has_seq_lens = 1)");
    if (d->total_q < 0 || d->total_kv < 0)
      return fail(SDPA_ERR_INVALID_ARG, "total_q %lld / total_kv %lld must be >= 0", (long long)d->total_q,
                  (long long)d->total_kv);
  } else if (d->bottom_right && d->seq_q > d->seq_kv && !d->has_seq_lens) {
    // Early rows would have a negative anchor and see no key at all.
    return fail(SDPA_ERR_UNSUPPORTED, "bottom-right mask with seq_q %d > seq_kv %d is not supported",
                d->seq_q, d->seq_kv);
  }
  sdpa_status st;
  if ((st = check_strides("q", d->stride_q, d))) return st;
  if ((st = check_strides("k", d->stride_k, d))) return st;
  if ((st = check_strides("v", d->stride_v, d))) return st;
  if ((st = check_strides("o", d->stride_o, d))) return st;
  if (backward) {
    if ((st = check_strides("do", d->stride_do, d))) return st;
    if ((st = check_strides("dq", d->stride_dq, d))) return st;
    if ((st = check_strides("dk", d->stride_dk, d))) return st;
    if ((st = check_strides("dv", d->stride_dv, d))) return st;
  }
  return SDPA_OK;
}

// The streaming kernel covers multi-head attention with a causal mask and a
// left window of at most 128 keys at head_dim 64 (its ring of q-tile slots
// is sized for that), without a right band.  It addresses rows with 32-bit
// row strides, and one (batch, head)'s fp32 dQ partial rows with 32-bit
// byte offsets.
bool stream_eligible(const sdpa_attn_desc* d) {
  bool small_rows = (int64_t)d->seq_q * d->head_dim * (int64_t)sizeof(float) <= INT32_MAX;
  for (const int64_t rs : {d->stride_q[2], d->stride_k[2], d->stride_v[2], d->stride_do[2], d->stride_dq[2],
                           d->stride_dk[2], d->stride_dv[2]})
    small_rows &= rs > 0 && rs <= INT32_MAX;
  return d->heads_q == d->heads_kv && d->causal && d->window_right == 0 && d->window_left >= 0 &&
         d->window_left <= 128 && d->head_dim == 64 && small_rows;
}

enum { ENGINE_STREAM_ATOMIC = 1, ENGINE_STREAM_RELAY = 2, ENGINE_TILE_QMAJOR = 3, ENGINE_TILE_RELAY = 4,
       ENGINE_QSTREAM = 5 };

// The q-major streaming kernel (bwd_qstream): head_dim 128, causal with no
// right band, left window 0..96, dense sequences without padding lengths
// whose diagonal offset is a multiple of 32; with a sink, groups of at most
// 64 query heads.
bool qstream_eligible(const sdpa_attn_desc* d) {
  bool small_rows = true;
  for (const int64_t rs : {d->stride_q[2], d->stride_k[2], d->stride_v[2], d->stride_o[2], d->stride_do[2],
                           d->stride_dq[2], d->stride_dk[2], d->stride_dv[2]})
    small_rows &= rs > 0 && rs <= INT32_MAX;
  const int64_t diag = d->bottom_right ? (int64_t)d->seq_kv - d->seq_q : 0;
  return d->layout == SDPA_LAYOUT_BHSD && !d->has_seq_lens && d->causal && d->window_right == 0 &&
         (!d->has_sink || d->heads_q / d->heads_kv <= 64) &&
         d->window_left >= 0 && d->window_left <= 96 && d->head_dim == 128 && diag >= 0 && diag % 32 == 0 &&
         d->seq_q > 0 && small_rows;
}

// The q-major forward (fwd_qstream): the same shapes, checked on the tensors
// the forward reads and writes, with query-head groups of a multiple of 8
// (each of the block's 8 waves owns whole heads) and a non-empty kv sequence.
bool fwd_qstream_eligible(const sdpa_attn_desc* d) {
  bool small_rows = true;
  for (const int64_t rs : {d->stride_q[2], d->stride_k[2], d->stride_v[2], d->stride_o[2]})
    small_rows &= rs > 0 && rs <= INT32_MAX;
  const int64_t diag = d->bottom_right ? (int64_t)d->seq_kv - d->seq_q : 0;
  const int G = d->heads_q / d->heads_kv;
  return d->layout == SDPA_LAYOUT_BHSD && !d->has_seq_lens && d->causal && d->window_right == 0 &&
         d->window_left >= 0 && d->window_left <= 96 && d->head_dim == 128 && diag >= 0 && diag % 32 == 0 &&
         d->seq_q > 0 && d->seq_kv > 0 && G % 8 == 0 && G / 8 <= 64 && small_rows;
}

// Chunks of a q-major kernel's grid: one 8-wave block per CU walks `c`
// consecutive 32-row q-steps of one (sequence, kv head), `per_step` steps of
// work each; with r rounds of 256 CUs the chunks are ceil(nqt / floor(256 r /
// bh)) q-steps long (at least min_len), and r minimizes the estimated makespan
// r (c per_step + startup) in steps (fewer rounds on a tie).
int64_t qstream_chunk(int64_t bh, int64_t nqt, int64_t per_step, int64_t startup, int64_t min_len) {
  const int64_t n_cap = std::max<int64_t>(1, nqt / min_len);
  int64_t best_c = nqt, best_cost = INT64_MAX;
  for (int64_t rounds = 1; rounds <= 64; ++rounds) {
    const int64_t n0 = std::min(std::max<int64_t>(256 * rounds / bh, 1), n_cap);
    const int64_t c = (nqt + n0 - 1) / n0, n = (nqt + c - 1) / c;
    const int64_t cost = ((bh * n + 255) / 256) * (c * per_step + startup);
    if (cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
    if (n0 == n_cap) break;
  }
  return best_c;
}

// The backward's kernels and dQ mechanism: a forced engine (validated
// against the shape and the deterministic promise) or the plan's default.
sdpa_status resolve_engine(const sdpa_attn_desc* d, int* engine) {
  const bool stream_ok = stream_eligible(d);
  if (d->engine < 0 || d->engine > 5) return fail(SDPA_ERR_INVALID_ARG, "engine %d is not 0..5", d->engine);
  if (d->engine) {
    if (d->engine == ENGINE_QSTREAM && !qstream_eligible(d))
      return fail(SDPA_ERR_UNSUPPORTED,
                  "engine 5 (q-major streaming kernel) needs head_dim 128, causal, window_right 0, window_left "
                  "0..96, dense sequences without seq_lens, seq_kv - seq_q a multiple of 32 (bottom-right), "
                  "at most 64 query heads per kv head with a sink, and row strides below 2^31");
    if ((d->engine == ENGINE_STREAM_ATOMIC || d->engine == ENGINE_STREAM_RELAY) && !stream_ok)
      return fail(SDPA_ERR_UNSUPPORTED,
                  "engine %d (streaming kernel) needs heads_q == heads_kv, causal, window_right 0, window_left "
                  "0..128, head_dim 64 and row strides below 2^31", d->engine);
    if (d->engine == ENGINE_STREAM_ATOMIC && d->deterministic)
      return fail(SDPA_ERR_INVALID_ARG, "engine 1 (fp32 atomics) is not repeatable: it needs deterministic 0");
    if (d->deterministic == 2 && d->engine != ENGINE_TILE_RELAY)
      return fail(SDPA_ERR_INVALID_ARG, "deterministic 2 asks for the per-kv-tile relay: engine must be 0 or 4");
    *engine = d->engine;
    return SDPA_OK;
  }
  // The measured table (MI355X, head_dim 64, causal, windows 64 / 128, both
  // anchors; batch x heads 2 .. 128, 1K .. 16K rows; the engine study of
  // this package): the streaming kernel, one block per CU, leaves the chip
  // idle below about 2^16 query rows (B Hq S_q) and there loses to the
  // per-tile kernels by 24-50%; above, it wins by 15-30%.  Its chunk relay
  // ties or beats its fp32 atomics everywhere (within 1.5% at the largest
  // shape) and is repeatable, so it serves both deterministic 0 and 1.
  //
  // Head_dim 128 (the study's d128 family: causal, windows 32 / 96, groups
  // of 8 and multi-head, 1 .. 72 (sequence, kv head) pairs, 1K .. 16K rows):
  // the q-major streaming kernel wins on every multi-head shape (by
  // 10-80%) and wherever the window is 64 keys or more (by 15-55%), also on
  // the smallest grids; with groups of 8 and a 32-key window it wins once
  // the grid holds at least 1024 q-steps (B Hkv S_q / 32), or 512 with a
  // sink (where the per-tile path also runs bwd_dot), and below that the
  // per-tile kernels lead by up to 16%.  Both are bitwise repeatable
  // (deterministic 0 and 1).
  const int64_t q_rows =
      (d->layout == SDPA_LAYOUT_THD ? d->total_q : (int64_t)d->batch * d->seq_q) * (int64_t)d->heads_q;
  const int64_t q_steps = (int64_t)d->batch * d->heads_kv * (((int64_t)d->seq_q + 31) / 32);
  if (d->deterministic == 2)
    *engine = ENGINE_TILE_RELAY;
  else if (qstream_eligible(d) &&
           (d->heads_q == d->heads_kv || d->window_left >= 64 || q_steps >= (d->has_sink ? 512 : 1024)))
    *engine = ENGINE_QSTREAM;
  else if (stream_ok && q_rows >= (int64_t(1) << 16))
    *engine = ENGINE_STREAM_RELAY;
  else
    *engine = ENGINE_TILE_QMAJOR;
  return SDPA_OK;
}

swa::Problem make_problem(const sdpa_attn_desc* d, int engine) {
  swa::Problem p{};
  p.B = d->batch;
  p.Hq = d->heads_q;
  p.Hkv = d->heads_kv;
  p.G = d->heads_q / d->heads_kv;
  p.D = d->head_dim;
  p.seq_q = d->seq_q;
  p.seq_kv = d->seq_kv;
  p.layout = d->layout;
  p.total_q = d->layout == SDPA_LAYOUT_THD ? d->total_q : (int64_t)d->batch * d->seq_q;
  p.total_kv = d->layout == SDPA_LAYOUT_THD ? d->total_kv : (int64_t)d->batch * d->seq_kv;
  p.causal = d->causal;
  p.bottom_right = d->bottom_right;
  // A band wider than both sequences together masks nothing more; clamping
  // keeps the schedule's integer arithmetic far from overflow.
  p.window = clamp_band(d->window_left, d->seq_q, d->seq_kv);
  p.right = d->causal ? clamp_band(d->window_right, d->seq_q, d->seq_kv) : 0;
  p.scale = d->scale;
  p.scale_log2 = d->scale * swa::kLog2e;
  p.has_sink = d->has_sink;
  for (int k = 0; k < 3; ++k) {
    p.sq[k] = d->stride_q[k];
    p.sk[k] = d->stride_k[k];
    p.sv[k] = d->stride_v[k];
    p.so[k] = d->stride_o[k];
    p.sdo[k] = d->stride_do[k];
    p.sdq[k] = d->stride_dq[k];
    p.sdk[k] = d->stride_dk[k];
    p.sdv[k] = d->stride_dv[k];
  }
  p.n_q_tiles = (d->seq_q + kTile - 1) / kTile;
  p.n_kv_tiles = (d->seq_kv + kTile - 1) / kTile;
  // Engines: the streaming kernel (boundary q-tiles of its chunks through
  // fp32 atomics or the chunk relay), or the per-tile kernel with dQ from
  // the q-major pass (no fp32 accumulator: each dQ row is summed inside one
  // block in a fixed order, so this is bitwise repeatable) or from the
  // per-kv-tile relay of the pages.
  p.stream = engine == ENGINE_STREAM_ATOMIC || engine == ENGINE_STREAM_RELAY;
  p.stream_relay = engine == ENGINE_STREAM_RELAY;
  p.step_kv = p.stream ? 128 : kTile;
  p.split_dq = engine == ENGINE_TILE_QMAJOR;
  // Consecutive q-tiles one block of the q-major passes walks.  A run
  // pays the block's start-up latency once, but needs registers for the
  // next q-tile's rows; a measured study over head_dim and band width on
  // MI355X (bwd_dq and the forward, runs of 1 / 2 / 4 / 8, GQA and the
  // workloads of the pages) picked these classes:
  //   head_dim 128, band <= 256 keys: runs of 8 (both passes);
  //   head_dim 64, band <= 64 keys: runs of 4 for the forward;
  //   otherwise one q-tile per block (at head_dim 64 that keeps four blocks
  //   per CU).
  {
    const int64_t band = (d->window_left >= 0 ? (int64_t)d->window_left : (int64_t)d->seq_kv + d->seq_q) +
                         (d->causal ? (int64_t)d->window_right : (int64_t)d->seq_kv + d->seq_q);
    p.dq_tiles = d->head_dim == 128 && band <= 256 ? 8 : 1;
    p.fwd_tiles = d->head_dim == 128 && band <= 256 ? 8 : (band <= 64 ? 4 : 1);
    if (d->q_run_tiles > 0) p.dq_tiles = p.fwd_tiles = d->q_run_tiles;
  }
  // Where the dQ pass walks runs of q-tiles (short windows, whose passes
  // stream Q / dO / O at full size), at head_dim 128 (where its run and
  // single-tile kernels both hold two blocks per CU), or where its grid fits
  // one round at two blocks per CU (at most 512 blocks), it also forms
  // delta from the dO rows it holds, replacing the bwd_dot pass and its
  // second read of dO and one launch (on MI355X: the f16 head_dim-128 GQA
  // workload at S = 128, 71.4 -> 67.4 us per step; the 256-row two-head
  // workload, 19.9 -> 16.9 us); the per-q-tile dSink partials stay with
  // bwd_dot.
  const int64_t dq_blocks = (int64_t)p.n_q_tiles * d->heads_q * d->batch;
  p.dq_delta = p.split_dq && (p.dq_tiles > 1 || d->head_dim == 128 || dq_blocks <= 512) && !d->has_sink;
  p.stream_delta = p.stream && !d->has_sink;
  // bwd_clear: q-tiles per block such that its grid has about 512 blocks
  // (with fp32 atomics its blocks zero 16 KB slots, and a grid of a few
  // dozen blocks left most CUs idle: 8.5 us at c2's 4096 rows)
  {
    const int64_t tiles = (int64_t)p.n_q_tiles * d->heads_q * d->batch;
    p.clear_tiles = (int)std::min<int64_t>(64, std::max<int64_t>(1, tiles / 512));
  }
  p.qstream = engine == ENGINE_QSTREAM;
  if (p.qstream) {
    // One 8-wave block per CU walks a chunk of consecutive 32-row q-steps of
    // one (sequence, kv head), one step per query head of the group.  With
    // r rounds of 256 CUs the chunks are ceil(nqt / floor(256 r / bh))
    // q-steps long; pick r to minimize the estimated makespan r (C G + 6)
    // in steps (6: a chunk's start-up and its boundary tiles, as measured on
    // MI355X for G = 8 between chunks of 4 and 19 q-steps), chunks of at
    // least 3 q-steps (so a 32-key tile, seen by at most 4 q-steps, is
    // shared by at most two chunks); fewer rounds on a tie.
    const int64_t bh = (int64_t)d->batch * d->heads_kv, nqt = ((int64_t)d->seq_q + 31) / 32;
    const int64_t best_c = qstream_chunk(bh, nqt, p.G, 6, 3);
    p.qs_chunk = (int)best_c;
    p.qs_nch = (int)((nqt + best_c - 1) / best_c);
  }
  p.sink_tiles = p.qstream ? (d->seq_q + 31) / 32 : p.n_q_tiles;
  if (p.stream) {
    // One block per CU: chunks of kv-steps sized so the grid is about one
    // block per MI355X CU, never shorter than 2 steps (so a q-tile has at
    // most two visiting chunks).
    const int64_t steps_per_seq = (d->seq_kv + p.step_kv - 1) / p.step_kv;
    const int64_t total = steps_per_seq * d->batch * d->heads_q;
    int64_t chunk = (total + 255) / 256;
    if (chunk < 2) chunk = 2;
    p.chunk = (int)chunk;
    p.n_chunks = (int)((steps_per_seq + chunk - 1) / chunk);
  } else {
    p.chunk = 1;
    p.n_chunks = 0;
  }
  return p;
}

// Pointer must be device (or managed) memory of the current device.
sdpa_status check_dev_ptr(const void* ptr, const char* name, bool may_be_null, size_t align) {
  if (!ptr) return may_be_null ? SDPA_OK : fail(SDPA_ERR_INVALID_ARG, "tensor %s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % align)
    return fail(SDPA_ERR_INVALID_ARG, "tensor %s at %p is not %zu-byte aligned", name, ptr, align);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SDPA_ERR_HIP, "hipGetDevice failed");
  hipPointerAttribute_t at;
  std::memset(&at, 0, sizeof at);
  hipError_t e = hipPointerGetAttributes(&at, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(SDPA_ERR_INVALID_ARG, "tensor %s at %p is not device memory (expected device %d)", name, ptr, dev);
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
    return fail(SDPA_ERR_INVALID_ARG, "tensor %s at %p is host memory, expected device %d", name, ptr, dev);
  if (at.device != dev)
    return fail(SDPA_ERR_INVALID_ARG, "tensor %s is on device %d, expected device %d", name, at.device, dev);
  return SDPA_OK;
}

}  // namespace

extern "C" {

const char* sdpa_status_string(sdpa_status s) {
  switch (s) {
    case SDPA_OK: return "SDPA_OK";
    case SDPA_ERR_INVALID_ARG: return "SDPA_ERR_INVALID_ARG";
    case SDPA_ERR_UNSUPPORTED: return "SDPA_ERR_UNSUPPORTED";
    case SDPA_ERR_WORKSPACE: return "SDPA_ERR_WORKSPACE";
    case SDPA_ERR_HIP: return "SDPA_ERR_HIP";
    case SDPA_ERR_RELAY_TIMEOUT: return "SDPA_ERR_RELAY_TIMEOUT";
  }
  return "SDPA_ERR_UNKNOWN";
}

const char* sdpa_last_error(void) { return g_err; }

sdpa_status sdpa_bwd_plan(const sdpa_attn_desc* desc, sdpa_bwd_plan_t** plan, size_t* workspace_bytes) {
  if (!plan || !workspace_bytes) return fail(SDPA_ERR_INVALID_ARG, "plan / workspace_bytes out-pointer is NULL");
  *plan = nullptr;
  sdpa_status st = check_desc(desc, true);
  if (st) return st;
  int engine = 0;
  if ((st = resolve_engine(desc, &engine))) return st;
  auto* pl = new (std::nothrow) struct sdpa_bwd_plan();
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "out of host memory");
  pl->desc = *desc;
  pl->prob = make_problem(desc, engine);
  const swa::Problem& p = pl->prob;
  pl->stat_rows = (int64_t)p.Hq * p.total_q;
  size_t off = 0;
  pl->off_delta = off;
  if (!p.qstream) off = align256(off + sizeof(float) * (size_t)pl->stat_rows);  // (bwd_qstream keeps delta in LDS)
  pl->off_acc = off;
  if (p.qstream) {
    // the fp32 dK / dV partials of the 32-key tiles neighbouring chunks
    // share: per (sequence, kv head, chunk boundary) 3 tiles x 2 sides
    off = align256(off + sizeof(float) * (size_t)p.B * p.Hkv * p.qs_nch * 6 * 32 * 2 * p.D);
  } else if (!p.split_dq) {
    size_t acc_floats = (size_t)pl->stat_rows * p.D;
    // the streaming kernel's unordered mode keeps each q-tile's partial sum
    // in a 64-row slot of its own (stream_slot: dense B x Hq x n_q_tiles
    // slots, packed Hq x (total_q / 64 + B + 1))
    if (p.stream && !p.stream_relay) {
      const size_t slots = p.layout == swa::LAYOUT_THD
                               ? (size_t)p.Hq * (size_t)((p.total_q >> 6) + p.B + 1)
                               : (size_t)p.B * p.Hq * p.n_q_tiles;
      acc_floats = std::max(acc_floats, slots * swa::kTile * p.D);
    }
    off = align256(off + sizeof(float) * acc_floats);
  }
  pl->off_stash = off;
  if (p.stream && p.stream_relay) off = align256(off + sizeof(float) * (size_t)pl->stat_rows * p.D);
  pl->off_sem = off;
  off = align256(off + sizeof(int) * (size_t)p.B * p.Hq * p.n_q_tiles);
  pl->off_ctl = off;
  off = align256(off + sizeof(int) * 4);
  pl->off_sink = off;
  off = align256(off + sizeof(float) * (size_t)p.Hq * p.B * p.sink_tiles);
  pl->ws_bytes = off;
  pl->spin_limit = 1 << 20;  // ~55 ms of s_sleep per wait; legitimate waits take microseconds
  pl->relay_bias = 0;
  *plan = pl;
  *workspace_bytes = off;
  g_err[0] = 0;
  return SDPA_OK;
}

void sdpa_bwd_plan_destroy(sdpa_bwd_plan_t* plan) { delete plan; }

}  // extern "C"

namespace swa {

size_t bwd_plan_workspace_bytes(const sdpa_bwd_plan_t* pl) { return pl->ws_bytes; }

// The backward's launch sequence behind sdpa_bwd_run_events and the
// no-allocation entry point: validates the plan, the workspace size and
// alignment and the tensors, then enqueues the kernels.  check_ws_ptr asks
// the runtime whether the workspace is device memory of the current device
// (the library's own scratch array is known to be).
sdpa_status bwd_run(const sdpa_bwd_plan_t* pl, const sdpa_bwd_tensors* t, void* ws, size_t ws_bytes,
                    hipStream_t stream, hipEvent_t main_start, hipEvent_t main_stop, bool check_ws_ptr) {
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "plan is NULL");
  if (!t) return fail(SDPA_ERR_INVALID_ARG, "tensors is NULL");
  const sdpa_attn_desc& d = pl->desc;
  if (ws_bytes < pl->ws_bytes)
    return fail(SDPA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the planned %zu", ws_bytes, pl->ws_bytes);
  if (!ws && pl->ws_bytes) return fail(SDPA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(SDPA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  sdpa_status st;
  if (check_ws_ptr && (st = check_dev_ptr(ws, "workspace", false, 256)))
    return st == SDPA_ERR_INVALID_ARG ? SDPA_ERR_WORKSPACE : st;
  if ((st = check_dev_ptr(t->q, "q", false, 16))) return st;
  if ((st = check_dev_ptr(t->k, "k", false, 16))) return st;
  if ((st = check_dev_ptr(t->v, "v", false, 16))) return st;
  if ((st = check_dev_ptr(t->o, "o", false, 16))) return st;
  if ((st = check_dev_ptr(t->dO, "dO", false, 16))) return st;
  if ((st = check_dev_ptr(t->lse, "lse", false, 4))) return st;
  if ((st = check_dev_ptr(t->dq, "dq", false, 16))) return st;
  if ((st = check_dev_ptr(t->dk, "dk", false, 16))) return st;
  if ((st = check_dev_ptr(t->dv, "dv", false, 16))) return st;
  if (d.has_sink) {
    if ((st = check_dev_ptr(t->sink, "sink", false, 4))) return st;
    if ((st = check_dev_ptr(t->dsink, "dsink", false, 4))) return st;
  } else if (t->sink || t->dsink) {
    return fail(SDPA_ERR_INVALID_ARG, "sink / dsink given but the plan has has_sink = 0");
  }
  if (d.layout == SDPA_LAYOUT_THD) {
    if ((st = check_dev_ptr(t->cu_seqlens_q, "cu_seqlens_q", false, 4))) return st;
    if ((st = check_dev_ptr(t->cu_seqlens_kv, "cu_seqlens_kv", false, 4))) return st;
  }
  if (d.has_seq_lens) {
    if ((st = check_dev_ptr(t->seq_lens_q, "seq_lens_q", false, 4))) return st;
    if ((st = check_dev_ptr(t->seq_lens_kv, "seq_lens_kv", false, 4))) return st;
  }

  swa::BwdArgs a{};
  a.p = pl->prob;
  a.p.cu_q = d.layout == SDPA_LAYOUT_THD ? t->cu_seqlens_q : nullptr;
  a.p.cu_kv = d.layout == SDPA_LAYOUT_THD ? t->cu_seqlens_kv : nullptr;
  a.p.len_q = d.has_seq_lens ? t->seq_lens_q : nullptr;
  a.p.len_kv = d.has_seq_lens ? t->seq_lens_kv : nullptr;
  a.dtype = d.dtype;
  a.q = t->q;
  a.k = t->k;
  a.v = t->v;
  a.o = t->o;
  a.dO = t->dO;
  a.lse = t->lse;
  a.sink = t->sink;
  a.dq = t->dq;
  a.dk = t->dk;
  a.dv = t->dv;
  a.dsink = t->dsink;
  char* base = static_cast<char*>(ws);
  a.delta = reinterpret_cast<float*>(base + pl->off_delta);
  a.dq_acc = reinterpret_cast<float*>(base + pl->off_acc);
  a.dq_stash = reinterpret_cast<float*>(base + pl->off_stash);
  a.sem = reinterpret_cast<int*>(base + pl->off_sem);
  a.ctl = reinterpret_cast<int*>(base + pl->off_ctl);
  a.sink_part = reinterpret_cast<float*>(base + pl->off_sink);
  a.deterministic = d.deterministic;
  a.spin_limit = pl->spin_limit;
  a.relay_bias = pl->relay_bias;

  hipError_t e;
  // dq_delta: the dQ pass forms delta, so it runs first and bwd_dot not at
  // all; stream_delta: the streaming kernel forms delta, and bwd_clear does
  // the clearing bwd_dot would have done
  if (!a.p.dq_delta && !a.p.stream_delta && !a.p.qstream && (e = swa::launch_bwd_dot(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_dot launch: %s", hipGetErrorString(e));
  if (a.p.stream_delta && (e = swa::launch_bwd_clear(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_clear launch: %s", hipGetErrorString(e));
  if (a.p.dq_delta && (e = swa::launch_bwd_dq(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_dq launch: %s", hipGetErrorString(e));
  if (main_start && (e = hipEventRecord(main_start, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  if ((e = swa::launch_bwd_main(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_main launch: %s", hipGetErrorString(e));
  if (main_stop && (e = hipEventRecord(main_stop, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  if (a.p.split_dq && !a.p.dq_delta && (e = swa::launch_bwd_dq(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_dq launch: %s", hipGetErrorString(e));
  if (d.has_sink && (e = swa::launch_bwd_dsink(a, stream)) != hipSuccess)
    return fail(SDPA_ERR_HIP, "bwd_dsink launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return SDPA_OK;
}

sdpa_status set_error(sdpa_status st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace swa

extern "C" {

sdpa_status sdpa_bwd_run_events(const sdpa_bwd_plan_t* pl, const sdpa_bwd_tensors* t, void* ws,
                                size_t ws_bytes, hipStream_t stream, hipEvent_t main_start,
                                hipEvent_t main_stop) {
  return swa::bwd_run(pl, t, ws, ws_bytes, stream, main_start, main_stop, true);
}

sdpa_status sdpa_bwd_run(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* tensors, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return swa::bwd_run(plan, tensors, workspace, workspace_bytes, stream, nullptr, nullptr, true);
}

sdpa_status sdpa_bwd_schedule(const sdpa_bwd_plan_t* pl, int32_t len_q, int32_t len_kv, int32_t* tile_q,
                              int32_t* tile_kv, int32_t* n_q, int32_t* n_kv, int32_t kv_cap, int32_t* q_lo,
                              int32_t* q_hi, int32_t q_cap, int32_t* kv_first, int32_t* kv_last) {
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "plan is NULL");
  if (len_q < 0 || len_kv < 0) return fail(SDPA_ERR_INVALID_ARG, "len_q %d / len_kv %d must be >= 0", len_q, len_kv);
  // The streaming kernel evaluates its schedule in the shift form of
  // StreamSched with the plan's window; the per-tile kernels use SeqSched,
  // and so does the q-major streaming kernel, on 32-row q-steps and 32-key
  // tiles.  Reporting what each kernel itself computes lets host tests check
  // the form that runs.
  const int tq = pl->prob.qstream ? 32 : kTile, tkv = pl->prob.qstream ? 32 : pl->prob.step_kv;
  swa::SeqSched g;
  g.init(len_q, len_kv, pl->desc.bottom_right, pl->desc.causal, clamp_band(pl->desc.window_left, len_q, len_kv),
         clamp_band(pl->desc.window_right, len_q, len_kv), tq, tkv);
  swa::StreamSched gs;
  gs.init(len_q, len_kv, pl->desc.bottom_right, pl->prob.window);
  const bool stream = pl->prob.stream;
  const int nq = stream ? gs.n_q_tiles : g.n_q_tiles, nk = stream ? gs.n_kv_tiles : g.n_kv_tiles;
  if (tile_q) *tile_q = tq;
  if (tile_kv) *tile_kv = tkv;
  if (n_q) *n_q = nq;
  if (n_kv) *n_kv = nk;
  if ((q_lo || q_hi) && kv_cap < nk) return fail(SDPA_ERR_INVALID_ARG, "kv_cap %d < %d kv-tiles", kv_cap, nk);
  if ((kv_first || kv_last) && q_cap < nq) return fail(SDPA_ERR_INVALID_ARG, "q_cap %d < %d q-tiles", q_cap, nq);
  for (int j = 0; j < nk; ++j) {
    if (q_lo) q_lo[j] = stream ? gs.q_lo(j) : g.q_lo(j);
    if (q_hi) q_hi[j] = stream ? gs.q_hi(j) : g.q_hi(j);
  }
  for (int i = 0; i < nq; ++i) {
    if (kv_first) kv_first[i] = stream ? gs.kv_first(i) : g.kv_first(i);
    if (kv_last) kv_last[i] = stream ? gs.kv_last(i) : g.kv_last(i);
  }
  g_err[0] = 0;
  return SDPA_OK;
}

sdpa_status sdpa_bwd_relay_expiries(const sdpa_bwd_plan_t* pl, const void* ws, hipStream_t stream,
                                    int32_t* count) {
  if (!pl || !ws || !count) return fail(SDPA_ERR_INVALID_ARG, "plan / workspace / count is NULL");
  const char* base = static_cast<const char*>(ws);
  hipError_t e = hipMemcpyAsync(count, base + pl->off_ctl + sizeof(int), sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "reading the relay watchdog counter: %s", hipGetErrorString(e));
  if (*count > 0)
    return fail(SDPA_ERR_RELAY_TIMEOUT,
                "%d ordered-relay wait(s) of the last run gave up after %d spins: that run's dQ is invalid "
                "(the turns that gave up added NaN)", *count, pl->spin_limit);
  g_err[0] = 0;
  return SDPA_OK;
}

sdpa_status sdpa_bwd_plan_set_relay_watchdog(sdpa_bwd_plan_t* pl, int32_t spin_limit, int32_t unreachable) {
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "plan is NULL");
  if (spin_limit < 0) return fail(SDPA_ERR_INVALID_ARG, "spin_limit %d < 0", spin_limit);
  if (unreachable != 0 && unreachable != 1) return fail(SDPA_ERR_INVALID_ARG, "unreachable %d is not 0/1", unreachable);
  pl->spin_limit = spin_limit > 0 ? spin_limit : (1 << 20);
  // counters only ever hold turns below a q-tile's visitor count (<= 2^31 / 64)
  pl->relay_bias = unreachable ? (1 << 30) : 0;
  g_err[0] = 0;
  return SDPA_OK;
}

sdpa_status sdpa_fwd_plan(const sdpa_attn_desc* desc, sdpa_fwd_plan_t** plan, size_t* workspace_bytes) {
  if (!plan || !workspace_bytes) return fail(SDPA_ERR_INVALID_ARG, "plan / workspace_bytes out-pointer is NULL");
  *plan = nullptr;
  sdpa_status st = check_desc(desc, false);
  if (st) return st;
  // The forward's kernel: the q-major forward where it applies (engine 0 or
  // 5; 5 fails elsewhere), else the per-tile forward (any other engine).
  if (desc->engine < 0 || desc->engine > 5) return fail(SDPA_ERR_INVALID_ARG, "engine %d is not 0..5", desc->engine);
  const bool qs_ok = fwd_qstream_eligible(desc);
  if (desc->engine == ENGINE_QSTREAM && !qs_ok)
    return fail(SDPA_ERR_UNSUPPORTED,
                "engine 5 (q-major forward) needs head_dim 128, causal, window_right 0, window_left 0..96, "
                "dense sequences without seq_lens, seq_kv - seq_q a multiple of 32 (bottom-right), seq_kv > 0, "
                "heads_q / heads_kv a multiple of 8 (at most 512) and row strides below 2^31");
  auto* pl = new (std::nothrow) struct sdpa_fwd_plan();
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "out of host memory");
  pl->desc = *desc;
  pl->prob = make_problem(desc, ENGINE_TILE_QMAJOR);  // (the backward's engine does not apply)
  if (qs_ok && (desc->engine == 0 || desc->engine == ENGINE_QSTREAM)) {
    // One 8-wave block per CU walks a chunk of q-steps of one (sequence, kv
    // head), G / 8 (q-step, head) steps per q-step; a chunk's start-up (its
    // ring's first tiles and rows) costs about two steps.
    const int64_t bh = (int64_t)desc->batch * desc->heads_kv, nqt = ((int64_t)desc->seq_q + 31) / 32;
    const int64_t c = qstream_chunk(bh, nqt, pl->prob.G / 8, 2, 1);
    pl->prob.qstream = 1;
    pl->prob.qs_chunk = (int)c;
    pl->prob.qs_nch = (int)((nqt + c - 1) / c);
  }
  *plan = pl;
  *workspace_bytes = 0;
  g_err[0] = 0;
  return SDPA_OK;
}

void sdpa_fwd_plan_destroy(sdpa_fwd_plan_t* plan) { delete plan; }

sdpa_status sdpa_fwd_run(const sdpa_fwd_plan_t* pl, const sdpa_fwd_tensors* t, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (!pl) return fail(SDPA_ERR_INVALID_ARG, "plan is NULL");
  if (!t) return fail(SDPA_ERR_INVALID_ARG, "tensors is NULL");
  const sdpa_attn_desc& d = pl->desc;
  sdpa_status st;
  if ((st = check_dev_ptr(t->q, "q", false, 16))) return st;
  if ((st = check_dev_ptr(t->k, "k", false, 16))) return st;
  if ((st = check_dev_ptr(t->v, "v", false, 16))) return st;
  if ((st = check_dev_ptr(t->o, "o", false, 16))) return st;
  if ((st = check_dev_ptr(t->lse, "lse", false, 4))) return st;
  if (d.has_sink) {
    if ((st = check_dev_ptr(t->sink, "sink", false, 4))) return st;
  } else if (t->sink) {
    return fail(SDPA_ERR_INVALID_ARG, "sink given but the plan has has_sink = 0");
  }
  if (d.layout == SDPA_LAYOUT_THD) {
    if ((st = check_dev_ptr(t->cu_seqlens_q, "cu_seqlens_q", false, 4))) return st;
    if ((st = check_dev_ptr(t->cu_seqlens_kv, "cu_seqlens_kv", false, 4))) return st;
  }
  if (d.has_seq_lens) {
    if ((st = check_dev_ptr(t->seq_lens_q, "seq_lens_q", false, 4))) return st;
    if ((st = check_dev_ptr(t->seq_lens_kv, "seq_lens_kv", false, 4))) return st;
  }
  swa::FwdArgs a{};
  a.p = pl->prob;
  a.p.cu_q = d.layout == SDPA_LAYOUT_THD ? t->cu_seqlens_q : nullptr;
  a.p.cu_kv = d.layout == SDPA_LAYOUT_THD ? t->cu_seqlens_kv : nullptr;
  a.p.len_q = d.has_seq_lens ? t->seq_lens_q : nullptr;
  a.p.len_kv = d.has_seq_lens ? t->seq_lens_kv : nullptr;
  a.dtype = d.dtype;
  a.q = t->q;
  a.k = t->k;
  a.v = t->v;
  a.sink = t->sink;
  a.o = t->o;
  a.lse = t->lse;
  hipError_t e = swa::launch_fwd(a, stream);
  if (e != hipSuccess) return fail(SDPA_ERR_HIP, "fwd launch: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return SDPA_OK;
}

}  // extern "C"
