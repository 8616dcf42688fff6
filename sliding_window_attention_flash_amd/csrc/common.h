// Shared device-side definitions of the swa_sdpa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_sched.h"

namespace swa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kTile = 64;      // rows of a q-tile and of a kv-tile
constexpr int kThreads = 256;  // 4 waves of 64 lanes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum { LAYOUT_BHSD = 0, LAYOUT_THD = 1 };

// Everything a kernel needs to address one problem.  Strides are in
// elements, (batch, head, row); the head_dim axis is contiguous.
struct Problem {
  int B, Hq, Hkv, G, D;
  int seq_q, seq_kv;          // dense lengths, or max slot capacity (THD)
  int layout;
  int64_t total_q, total_kv;  // packed rows (THD)
  int causal, bottom_right, window;
  int right;                  // causal only: inclusive right band (0: plain causal)
  float scale;                // softmax scale
  float scale_log2;           // scale * log2(e)
  int has_sink;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* len_q;
  const int32_t* len_kv;
  int64_t sq[3], sk[3], sv[3], so[3], sdo[3], sdq[3], sdk[3], sdv[3];
  int n_q_tiles;              // ceil(seq_q / kTile)
  int n_kv_tiles;             // ceil(seq_kv / kTile)
  // streaming main kernel (see bwd_stream): kv-step width, kv-steps per
  // chunk and chunks per sequence; stream == 0 selects the per-tile kernel
  int split_dq;  // general path, unordered mode: dQ by its own q-major pass
  int dq_tiles;  // consecutive q-tiles one block of that pass walks
  int dq_delta;  // that pass forms delta and runs before bwd_main (no bwd_dot)
  int fwd_tiles; // the same for the forward
  int stream;
  int stream_relay;  // streaming kernel: boundary q-tiles by the chunk relay (else fp32 atomics)
  int stream_delta;  // streaming kernel forms delta as it stages q-tiles (no bwd_dot; no sink)
  int clear_tiles;   // q-tiles per block of bwd_clear (1 .. 64)
  int sink_tiles;    // dSink partials per (query head, sequence): 64-row q-tiles, or 32-row q-steps (bwd_qstream)
  int step_kv;
  int chunk;
  int n_chunks;
  // q-major streaming kernel (see bwd_qstream): q-tiles per chunk and
  // chunks per (sequence, kv head)
  int qstream;
  int qs_chunk;
  int qs_nch;
};

// One sequence (or dense batch entry): valid lengths, slot capacities,
// first packed row and where its row statistics start.
struct Seq {
  int len_q, len_kv, cap_q, cap_kv;
  int64_t row0_q, row0_kv;  // first packed row (THD), 0 for BHSD
  int64_t stat0;            // stat index of (head 0, row 0)
  int64_t stat_hs;          // stat index stride between heads
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Reads sequence b's geometry.  Device metadata is clamped so that a bad
// cu_seqlens / seq_lens entry can never address outside the buffers.
__device__ __forceinline__ Seq load_seq(const Problem& p, int b) {
  Seq s;
  if (p.layout == LAYOUT_THD) {
    int64_t q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    int64_t k0 = p.cu_kv[b], k1 = p.cu_kv[b + 1];
    q0 = q0 < 0 ? 0 : (q0 > p.total_q ? p.total_q : q0);
    q1 = q1 < q0 ? q0 : (q1 > p.total_q ? p.total_q : q1);
    k0 = k0 < 0 ? 0 : (k0 > p.total_kv ? p.total_kv : k0);
    k1 = k1 < k0 ? k0 : (k1 > p.total_kv ? p.total_kv : k1);
    s.row0_q = q0;
    s.row0_kv = k0;
    s.cap_q = (int)(q1 - q0 < p.seq_q ? q1 - q0 : p.seq_q);
    s.cap_kv = (int)(k1 - k0 < p.seq_kv ? k1 - k0 : p.seq_kv);
    s.stat0 = q0;
    s.stat_hs = p.total_q;
  } else {
    s.row0_q = s.row0_kv = 0;
    s.cap_q = p.seq_q;
    s.cap_kv = p.seq_kv;
    s.stat0 = (int64_t)b * p.Hq * p.seq_q;
    s.stat_hs = p.seq_q;
  }
  s.len_q = p.len_q ? clampi(p.len_q[b], 0, s.cap_q) : s.cap_q;
  s.len_kv = p.len_kv ? clampi(p.len_kv[b], 0, s.cap_kv) : s.cap_kv;
  return s;
}

// Element offset of (b, h, row) in a tensor with strides st.
__device__ __forceinline__ int64_t elem_off(const Problem& p, const int64_t* st, int b,
                                            int64_t row0, int h, int row) {
  if (p.layout == LAYOUT_THD) return (row0 + row) * st[2] + (int64_t)h * st[1];
  return (int64_t)b * st[0] + (int64_t)h * st[1] + (int64_t)row * st[2];
}

// Mask of the pages: anchor a = row (+ diag for bottom-right); key visible
// when inside both valid lengths, key <= a + R if causal (R: right band,
// 0 for plain causal), a - key <= W if W >= 0.
__device__ __forceinline__ bool visible(const SeqSched& g, int row, int key) {
  const int a = row + g.diag;
  bool v = (row < g.len_q) & (key < g.len_kv);
  if (g.causal) v &= key <= a + g.right;
  if (g.window >= 0) v &= (a - key) <= g.window;
  return v;
}

// Storage type traits: 16-bit element <-> float.
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ __bf16 from_float(float x) { return (__bf16)x; }
  static __device__ __forceinline__ float to_float(__bf16 x) { return (float)x; }
};
template <>
struct Elem<_Float16> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ _Float16 from_float(float x) { return (_Float16)x; }
  static __device__ __forceinline__ float to_float(_Float16 x) { return (float)x; }
};

// MFMA 16x16x32 (fp32 accumulate) on 8-element 16-bit operands.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The schedule the main kernel runs: kv-tiles of kTile keys (per-tile
// kernel) or kv-steps of step_kv keys (streaming kernel); q-tiles of kTile.
__device__ __forceinline__ void main_sched(const Problem& p, const Seq& s, SeqSched& g) {
  g.init(s.len_q, s.len_kv, p.bottom_right, p.causal, p.window, p.right, kTile,
         p.stream ? p.step_kv : kTile);
}

// Streaming kernel, unordered mode: index of the 64-row fp32 partial-sum
// slot of q-tile i of (sequence b, head h).  Dense: b, h, i row-major over
// n_q_tiles per (b, h).  Packed (THD): per head, sequence b's slots start at
// floor(q0 / 64) + b, where q0 is its first packed row; consecutive
// sequences never overlap (floor(x) - floor(y) + 1 >= ceil(x - y)), and a
// head needs at most total_q / 64 + B + 1 slots.
__device__ __forceinline__ int64_t stream_slot(const Problem& p, const Seq& s, int b, int h, int i) {
  if (p.layout == LAYOUT_THD) return (int64_t)h * ((p.total_q >> 6) + p.B + 1) + (s.row0_q >> 6) + b + i;
  return ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
}

// Streaming kernel: number of chunks (blocks) that visit q-tile i.  A q-tile
// with more than one visiting chunk is a boundary tile whose dQ goes through
// the fp32 accumulator (relay or atomics); the others are written directly.
__device__ __forceinline__ int chunk_visitors(const Problem& p, const SeqSched& g, int i) {
  if (g.n_visitors(i) == 0) return 0;
  return g.kv_last(i) / p.chunk - g.kv_first(i) / p.chunk + 1;
}

}  // namespace swa
