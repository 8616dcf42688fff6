// Backward kernels of the sliding-window attention (gfx950).
//
//   bwd_dot   delta_i = <dO_i, O_i>, per-q-tile dSink partials, clearing of
//             the relay counters, of the dQ accumulator and of unvisited
//             dQ rows
//   bwd_main  kv-tile-stationary backward with the window-bounded q-loop
//             (dK, dV; dQ too in relay mode, deterministic = 2)
//   bwd_dq    q-tile-stationary dQ pass (per-tile path, modes 0 and 1)
//   bwd_dsink fixed-order dSink reduction
//
// Method sources (web pages): cudnn-frontend PR #866 "frost(sdpa): bound the
// SM80 backward q-loop by the sliding window ... + window-aware deterministic
// relay" (commit message, Change) for the q-loop bounds, the zero store and
// the relay turn; cudnn-frontend PR #557 "frost(sdpa): GQA/MQA, padding mask,
// right-band widening, and sink-token gradients for the SM120 f16 backward"
// (Summary, review comments) for the dot / main / reduce split, GQA,
// per-sequence lengths and dSink.  The kernel design itself is written for
// CDNA4 and is not taken from those pages.
#include <type_traits>

#include "kernels.h"
#include "tiles.h"

namespace swa {

// ---- ordered dQ relay ------------------------------------------------------
// One q-tile's fp32 partial is touched only through agent-scope atomics: the
// first visitor exchanges its partial in, middle visitors add, the last
// visitor's fetch-add returns the sum of all earlier turns, to which it adds
// its own and writes the 16-bit result.  A single visitor writes directly.

// Spins until the q-tile's counter reaches `turn` (plus the test bias).  A
// wait that exceeds the spin limit gives up so that the device never hangs:
// it counts an expiry (reported by sdpa_bwd_relay_expiries) and returns
// true, and the caller then adds NaN instead of its partial, so the q-tile's
// dQ comes out poisoned rather than plausible but out of order.
__device__ __forceinline__ bool relay_wait(int* semp, int turn, int spin_limit, int* expiries) {
  int spins = 0;
  while (__hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != turn) {
    if (++spins > spin_limit) {
      atomicAdd(expiries, 1);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

template <typename T>
__device__ __forceinline__ void relay_add(float* ap, float val, int turn, int nv, float scale, T* out) {
  if (nv == 1) {
    *out = Elem<T>::from_float(scale * val);
  } else if (turn == 0) {
    __hip_atomic_exchange(ap, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (turn < nv - 1) {
    __hip_atomic_fetch_add(ap, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const float old = __hip_atomic_fetch_add(ap, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *out = Elem<T>::from_float(scale * (old + val));
  }
}

// Every wave waits for its own atomics to complete, then one thread passes
// the turn on.
__device__ __forceinline__ void relay_release(int* semp, int turn, int nv, int tid) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0 && nv > 1) __hip_atomic_store(semp, turn + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// bwd_dot: one block per (group of DOT_TILES q-tiles, query head, sequence).
// Every thread issues all of its O / dO loads before the first product, so
// a block keeps DOT_TILES * 64 rows of loads in flight.  One q-tile per block
// (measured on MI355X against 2 and 4): the same speed on long sequences,
// where the pass runs at the read bandwidth, and more blocks in flight on
// short ones, where it is latency-bound (batch 2, 16 heads, S = 4096: the
// whole backward step 66 -> 62 us).

constexpr int DOT_TILES = 1;

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dot_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  const Problem& p = a.p;
  const int tile0 = blockIdx.x * DOT_TILES, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const Seq s = load_seq(p, b);
  if (tile0 == 0 && h == 0 && b == 0 && tid < 2) a.ctl[tid] = 0;
  if (!p.split_dq && tid < DOT_TILES && tile0 + tid < p.n_q_tiles)  // relay or chunk counters
    a.sem[((int64_t)b * p.Hq + h) * p.n_q_tiles + tile0 + tid] = 0;

  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RPP = kThreads / CH;  // rows per pass
  constexpr int NPT = kTile / RPP;    // passes per q-tile
  constexpr int NP = DOT_TILES * NPT;
  __shared__ float s_term[DOT_TILES * kTile];
  const int c = tid % CH, rl = tid / CH;
  const T* __restrict__ ob = static_cast<const T*>(a.o) + elem_off(p, p.so, b, s.row0_q, h, 0) + 8 * c;
  const T* __restrict__ gb = static_cast<const T*>(a.dO) + elem_off(p, p.sdo, b, s.row0_q, h, 0) + 8 * c;
  const int64_t rs_o = p.so[2], rs_g = p.sdo[2];
  V8 ov[NP], gv[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {  // rows past the sequence read row 0 and are dropped
    const int row = tile0 * kTile + ps * RPP + rl;
    const int rr = row < s.len_q ? row : 0;
    if (s.len_q > 0) {
      // O is read only here: keep it from displacing dO, which the main
      // kernel reads next
      ov[ps] = __builtin_nontemporal_load(reinterpret_cast<const V8*>(ob + rr * rs_o));
      gv[ps] = *reinterpret_cast<const V8*>(gb + rr * rs_g);
    }
  }
  float* __restrict__ delta = a.delta + s.stat0 + h * s.stat_hs;
  const float* __restrict__ lse = a.lse + s.stat0 + h * s.stat_hs;
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int row = tile0 * kTile + ps * RPP + rl;
    float acc = 0.f;
    if (row < s.len_q)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += Elem<T>::to_float(ov[ps][e]) * Elem<T>::to_float(gv[ps][e]);
    acc = CH == 8 ? lanes8_sum(acc) : lanes16_sum(acc);  // the lanes of the row
    if (c == 0) {
      float t = 0.f;
      if (row < s.cap_q) {
        delta[row] = acc;
        if (p.has_sink && row < s.len_q) {
          const float l = lse[row];
          t = (l == -INFINITY) ? 0.f : expf(a.sink[h] - l) * acc;
        }
      }
      s_term[ps * RPP + rl] = t;
    }
  }
  if (p.has_sink) {
    __syncthreads();
    if (tid < DOT_TILES && tile0 + tid < p.n_q_tiles) {
      float sum = 0.f;
      for (int r = 0; r < kTile; ++r) sum += s_term[tid * kTile + r];
      a.sink_part[((int64_t)h * p.B + b) * p.n_q_tiles + tile0 + tid] = sum;
    }
  }

  // Clearing for the main kernel: dQ rows of a q-tile that no kv-tile (no
  // chunk of the streaming kernel) visits, where no other kernel writes them
  // (the relay, and the streaming kernel in either mode; the q-major dQ
  // pass of the per-tile path writes its own zeros); and in the streaming
  // kernel's atomic mode the fp32 partial-sum slots (one per q-tile) of
  // q-tiles several chunks visit.
  SeqSched g;
  main_sched(p, s, g);
  for (int t = 0; t < DOT_TILES; ++t) {
    const int tile = tile0 + t, row_base = tile * kTile;
    const int rows = min(kTile, s.cap_q - row_base);
    if (tile >= p.n_q_tiles || rows <= 0) break;
    if (p.split_dq) break;
    const int nv = p.stream ? chunk_visitors(p, g, tile) : g.n_visitors(tile);
    if (nv == 0) {
      T* dqp = static_cast<T*>(a.dq);
      V8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = Elem<T>::from_float(0.f);
      for (int e = tid; e < rows * CH; e += kThreads)
        st8(dqp + elem_off(p, p.sdq, b, s.row0_q, h, row_base + e / CH) + 8 * (e % CH), z);
    } else if (p.stream && !p.stream_relay && nv > 1) {
      float4* acc = reinterpret_cast<float4*>(a.dq_acc + stream_slot(p, s, b, h, tile) * kTile * D);
      const float4 z = {0.f, 0.f, 0.f, 0.f};
      for (int e = tid; e < kTile * (D / 4); e += kThreads) acc[e] = z;
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_clear: where the streaming kernel forms delta itself (no sink), the
// clearing bwd_dot would do for it: the control words, the q-tile counters,
// the dQ rows of q-tiles no chunk visits and, with fp32 atomics, the
// partial-sum slots of q-tiles several chunks visit.  A block takes up to
// 64 q-tiles (the plan's clear_tiles, chosen so that the grid fills the
// chip): each thread of the first ones clears one counter and decides
// whether its tile needs more; the whole block then clears those tiles in
// turn (head_dim 64, the streaming kernel's).

constexpr int kClearTiles = 64;  // most q-tiles per block

template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_clear_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  constexpr int CH = 64 / 8;  // 16-byte chunks per row
  __shared__ int s_tile[kClearTiles];
  __shared__ int s_n;
  const Problem& p = a.p;
  const int tid = threadIdx.x, h = blockIdx.y, b = blockIdx.z, nt = p.clear_tiles, t0 = blockIdx.x * nt;
  if (blockIdx.x == 0 && h == 0 && b == 0 && tid < 2) a.ctl[tid] = 0;
  if (tid == 0) s_n = 0;
  __syncthreads();
  const Seq s = load_seq(p, b);
  if (tid < nt && t0 + tid < p.n_q_tiles) {
    const int tile = t0 + tid;
    a.sem[((int64_t)b * p.Hq + h) * p.n_q_tiles + tile] = 0;
    if (tile * kTile < s.cap_q) {
      SeqSched g;
      main_sched(p, s, g);
      const int nv = chunk_visitors(p, g, tile);
      // nv == 0: zero dQ rows; nv > 1 with fp32 atomics: zero the slot
      if (nv == 0) s_tile[atomicAdd(&s_n, 1)] = tile;
      else if (!p.stream_relay && nv > 1) s_tile[atomicAdd(&s_n, 1)] = -1 - tile;
    }
  }
  __syncthreads();
  const int n = s_n;
  for (int k = 0; k < n; ++k) {
    const int e0 = s_tile[k];
    if (e0 >= 0) {
      const int row_base = e0 * kTile, rows = min(kTile, s.cap_q - row_base);
      T* dqp = static_cast<T*>(a.dq);
      V8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = Elem<T>::from_float(0.f);
      for (int e = tid; e < rows * CH; e += kThreads)
        st8(dqp + elem_off(p, p.sdq, b, s.row0_q, h, row_base + e / CH) + 8 * (e % CH), z);
    } else {
      float4* acc = reinterpret_cast<float4*>(a.dq_acc + stream_slot(p, s, b, h, -1 - e0) * kTile * 64);
      const float4 z = {0.f, 0.f, 0.f, 0.f};
      for (int e = tid; e < kTile * 64 / 4; e += kThreads) acc[e] = z;
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_main: one block (4 waves) per (kv-tile of 64 keys, kv head, sequence);
// two blocks per CU.
//
// Each wave owns 16 keys of the tile.  For every query head of the kv
// head's group and every q-tile i in [q_lo, q_hi) (descending i):
//   S  = Q_i K^T,  dP = dO_i V^T         A: Q / dO rows (LDS), B: the wave's
//                                         K / V rows (registers)
//   P  = exp2(S c - LSE_i),  dS = P (dP - delta_i)             (fp32, masked)
//   dV^T += dO_i^T P,  dK^T += Q_i^T dS   A: transposed reads of the Q / dO
//                                         tile, B: P / dS from the accumulator
//   dQ_i = dS K                           A: transposed reads of dS^T,
//                                         B: transposed reads of the K tile
// and dQ_i is added into q-tile i's fp32 partial through the ordered relay
// (deterministic = 2); otherwise dQ is left to bwd_dq and the two
// dS^T / dQ steps drop out.  A wave skips the 16-row blocks its keys cannot see.  The
// next visit's Q / dO tile is loaded into registers while the current one
// computes.  All products are 16x16x32 MFMAs with fp32 accumulation.
//
// Q / dO / K tiles use the swizzled layout of tiles.h.

template <typename T, int D, bool RELAY>
__global__ __launch_bounds__(kThreads, 2) void bwd_main_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  constexpr int NS = D / 32;       // k-steps over the head dim
  constexpr int NDB = D / 16;      // 16-column blocks of the head dim
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RPP = kThreads / CH;
  constexpr int NPASS = kTile / RPP;

  // Q / dO tiles (Q, then dO) and their row statistics (LSE in log2 units,
  // then delta), double-buffered as separately named arrays: every access
  // names its array, so the compiler sees that reads of one buffer need not
  // wait for the loads streaming into the other.  The relay keeps one tile
  // buffer (its K tile and dS^T take the room; two blocks still fit on a CU
  // at head_dim 128) and refills it while the relay step runs.
  __shared__ __align__(16) T sQO0[2 * kTile * D];
  __shared__ __align__(16) T sQO1[RELAY ? 8 : 2 * kTile * D];
  __shared__ __align__(16) float sLD0[2 * kTile];
  __shared__ __align__(16) float sLD1[2 * kTile];
  __shared__ __align__(16) T sK[kTile * D];
  __shared__ __align__(16) T sdSt[kTile * kTile];  // dS^T [key][q], 64-wide swizzled rows
  __shared__ int sTicket;

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  int L;
  if (RELAY) {
    // Tickets hand out tiles in start order, kv-tile-major, so a tile's relay
    // predecessor (same head, kv-tile - 1) always started earlier: every
    // wait is on a block that is running or done.
    if (tid == 0) sTicket = atomicAdd(&a.ctl[0], 1);
    __syncthreads();
    L = sTicket;
  } else {
    L = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int nbh = p.B * p.Hkv;
  int b, hk, jt;
  if (RELAY) {
    jt = L / nbh;
    b = (L % nbh) / p.Hkv;
    hk = L % p.Hkv;
  } else {
    // kv-head-major: an XCD's contiguous range holds one (or a few) kv heads
    // of every sequence, so sequences of different lengths do not load the
    // XCDs unevenly; a (kv head, sequence)'s kv-tiles stay together
    jt = L % p.n_kv_tiles;
    b = (L / p.n_kv_tiles) % p.B;
    hk = L / (p.n_kv_tiles * p.B);
  }
  const Seq s = load_seq(p, b);
  const int kv0 = jt * kTile;
  if (kv0 >= s.cap_kv) return;
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, p.causal, p.window, p.right, kTile, kTile);
  const int qlo = g.q_lo(jt), nit = g.n_iters(jt);
  const int nvisit = nit * p.G;

  const T* qp = static_cast<const T*>(a.q);
  const T* dop = static_cast<const T*>(a.dO);
  V8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = Elem<T>::from_float(0.f);

  // Mask: with t = row + diag - key, an element is visible iff
  // tlo <= t <= thi (tlo = -R if causal, thi = W if windowed; otherwise far
  // out of reach).  A key past the sequence is pushed below tlo through its
  // lane term, and rows past the sequence carry LSE = +inf.
  const int tlo = p.causal ? -p.right : -(1 << 28), thi = p.window >= 0 ? p.window : (1 << 28);
  const unsigned trange = (unsigned)(thi - tlo);
  const int key = kv0 + 16 * w + c;
  const int tkey = key < s.len_kv ? g.diag - key - tlo : -(1 << 30);  // t - tlo = row + tkey

  // K / V rows of this wave's 16 keys (B operands of S = Q K^T, dP = dO V^T)
  // and the whole K tile in LDS (A operand of dQ^T = K^T dS^T).
  V8 kB[NS], vB[NS];
  {
    const bool ok = key < s.len_kv;
    const int kr = min(key, max(s.len_kv - 1, 0));
    const T* krow = static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, hk, kr) + 8 * gq;
    const T* vrow = static_cast<const T*>(a.v) + elem_off(p, p.sv, b, s.row0_kv, hk, kr) + 8 * gq;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      kB[st] = ok ? ld8(krow + 32 * st) : zero8;
      vB[st] = ok ? ld8(vrow + 32 * st) : zero8;
    }
  }
  if (RELAY) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = tid / CH + ps * RPP, ch = tid % CH, kk = kv0 + r;
      const V8 x = kk < s.len_kv
                       ? ld8(static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, hk, kk) + 8 * ch)
                       : zero8;
      *reinterpret_cast<V8*>(&sK[toff<D>(r, ch)]) = x;
    }
  }

  f32x4 dV[NDB], dK[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dV[db] = dK[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staging of one visit's Q / dO tile, straight into LDS, and of its row
  // statistics (registers first, then LDS).
  float rlse = 0.f, rdelta = 0.f;
  int st_i = 0;
  // Visits go head by head through the group, q-tiles descending within a
  // head: visit v is (head hk G + v / nit, q-tile qlo + nit - 1 - v % nit),
  // walked here with two counters instead of a division per visit.
  auto next_visit = [&](int& vh, int& vi) {
    if (vi > qlo) {
      --vi;
    } else {
      ++vh;
      vi = qlo + nit - 1;
    }
  };
  // this thread's 16-byte chunk of row 0, head 0; a row r of head h is
  // r * (row stride) + h * (head stride) further in either layout.  Lane l
  // of a wave fills bytes 16 l of the wave's 1 KB piece of a pass: row
  // tid / CH + ps RPP, stored chunk tid % CH, which holds logical chunk
  // (tid % CH) ^ tsw(row) (the same in every pass).  Rows past the sequence
  // repeat its last row: finite values, and P = 0 there (LSE = +inf).
  const int qch = (tid % CH) ^ tsw<D>(tid / CH);
  const T* q00 = qp + elem_off(p, p.sq, b, s.row0_q, 0, 0) + 8 * qch;
  const T* o00 = dop + elem_off(p, p.sdo, b, s.row0_q, 0, 0) + 8 * qch;
  auto stage_load = [&](int h, int i, T* dst) {  // a visited q-tile: the sequence has rows
    st_i = i;
    const int row0 = i * kTile;
    // the statistics first: waiting for them does not wait for the tiles
    if (tid < kTile) {
      const int64_t si = s.stat0 + h * s.stat_hs + min(row0 + tid, s.len_q - 1);
      rlse = a.lse[si];
      rdelta = a.delta[si];
    }
    const T* qh = q00 + h * p.sq[1];
    const T* oh = o00 + h * p.sdo[1];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int qi = min(row0 + tid / CH + ps * RPP, s.len_q - 1);
      const int piece = (ps * kThreads + 64 * w) * 8;  // wave-uniform element offset
      ld16_to_lds(row_at(qh, qi, p.sq[2]), dst + piece);
      ld16_to_lds(row_at(oh, qi, p.sdo[2]), dst + kTile * D + piece);
    }
  };
  auto stage_stats = [&](float* ld) {
    if (tid < kTile) {
      const bool ok = st_i * kTile + tid < s.len_q;
      ld[tid] = ok ? rlse * kLog2e : INFINITY;  // exp2(x - inf) = 0: padding rows carry no weight
      ld[kTile + tid] = ok ? rdelta : 0.f;
    }
  };

  // per-lane LDS offsets (elements)
  int rd_off[NS], tr_off[NDB], ds_w[4];
#pragma unroll
  for (int st = 0; st < NS; ++st) rd_off[st] = toff<D>(c, 4 * st + gq);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_off[db] = troff<D>(c, gq, db);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) ds_w[mb] = toff<kTile>(16 * w + c, 2 * mb + (gq >> 1)) + 4 * (gq & 1);
  const int ds_tr = troff<kTile>(c, gq, w);  // dS^T columns (q) 16 w ..

  int h = hk * p.G, i = qlo + nit - 1;  // the current visit
  if (nvisit > 0) {
    stage_load(h, i, sQO0);
    stage_stats(sLD0);
  }
  // Every load has landed before the first visit (and on the path that
  // skips the staging the compiler would otherwise keep the K / V loads
  // outstanding and make each visit's first products wait for the next
  // visit's prefetch).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  T* dqp = static_cast<T*>(a.dq);
  int v = 0, nh = h, ni = i;  // the visit count and the next visit
  // One visit: reads the tile in (sQ, sdO) and its statistics (sLse,
  // sDelta), and streams the next visit's into (nQO, nLD), which were last
  // read before the previous barrier.  False after the last visit.
  auto visit = [&](const T* sQ, const float* sLse, T* nQO, float* nLD) -> bool {
    const T* sdO = sQ + kTile * D;
    const float* sDelta = sLse + kTile;
    nh = h;
    ni = i;
    next_visit(nh, ni);
    const bool more = v + 1 < nvisit;
    if (!RELAY && more) stage_load(nh, ni, nQO);
    const int q0 = i * kTile;
    // t - tlo of (row q0, key kv0 + 16 w); block mb spans [u_mb - 15, u_mb + 15]
    const int u0 = q0 + g.diag - (kv0 + 16 * w) - tlo;

    // Where the wave's 16 keys see all 64 rows (t - tlo in [u0 - 15,
    // u0 + 63] inside [0, trange], every key in the sequence) the mask and
    // the per-block tests drop out (FULL: straight-line products, one
    // 16-row block at a time to bound register use); rows past the sequence
    // still get P = 0 from LSE = +inf.
    // Otherwise the wave skips its 16-row blocks and 32-row halves that see
    // no key, and masks.
    const bool full = u0 >= 15 && u0 + 63 <= (int)trange && kv0 + 16 * w + 15 < s.len_kv;
    auto visit_body = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      f32x4 S[4], dP[4];
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FULL) {
        // every block: one straight run, each block's operands read while
        // the previous block's products run
        V8 aq[2][NS], ao[2][NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          aq[0][st] = *reinterpret_cast<const V8*>(&sQ[rd_off[st]]);
          ao[0][st] = *reinterpret_cast<const V8*>(&sdO[rd_off[st]]);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb + 1 < 4) {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              aq[(mb + 1) & 1][st] = *reinterpret_cast<const V8*>(&sQ[16 * (mb + 1) * D + rd_off[st]]);
              ao[(mb + 1) & 1][st] = *reinterpret_cast<const V8*>(&sdO[16 * (mb + 1) * D + rd_off[st]]);
            }
          }
          S[mb] = mfma16(aq[mb & 1][0], kB[0], zero4);
          dP[mb] = mfma16(ao[mb & 1][0], vB[0], zero4);
#pragma unroll
          for (int st = 1; st < NS; ++st) {
            S[mb] = mfma16(aq[mb & 1][st], kB[st], S[mb]);
            dP[mb] = mfma16(ao[mb & 1][st], vB[st], dP[mb]);
          }
        }
      } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int um = u0 + 16 * mb;
          if (um + 15 < 0 || um - 15 > (int)trange) {
            S[mb] = dP[mb] = zero4;
            continue;
          }
          // the first product starts from a literal zero accumulator
          S[mb] = mfma16(*reinterpret_cast<const V8*>(&sQ[16 * mb * D + rd_off[0]]), kB[0], zero4);
          dP[mb] = mfma16(*reinterpret_cast<const V8*>(&sdO[16 * mb * D + rd_off[0]]), vB[0], zero4);
#pragma unroll
          for (int st = 1; st < NS; ++st) {
            S[mb] = mfma16(*reinterpret_cast<const V8*>(&sQ[16 * mb * D + rd_off[st]]), kB[st], S[mb]);
            dP[mb] = mfma16(*reinterpret_cast<const V8*>(&sdO[16 * mb * D + rd_off[st]]), vB[st], dP[mb]);
          }
        }
      }
      V8 pP[2], pS[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int um = u0 + 16 * mb;
        const bool any = FULL || (um + 15 >= 0 && um - 15 <= (int)trange);
        float pv[4] = {0.f, 0.f, 0.f, 0.f}, dsv[4] = {0.f, 0.f, 0.f, 0.f};
        if (FULL) {
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&sLse[16 * mb + 4 * gq]);
          const f32x4 del4 = *reinterpret_cast<const f32x4*>(&sDelta[16 * mb + 4 * gq]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[r] = fast_exp2(S[mb][r] * p.scale_log2 - lse4[r]);
            dsv[r] = pv[r] * (dP[mb][r] - del4[r]);
          }
        } else if (any) {
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&sLse[16 * mb + 4 * gq]);
          const f32x4 del4 = *reinterpret_cast<const f32x4*>(&sDelta[16 * mb + 4 * gq]);
          const int tb = q0 + 16 * mb + 4 * gq + tkey;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = S[mb][r] * p.scale_log2 - lse4[r];
            asm("" : "+v"(x));
            pv[r] = fast_exp2((unsigned)(tb + r) <= trange ? x : -INFINITY);
            dsv[r] = pv[r] * (dP[mb][r] - del4[r]);
          }
        }
        T pk[4], sk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pk[r] = Elem<T>::from_float(pv[r]);
          sk[r] = Elem<T>::from_float(dsv[r]);
          pP[mb >> 1][(mb & 1) * 4 + r] = pk[r];
          pS[mb >> 1][(mb & 1) * 4 + r] = sk[r];
        }
        if (RELAY) *reinterpret_cast<u32x2*>(&sdSt[ds_w[mb]]) = __builtin_bit_cast(u32x2, sk);
      }
      // dV^T += dO^T P, dK^T += Q^T dS over 32-row halves that see any key
      if constexpr (FULL) {
        // both halves, the transposed operands read one product ahead
        auto tro = [&](int x) { return trpair(&sdO[32 * (x / NDB) * D + tr_off[x % NDB]], &sdO[(32 * (x / NDB) + 16) * D + tr_off[x % NDB]]); };
        auto trq = [&](int x) { return trpair(&sQ[32 * (x / NDB) * D + tr_off[x % NDB]], &sQ[(32 * (x / NDB) + 16) * D + tr_off[x % NDB]]); };
        V8 to[2], tq[2];
        to[0] = tro(0);
        tq[0] = trq(0);
#pragma unroll
        for (int x = 0; x < 2 * NDB; ++x) {
          if (x + 1 < 2 * NDB) {
            to[(x + 1) & 1] = tro(x + 1);
            tq[(x + 1) & 1] = trq(x + 1);
          }
          dV[x % NDB] = mfma16(to[x & 1], pP[x / NDB], dV[x % NDB]);
          dK[x % NDB] = mfma16(tq[x & 1], pS[x / NDB], dK[x % NDB]);
        }
        return;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int um = u0 + 32 * s2;  // rows +0..31: t - tlo in [um - 15, um + 31]
        if (!FULL && (um + 31 < 0 || um - 15 > (int)trange)) continue;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dV[db] = mfma16(trpair(&sdO[32 * s2 * D + tr_off[db]], &sdO[(32 * s2 + 16) * D + tr_off[db]]), pP[s2],
                          dV[db]);
          dK[db] = mfma16(trpair(&sQ[32 * s2 * D + tr_off[db]], &sQ[(32 * s2 + 16) * D + tr_off[db]]), pS[s2],
                          dK[db]);
        }
      }
    };
    // (the straight-line body is kept to head_dim 64 without the relay: in
    // the others it would cost occupancy or spill)
    if constexpr (D == 64 && !RELAY) {
      if (full)
        visit_body(std::true_type());
      else
        visit_body(std::false_type());
    } else {
      visit_body(std::false_type());
    }
    if (!RELAY) {
      if (more) stage_stats(nLD);
      __builtin_amdgcn_s_waitcnt(0);  // the next tile has landed
      __syncthreads();                // and this one is free
      ++v;
      h = nh;
      i = ni;
      return more;
    }
    __syncthreads();  // dS^T complete; the Q / dO tile is free
    if (more) stage_load(nh, ni, nQO);

    // dQ rows q0 + 16 w + 4 gq + r, d = 16 db + c: each relay add covers 16
    // consecutive floats of 4 rows
    f32x4 dQ[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dQ[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const V8 as = trpair(&sdSt[32 * ks * kTile + ds_tr], &sdSt[(32 * ks + 16) * kTile + ds_tr]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dQ[db] = mfma16(as, trpair(&sK[32 * ks * D + tr_off[db]], &sK[(32 * ks + 16) * D + tr_off[db]]), dQ[db]);
    }

    // Ordered relay: visitors of q-tile i add in kv-tile order; a turn is
    // counted from i's first visitor kv_first(i).  Every access to the fp32
    // partial is an agent-scope atomic read-modify-write (coherent across
    // XCDs), so a release only has to wait until this block's atomics have
    // completed (s_waitcnt) before passing the turn on; no L2 write-back is
    // needed.
    const int qr0 = q0 + 16 * w + 4 * gq;  // row of dQ[.][0]
    float* accr = a.dq_acc + (s.stat0 + h * s.stat_hs + qr0) * D + c;
    const int turn = g.relay_turn(i, jt), nv = g.n_visitors(i);
    int* semp = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
    if (tid == 0) sTicket = turn > 0 && relay_wait(semp, turn + a.relay_bias, a.spin_limit, a.ctl + 1);
    __syncthreads();
    const bool expired = sTicket != 0;  // then this turn adds NaN (poison)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (qr0 + r >= s.cap_q) continue;
      T* outr = dqp + elem_off(p, p.sdq, b, s.row0_q, h, qr0 + r) + c;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        relay_add<T>(accr + r * D + 16 * db, expired ? __builtin_nanf("") : dQ[db][r], turn, nv, p.scale,
                     outr + 16 * db);
    }
    relay_release(semp, turn, nv, tid);
    if (more) stage_stats(nLD);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // next tile staged; dS^T reads done
    ++v;
    h = nh;
    i = ni;
    return more;
  };
  if (nvisit > 0) {
    if constexpr (RELAY) {
      while (visit(sQO0, sLD0, sQO0, sLD1) && visit(sQO0, sLD1, sQO0, sLD0)) {
      }
    } else {
      while (visit(sQO0, sLD0, sQO1, sLD1) && visit(sQO1, sLD1, sQO0, sLD0)) {
      }
    }
  }

  // Epilogue: dK = scale * sum dS^T Q, dV = sum P^T dO; a tile that visited
  // nothing stores zeros.  Lane holds d = 16 db + 4 gq + r of key `key`.
  if (key < s.cap_kv) {
    T* dkp = static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, hk, key);
    T* dvp = static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, hk, key);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      T kx[4], vx[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kx[r] = Elem<T>::from_float(p.scale * dK[db][r]);
        vx[r] = Elem<T>::from_float(dV[db][r]);
      }
      *reinterpret_cast<u32x2*>(dkp + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, kx);
      *reinterpret_cast<u32x2*>(dvp + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, vx);
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_dq: q-tile-stationary dQ pass of the per-tile path (deterministic 0
// and 1: it sums each row's kv-tiles in a fixed order), one block (4
// waves) per (run of p.dq_tiles consecutive q-tiles, query head, sequence);
// two blocks per CU.
//
// Each wave owns 16 query rows of the current q-tile i; a lane keeps its
// row's Q and dO slices (the B operands below), LSE and delta in registers.
// For every kv-tile j in [kv_first(i), kv_last(i)]:
//   S^T = K Q^T,  dP^T = V dO^T       A: K / V rows (LDS), B: Q / dO
//   P^T = exp2(S^T c - LSE),  dS^T = P^T (dP^T - delta)        (fp32, masked)
//   dQ^T += K^T dS^T                   A: transposed reads of the K tile,
//                                      B: dS^T straight from the accumulator
// The block walks the (q-tile, kv-tile) pairs of its run as one pipeline:
// K and V are double-buffered in LDS and the next pair's tiles load into
// registers while the current pair computes, also across a q-tile boundary,
// where the next q-tile's Q / dO rows are prefetched the same way.  Short
// visitor ranges (a narrow window) then pay no per-q-tile start-up latency.
// Every dQ row is produced by one wave and leaves as 16-bit values once, so
// no fp32 accumulator or conversion pass exists.  The transposed orientation
// leaves each lane with 4 consecutive head-dim values of one row: one 8-byte
// store per 16 columns.  A wave skips the 16-key blocks its rows cannot see.

// With DELTA (runs of q-tiles, or head_dim 128; no sink; a single-tile
// block takes the run path with a run of one) the pass also forms each row's
// delta = <dO, O> from the dO rows it holds and an extra read of O, and
// stores it for bwd_main, which then runs after it: the separate bwd_dot
// pass, which reads dO and O once more, is not launched.
//
// Occupancy: two blocks per CU, four for single-tile blocks at D = 64, whose
// registers fit in 128 per lane.
template <typename T, int D, bool RUN, bool DELTA>
__global__ __launch_bounds__(kThreads, (D == 64 && !RUN) ? 4 : 2) void bwd_dq_kernel(BwdArgs a) {
  static_assert(!DELTA || RUN, "delta is formed on the q-tile-run path");
  typedef typename Elem<T>::vec8 V8;
  constexpr int NS = D / 32;   // k-steps over the head dim
  constexpr int NDB = D / 16;  // 16-column blocks of the head dim
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int RPP = kThreads / CH;
  constexpr int NPASS = kTile / RPP;

  // K / V double buffer as two arrays (K tile, then V tile): every access
  // names its array, so the compiler sees that reads of one buffer need not
  // wait for the loads streaming into the other
  __shared__ __align__(16) T sKV0[2 * kTile * D];
  __shared__ __align__(16) T sKV1[2 * kTile * D];

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // bwd_dot is not launched: clear the control words it would have
  if (DELTA && blockIdx.x == 0 && tid < 2) a.ctl[tid] = 0;

  // block -> (kv head, sequence, run of q-tiles, head within the group): the
  // heads that share a kv head, and neighbouring runs, read the same K / V
  // tiles and run next to each other on one XCD; kv-head-major, so an XCD's
  // range spans every sequence (balanced over mixed lengths), and runs
  // descending, so the later q-tiles, which a causal mask gives the most
  // kv-tiles, start first
  const int nruns = (p.n_q_tiles + p.dq_tiles - 1) / p.dq_tiles;
  int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = L % p.G;
  L /= p.G;
  const int run = nruns - 1 - L % nruns;
  L /= nruns;
  const int b = L % p.B, hk = L / p.B, h = hk * p.G + hg;
  const Seq s = load_seq(p, b);
  const int ia = run * p.dq_tiles;
  const int ib = min(ia + p.dq_tiles, (s.cap_q + kTile - 1) / kTile);  // q-tiles holding slot rows
  if (ia >= ib) return;
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, p.causal, p.window, p.right, kTile, kTile);

  T* dqp = static_cast<T*>(a.dq);
  // dQ = scale * dS K; lane holds d = 16 db + 4 gq + r of row 16 w + c of
  // q-tile i.  Rows past the slot are not stored.
  auto store_dq = [&](int i, const f32x4* v) {
    const int row = i * kTile + 16 * w + c;
    if (row >= s.cap_q) return;
    T* dqr = dqp + elem_off(p, p.sdq, b, s.row0_q, h, row) + 4 * gq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      T x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = Elem<T>::from_float(p.scale * v[db][r]);
      *reinterpret_cast<u32x2*>(dqr + 16 * db) = __builtin_bit_cast(u32x2, x);
    }
  };
  f32x4 dQt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dQt[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // q-tiles no kv-tile visits (rows past the sequence, or out of every
  // window) get zeros
  for (int i = ia; i < ib; ++i)
    if (g.n_visitors(i) == 0) store_dq(i, dQt);
  auto next_visited = [&](int i) {
    while (i < ib && g.n_visitors(i) == 0) ++i;
    return i;
  };
  int ci = next_visited(ia);  // current pair (ci, cj)
  if (ci >= ib) return;
  int cj = g.kv_first(ci);

  // Q / dO rows and row statistics of a visited q-tile (len_q > 0); rows
  // past the sequence repeat its last row and carry LSE = +inf, so that
  // P = exp2(-inf) = 0
  V8 qB[NS], oB[NS], nqB[NS], noB[NS];
  V8 xB[DELTA ? NS : 1], nxB[DELTA ? NS : 1];  // O rows (DELTA)
  float lse2, del, nlse2 = 0.f, ndel = 0.f;
  const T* q0h = static_cast<const T*>(a.q) + elem_off(p, p.sq, b, s.row0_q, h, 0) + 8 * gq;
  const T* o0h = static_cast<const T*>(a.dO) + elem_off(p, p.sdo, b, s.row0_q, h, 0) + 8 * gq;
  const T* x0h = static_cast<const T*>(a.o) + elem_off(p, p.so, b, s.row0_q, h, 0) + 8 * gq;
  auto load_q = [&](int i, V8* qv, V8* ov, V8* xv, float& l2, float& dl) {
    const int row = i * kTile + 16 * w + c;
    const int qr = min(row, s.len_q - 1);
    // the row statistics first: waiting for them then does not wait for
    // the row loads behind them
    l2 = INFINITY;
    dl = 0.f;
    if (row < s.len_q) {
      const int64_t si = s.stat0 + h * s.stat_hs + row;
      l2 = a.lse[si];
      if (!DELTA) dl = a.delta[si];
    }
    const T* qrow = row_at(q0h, qr, p.sq[2]);
    const T* orow = row_at(o0h, qr, p.sdo[2]);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      qv[st] = ld8(qrow + 32 * st);
      ov[st] = ld8(orow + 32 * st);
    }
    if (DELTA) {
      const T* xrow = row_at(x0h, qr, p.so[2]);
#pragma unroll
      for (int st = 0; st < NS; ++st) xv[st] = ld8(xrow + 32 * st);
    }
  };
  // DELTA: delta of the lane's row from its dO and O slices (the 4 lanes
  // holding a row's head-dim quarters reduce by two exchanges); 0 past the
  // sequence; stored for bwd_main for every row of the slot
  auto form_delta = [&](int i, const V8* ov, const V8* xv) {
    float acc = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += Elem<T>::to_float(ov[st][e]) * Elem<T>::to_float(xv[st][e]);
    acc = col4_sum(acc);
    const int row = i * kTile + 16 * w + c;
    const float dl = row < s.len_q ? acc : 0.f;
    if (gq == 0 && row < s.cap_q) a.delta[s.stat0 + h * s.stat_hs + row] = dl;
    return dl;
  };

  // K / V staging (a visited kv-tile: len_kv > 0); rows past the sequence
  // repeat its last key (finite values; the mask gives them zero weight)
  // Straight into LDS: lane l of a wave fills bytes 16 l of the wave's 1 KB
  // piece of a pass, i.e. row tid / CH + ps RPP, stored chunk tid % CH,
  // which holds logical chunk (tid % CH) ^ tsw(row) (rows of a pass differ
  // by multiples of 8, so the chunk is the same in every pass).
  const int kch = (tid % CH) ^ tsw<D>(tid / CH);
  const T* k0 = static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, hk, 0) + 8 * kch;
  const T* v0 = static_cast<const T*>(a.v) + elem_off(p, p.sv, b, s.row0_kv, hk, 0) + 8 * kch;
  auto load_kv = [&](int j, T* dK, T* dV) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int kk = min(j * kTile + tid / CH + ps * RPP, s.len_kv - 1);
      const int piece = (ps * kThreads + 64 * w) * 8;  // wave-uniform element offset
      ld16_to_lds(row_at(k0, kk, p.sk[2]), dK + piece);
      ld16_to_lds(row_at(v0, kk, p.sv[2]), dV + piece);
    }
  };

  // per-lane LDS offsets (elements)
  int rd_off[NS], tr_off[NDB];
#pragma unroll
  for (int st = 0; st < NS; ++st) rd_off[st] = toff<D>(c, 4 * st + gq);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_off[db] = troff<D>(c, gq, db);

  // Mask as in bwd_main: with t = row + diag - key, visible iff
  // 0 <= t - tlo <= trange, and the key lies inside the sequence.
  const int tlo = p.causal ? -p.right : -(1 << 28), thi = p.window >= 0 ? p.window : (1 << 28);
  const unsigned trange = (unsigned)(thi - tlo);

  load_q(ci, qB, oB, xB, lse2, del);
  lse2 *= kLog2e;
  load_kv(cj, sKV0, sKV0 + kTile * D);
  if (DELTA) del = form_delta(ci, oB, xB);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One pair: reads the tiles in (cK, cV) and streams the next pair's into
  // (nK, nV), which were last read before the previous barrier.  False once
  // the run is done.
  auto step = [&](const T* cK, const T* cV, T* nK, T* nV) -> bool {
    // the pair after (ci, cj): the next kv-tile of ci, else the first of
    // the next visited q-tile of the run
    int ni = ci, nj = cj + 1;
    if (nj > g.kv_last(ci)) {
      ni = RUN ? next_visited(ci + 1) : ib;
      nj = ni < ib ? g.kv_first(ni) : 0;
    }
    const bool more = ni < ib;
    if (more) {
      load_kv(nj, nK, nV);
      if (RUN && ni != ci) load_q(ni, nqB, noB, nxB, nlse2, ndel);
    }
    const int kv0 = cj * kTile;
    const int kvn = s.len_kv - kv0;                               // keys of this tile inside the sequence
    const int u0 = ci * kTile + 16 * w + g.diag - tlo - kv0;      // t - tlo at (row 16 w, key kv0)
    const int tq = u0 + c - 4 * gq;                               // t - tlo at (row, key kv0 + 4 gq), minus 16 nb + r

    // The pair's products.  Where the wave's 16 rows see all 64 keys (t - tlo
    // in [u0 - 63, u0 + 15] inside [0, trange], every key in the sequence)
    // the mask and the per-block liveness tests drop out: FULL is the
    // straight-line body for that case (nearly every pair of a long window),
    // the other one skips the 16-key blocks the rows cannot see and masks.
    const bool full = u0 >= 63 && u0 + 15 <= (int)trange && kvn >= kTile;
    auto pair_body = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      f32x4 St[4], dPt[4];
      bool live[4];
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      const f32x4 ndel4 = {-del, -del, -del, -del};  // dP^T accumulates from -delta: it leaves as dP - delta
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int um = u0 - 16 * nb;  // the block spans t - tlo in [um - 15, um + 15]
        live[nb] = FULL || (um + 15 >= 0 && um - 15 <= (int)trange && 16 * nb < kvn);
        if (!live[nb]) {
          St[nb] = dPt[nb] = zero4;
          continue;
        }
        // the first product starts from a literal zero accumulator
        St[nb] = mfma16(*reinterpret_cast<const V8*>(&cK[16 * nb * D + rd_off[0]]), qB[0], zero4);
        dPt[nb] = mfma16(*reinterpret_cast<const V8*>(&cV[16 * nb * D + rd_off[0]]), oB[0], ndel4);
#pragma unroll
        for (int st = 1; st < NS; ++st) {
          St[nb] = mfma16(*reinterpret_cast<const V8*>(&cK[16 * nb * D + rd_off[st]]), qB[st], St[nb]);
          dPt[nb] = mfma16(*reinterpret_cast<const V8*>(&cV[16 * nb * D + rd_off[st]]), oB[st], dPt[nb]);
        }
      }
      // dS^T of key 16 nb + 4 gq + r; blocks 2 ks and 2 ks + 1 form the
      // 32-key B operand of step ks
      V8 bS[2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float dsv[4] = {0.f, 0.f, 0.f, 0.f};
        if (FULL) {
#pragma unroll
          for (int r = 0; r < 4; ++r) dsv[r] = fast_exp2(St[nb][r] * p.scale_log2 - lse2) * dPt[nb][r];
        } else if (live[nb]) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = St[nb][r] * p.scale_log2 - lse2;
            asm("" : "+v"(x));
            const bool vis = (unsigned)(tq - 16 * nb - r) <= trange && 16 * nb + 4 * gq + r < kvn;
            dsv[r] = fast_exp2(vis ? x : -INFINITY) * dPt[nb][r];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) bS[nb >> 1][(nb & 1) * 4 + r] = Elem<T>::from_float(dsv[r]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (!live[2 * ks] && !live[2 * ks + 1]) continue;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dQt[db] = mfma16(trpair(&cK[32 * ks * D + tr_off[db]], &cK[(32 * ks + 16) * D + tr_off[db]]), bS[ks],
                           dQt[db]);
      }
    };
    if (full)
      pair_body(std::true_type());
    else
      pair_body(std::false_type());
    if (ni != ci) {  // q-tile ci is complete
      store_dq(ci, dQt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) dQt[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (RUN && more) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          qB[st] = nqB[st];
          oB[st] = noB[st];
        }
        lse2 = nlse2 * kLog2e;
        del = DELTA ? form_delta(ni, noB, nxB) : ndel;
      }
    }
    if (!more) return false;
    __builtin_amdgcn_s_waitcnt(0);  // the next tiles have landed in LDS
    __syncthreads();                // and (cK, cV) are free
    ci = ni;
    cj = nj;
    return true;
  };
  while (step(sKV0, sKV0 + kTile * D, sKV1, sKV1 + kTile * D) &&
         step(sKV1, sKV1 + kTile * D, sKV0, sKV0 + kTile * D)) {
  }
}

// ---------------------------------------------------------------------------
// bwd_dsink: dSink[h] = -sum of the per-q-tile (per-q-step with the q-major
// streaming kernel) partials, in a fixed order.

__global__ __launch_bounds__(64) void bwd_dsink_kernel(BwdArgs a) {
  const int h = blockIdx.x, l = threadIdx.x;
  const int n = a.p.B * a.p.sink_tiles;
  const float* part = a.sink_part + (int64_t)h * n;
  float acc = 0.f;
  for (int e = l; e < n; e += 64) acc += part[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (l == 0) a.dsink[h] = -acc;
}

// ---------------------------------------------------------------------------
// launchers

template <typename T>
static hipError_t dot_t(const BwdArgs& a, hipStream_t st) {
  dim3 grid((a.p.n_q_tiles + DOT_TILES - 1) / DOT_TILES, a.p.Hq, a.p.B);
  if (a.p.D == 64)
    hipLaunchKernelGGL((bwd_dot_kernel<T, 64>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_dot_kernel<T, 128>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_clear(const BwdArgs& a, hipStream_t st) {
  if (a.p.n_q_tiles == 0) return hipSuccess;
  dim3 grid((a.p.n_q_tiles + a.p.clear_tiles - 1) / a.p.clear_tiles, a.p.Hq, a.p.B);
  if (a.dtype == 0)
    hipLaunchKernelGGL((bwd_clear_kernel<__bf16>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_clear_kernel<_Float16>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dot(const BwdArgs& a, hipStream_t st) {
  if (a.p.n_q_tiles == 0) return hipSuccess;
  return a.dtype == 0 ? dot_t<__bf16>(a, st) : dot_t<_Float16>(a, st);
}

template <typename T, int D>
static hipError_t main_td(const BwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hkv * a.p.n_kv_tiles;
  if (!a.p.split_dq)
    hipLaunchKernelGGL((bwd_main_kernel<T, D, true>), dim3(n), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<T, D, false>), dim3(n), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t st) {
  if (a.p.stream) return launch_bwd_stream(a, st);
  if (a.p.qstream) return launch_bwd_qstream(a, st);
  if (a.p.n_kv_tiles == 0) return hipSuccess;
  if (a.dtype == 0) return a.p.D == 64 ? main_td<__bf16, 64>(a, st) : main_td<__bf16, 128>(a, st);
  return a.p.D == 64 ? main_td<_Float16, 64>(a, st) : main_td<_Float16, 128>(a, st);
}

template <typename T>
static hipError_t dq_t(const BwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hq * ((a.p.n_q_tiles + a.p.dq_tiles - 1) / a.p.dq_tiles);
  const bool run = a.p.dq_tiles > 1;
  if (a.p.D == 64) {
    if (a.p.dq_delta)
      hipLaunchKernelGGL((bwd_dq_kernel<T, 64, true, true>), dim3(n), dim3(kThreads), 0, st, a);
    else if (run)
      hipLaunchKernelGGL((bwd_dq_kernel<T, 64, true, false>), dim3(n), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, 64, false, false>), dim3(n), dim3(kThreads), 0, st, a);
  } else {
    if (a.p.dq_delta)
      hipLaunchKernelGGL((bwd_dq_kernel<T, 128, true, true>), dim3(n), dim3(kThreads), 0, st, a);
    else if (run)
      hipLaunchKernelGGL((bwd_dq_kernel<T, 128, true, false>), dim3(n), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, 128, false, false>), dim3(n), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  if (a.p.n_q_tiles == 0) return hipSuccess;
  return a.dtype == 0 ? dq_t<__bf16>(a, st) : dq_t<_Float16>(a, st);
}

hipError_t launch_bwd_dsink(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(bwd_dsink_kernel, dim3(a.p.Hq), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace swa
