// Streaming main backward kernel for multi-head attention with a short left
// window (gfx950, head_dim 64).
//
// The window-bounded schedule -- kv-step j feeds the q-tiles
// [q_lo(j), q_hi(j)) with q_lo from the causal skip and
// q_hi = ceil((kv_base + step + W - diag) / tile_q) (cudnn-frontend PR #866
// "frost(sdpa): bound the SM80 backward q-loop by the sliding window ...",
// commit message and Change) -- is walked by one block over a chunk of
// consecutive kv-steps.  Because the window is short, the q-tiles a step
// feeds are few and slide forward with it, so:
//   * each q-tile's Q, dO, LSE and delta are staged once into a ring of LDS
//     slots and reused by every kv-step of the chunk that visits it;
//   * each q-tile's dQ is accumulated in registers across those kv-steps and
//     written once, as 16-bit, when its last visitor in the chunk is done;
//   * only q-tiles that two chunks visit (at chunk boundaries) go through the
//     fp32 accumulator: in the ordered relay, a chunk's turn counts from the
//     q-tile's first visiting chunk, kv_first(i) / chunk (the PR's
//     kv_first = max((q_row0 + diag - W) // tile_kv, 0) at chunk width), or
//     through fp32 atomics in the unordered mode.
// The next kv-step's K / V rows and new q-tiles are loaded into registers
// while the current step computes.  One block of 8 waves runs per CU (two
// waves per SIMD).
//
// Per visit (q-tile i of 64 rows, kv-step of 128 keys; wave w owns keys
// 16w .. 16w + 15):
//   S, dP  = Q_i K^T, dO_i V^T   A: Q / dO rows (LDS), B: the wave's K / V rows
//   P, dS  = exp2(S c - LSE_i), P (dP - delta_i)           (fp32, masked)
//   dV^T  += dO_i^T P,  dK^T += Q_i^T dS                   A: transposed reads
//   dQ_i  += dS K   (wave w: rows 16 (w mod 4), head-dim half w / 4)
// All products are v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 accumulate).  A
// wave skips the 16 x 16 blocks the mask hides entirely, and evaluates the
// mask only in blocks it cuts.
//
// LDS tiles are 64 elements (128 bytes) per row, unpadded, with the 16-byte
// chunks of row r permuted by XOR with (r mod 8).  Measured on gfx950
// (SQ_LDS_BANK_CONFLICT): 16-byte row reads are conflict-free in any layout,
// and this permutation also makes the transposed reads conflict-free (a
// plain 128-byte pitch costs 4x, a 144-byte pitch 2x).
// Transposed operands use ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element (i % 4) of lanes i / 4 + 4e (e = 0..3), so a lane
// pointing at row r0 + i / 4, column c0 + 4 (i % 4) receives rows
// r0 .. r0 + 3 of column c0 + i.
#include "kernels.h"

namespace swa {

namespace {

constexpr int SD = 64;        // head dim
constexpr int STEP = 128;     // keys per kv-step
constexpr int NSLOT = 6;      // ring slots: up to 5 active q-tiles + 1
constexpr int NACT = 5;       // most q-tiles one kv-step visits (W <= 128)
constexpr int TROW = 64;      // elements per LDS tile row (128 bytes)
constexpr int NTHR = 512;     // 8 waves

typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));

__device__ __forceinline__ int swz(int r) { return r & 7; }
// element offset of (row r, 16-byte chunk ch) in a swizzled tile
__device__ __forceinline__ int tile_off(int r, int ch) { return r * TROW + ((ch ^ swz(r)) << 3); }
// lane offset of a transposed read: row 4 g + c / 4, column 16 cb + 4 (c % 4)
__device__ __forceinline__ int tr_lane_off(int c, int gq, int cb) {
  const int r = 4 * gq + (c >> 2);
  return r * TROW + (((2 * cb + ((c & 3) >> 1)) ^ swz(r)) << 3) + 4 * (c & 1);
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 gld8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::vec8*>(p);
}

template <typename T>
__device__ __forceinline__ u32x2 ld_tr4(const T* lds_elem) {
  v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(lds_elem));
  return __builtin_bit_cast(u32x2, v);
}

// 8 contraction values for lane (c, g): rows r0 + 4g + e (e < 4) and
// r0 + 16 + 4g + (e - 4) of one column, from a lane offset.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 tr_pair(const T* p) {
  const u32x2 lo = ld_tr4(p);
  const u32x2 hi = ld_tr4(p + 16 * TROW);
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(typename Elem<T>::vec8, r);
}

}  // namespace

template <typename T, bool RELAY>
__global__ __launch_bounds__(NTHR, 1) void bwd_stream_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  __shared__ __align__(16) T sQ[NSLOT][kTile * TROW];
  __shared__ __align__(16) T sdO[NSLOT][kTile * TROW];
  __shared__ __align__(16) float sLse[NSLOT][kTile];
  __shared__ __align__(16) float sDelta[NSLOT][kTile];
  __shared__ __align__(16) T sK[STEP * TROW];
  __shared__ __align__(16) T sdSt[2][STEP * TROW];  // dS^T [key][q], double-buffered by visit
  __shared__ int sTicket;

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (scalar)
  const int wr = w & 3, wd = w >> 2;                        // dQ rows 16 wr, head-dim half wd

  // Chunk-major tickets: a chunk's relay predecessor (same head, chunk - 1)
  // always started earlier.
  if (tid == 0) sTicket = atomicAdd(&a.ctl[0], 1);
  __syncthreads();
  const int L = sTicket;
  const int nbh = p.B * p.Hq;
  const int chunk = L / nbh, bh = L % nbh, b = bh / p.Hq, h = bh % p.Hq;
  const Seq s = load_seq(p, b);
  SeqSched g;
  main_sched(p, s, g);
  const int n_cap_steps = (s.cap_kv + STEP - 1) / STEP;
  const int j0 = chunk * p.chunk;
  if (j0 >= n_cap_steps) return;
  const int j1 = min(j0 + p.chunk, n_cap_steps);
  const int W = p.window;

  const T* qp = static_cast<const T*>(a.q);
  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);
  const T* dop = static_cast<const T*>(a.dO);
  T* dqp = static_cast<T*>(a.dq);
  V8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = Elem<T>::from_float(0.f);

  // ---- per-lane LDS offsets (elements) --------------------------------------
  int rd_off[2];  // row read: row c, chunk 4 ks + gq
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off[ks] = tile_off(c, 4 * ks + gq);
  int tr_off[4];  // transposed read of a 16-column block db
#pragma unroll
  for (int db = 0; db < 4; ++db) tr_off[db] = tr_lane_off(c, gq, db);
  const int tr_off_q = tr_lane_off(c, gq, wr);  // dS^T columns 16 wr .. 16 wr + 15
  // K^T columns of this wave's dQ half (kept out of a runtime-indexed array,
  // which the compiler would place in scratch memory)
  const int tr_off_k0 = tr_lane_off(c, gq, 2 * wd), tr_off_k1 = tr_lane_off(c, gq, 2 * wd + 1);
  int ds_off[2][2];  // dS^T write: row 16w + c, q 32 s2 + 16 hf + 4 gq
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      ds_off[s2][hf] = c * TROW + (((4 * s2 + 2 * hf + (gq >> 1)) ^ swz(c)) << 3) + 4 * (gq & 1);

  // ---- loaders ------------------------------------------------------------
  // V rows of the wave's 16 keys (B operand of dP = dO V^T); the K rows (B
  // operand of S = Q K^T) are read from the step's LDS K tile.
  V8 kB[2], vB[2], vBn[2];
  auto load_v_regs = [&](int j, V8 (&vx)[2]) {
    const int key = j * STEP + 16 * w + c;
    const bool ok = key < s.len_kv;
    const int64_t vo = elem_off(p, p.sv, b, s.row0_kv, h, ok ? key : 0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vx[ks] = ok ? gld8(vp + vo + 32 * ks + 8 * gq) : zero8;
  };
  auto read_k_regs = [&]() {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) kB[ks] = *reinterpret_cast<const V8*>(sK + 16 * w * TROW + rd_off[ks]);
  };
  V8 ktn[2];  // K rows of the next step: 128 rows x 8 chunks over 512 threads
  auto load_k_rows = [&](int j) {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int r = (tid >> 3) + 64 * ps, ch = tid & 7, key = j * STEP + r;
      ktn[ps] = key < s.len_kv ? gld8(kp + elem_off(p, p.sk, b, s.row0_kv, h, key) + 8 * ch) : zero8;
    }
  };
  auto store_k_rows = [&]() {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int r = (tid >> 3) + 64 * ps, ch = tid & 7;
      *reinterpret_cast<V8*>(&sK[tile_off(r, ch)]) = ktn[ps];
    }
  };
  struct QRegs {
    V8 q, o;
    float lse, delta;
  };
  auto load_q_tile = [&](int i, QRegs& r) {
    const int row = tid >> 3, ch = tid & 7, qi = i * kTile + row;
    if (qi < s.len_q) {
      r.q = gld8(qp + elem_off(p, p.sq, b, s.row0_q, h, qi) + 8 * ch);
      r.o = gld8(dop + elem_off(p, p.sdo, b, s.row0_q, h, qi) + 8 * ch);
    } else {
      r.q = zero8;
      r.o = zero8;
    }
    if (tid < kTile) {
      const int q2 = i * kTile + tid;
      if (q2 < s.len_q) {
        const int64_t si = s.stat0 + h * s.stat_hs + q2;
        r.lse = a.lse[si] * kLog2e;
        r.delta = a.delta[si];
      } else {
        r.lse = INFINITY;  // exp2(x - inf) = 0: padding rows carry no weight
        r.delta = 0.f;
      }
    }
  };
  auto store_q_tile = [&](int i, const QRegs& r) {
    const int sl = i % NSLOT, row = tid >> 3, ch = tid & 7;
    *reinterpret_cast<V8*>(&sQ[sl][tile_off(row, ch)]) = r.q;
    *reinterpret_cast<V8*>(&sdO[sl][tile_off(row, ch)]) = r.o;
    if (tid < kTile) {
      sLse[sl][tid] = r.lse;
      sDelta[sl][tid] = r.delta;
    }
  };

  // ---- accumulators -------------------------------------------------------
  // dQ of q-tile q_lo(j) + k in dQa[k] (rows q = 16 wr + 4gq + r, d =
  // 16 (2 wd + e) + c), shifted down when q_lo advances between kv-steps
  f32x4 dQa[NACT][2];
  f32x4 dVa[4], dKa[4];  // dV^T / dK^T[d = 16db + 4gq + r][key = 16w + c]
#pragma unroll
  for (int k = 0; k < NACT; ++k) dQa[k][0] = dQa[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) dVa[db] = dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- dQ of a retiring q-tile ------------------------------------------------
  auto acc_ptr = [&](int i, int r, int e) -> float* {
    const int qi = i * kTile + 16 * wr + 4 * gq + r;
    return a.dq_acc + (s.stat0 + h * s.stat_hs + qi) * SD + 16 * (2 * wd + e) + c;
  };
  auto retire = [&](int i, f32x4 (&acc)[2]) {  // block-uniform arguments
    const int first = g.kv_first(i) / p.chunk, last = g.kv_last(i) / p.chunk;
    if (first == last) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = i * kTile + 16 * wr + 4 * gq + r;
        if (qi >= s.cap_q) continue;
        T* row = dqp + elem_off(p, p.sdq, b, s.row0_q, h, qi) + 32 * wd + c;
        row[0] = Elem<T>::from_float(p.scale * acc[0][r]);
        row[16] = Elem<T>::from_float(p.scale * acc[1][r]);
      }
    } else if (!RELAY) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * wr + 4 * gq + r < s.len_q) {
          unsafeAtomicAdd(acc_ptr(i, r, 0), acc[0][r]);
          unsafeAtomicAdd(acc_ptr(i, r, 1), acc[1][r]);
        }
    } else if (first == chunk) {
      // first visiting chunk of a boundary tile: turn 0, no wait
      int* semp = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * wr + 4 * gq + r < s.cap_q)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            __hip_atomic_exchange(acc_ptr(i, r, e), acc[e][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(semp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // a later turn: stash the partial; it is added in turn order once this
      // chunk has finished its own kv-steps
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * wr + 4 * gq + r < s.cap_q)
#pragma unroll
          for (int e = 0; e < 2; ++e) a.dq_stash[acc_ptr(i, r, e) - a.dq_acc] = acc[e][r];
    }
    acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- prologue -------------------------------------------------------------
  load_v_regs(j0, vB);
  load_k_rows(j0);
  store_k_rows();
  int loaded_hi = g.q_lo(j0);  // the ring holds q-tiles [.., loaded_hi)
  int acc_lo = g.q_lo(j0);     // q-tile held in dQa[0]
  QRegs pf[2];
  int pf_lo = 0, pf_n = 0;
  int vpar = 0;  // dS^T buffer of the current visit

  for (int j = j0; j < j1; ++j) {
    const int qlo = g.q_lo(j), nit = min(g.n_iters(j), NACT), qhi = qlo + nit;
    if (loaded_hi < qlo) loaded_hi = qlo;
    for (; loaded_hi < qhi; ++loaded_hi) {  // chunk start and gaps only
      QRegs t;
      load_q_tile(loaded_hi, t);
      store_q_tile(loaded_hi, t);
    }
    __syncthreads();  // ring and sK ready
    read_k_regs();
    for (; acc_lo < qlo; ++acc_lo) {  // realign dQa[0] with q_lo(j)
#pragma unroll
      for (int k = 0; k + 1 < NACT; ++k) {
        dQa[k][0] = dQa[k + 1][0];
        dQa[k][1] = dQa[k + 1][1];
      }
      dQa[NACT - 1][0] = dQa[NACT - 1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const bool has_next = j + 1 < j1;
    if (has_next) {
      load_v_regs(j + 1, vBn);
      load_k_rows(j + 1);
      const int nlo = g.q_lo(j + 1), nhi = nlo + min(g.n_iters(j + 1), NACT);
      pf_lo = max(loaded_hi, nlo);
      pf_n = max(0, min(2, nhi - pf_lo));
      if (pf_n > 0) load_q_tile(pf_lo, pf[0]);
      if (pf_n > 1) load_q_tile(pf_lo + 1, pf[1]);
    }

    const int kv0 = j * STEP;
    // t(row, key) = row + diag - key; visible iff 0 <= t <= W.  A key past
    // the sequence is pushed out of every window through its lane base.
    const int keyl = kv0 + 16 * w + c;
    const int tkey = keyl < s.len_kv ? g.diag - keyl : -(1 << 29);
    const bool keys_ok = kv0 + STEP <= s.len_kv;  // no key past the sequence

#pragma unroll
    for (int k = 0; k < NACT; ++k) {
      if (k >= nit) break;
      const int i = qlo + k, sl = i % NSLOT, q0 = i * kTile;
      const T* tQ = sQ[sl];
      const T* tO = sdO[sl];
      // t of (row q0, key kv0 + 16w); block mb spans t in [u - 15, u + 15]
      // with u = u0 + 16 mb
      const int u0 = q0 + g.diag - (kv0 + 16 * w);
      f32x4 S[4], dP[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        S[mb] = dP[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int um = u0 + 16 * mb;
        if (um + 15 < 0 || um - 15 > W) continue;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          S[mb] = mfma16(*reinterpret_cast<const V8*>(tQ + 16 * mb * TROW + rd_off[ks]), kB[ks], S[mb]);
          dP[mb] = mfma16(*reinterpret_cast<const V8*>(tO + 16 * mb * TROW + rd_off[ks]), vB[ks], dP[mb]);
        }
      }
      // P and dS in the accumulator layout (rows 16mb + 4gq + r)
      V8 pP[2], pS[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int um = u0 + 16 * mb;
        const bool any = um + 15 >= 0 && um - 15 <= W;
        const bool full = keys_ok && um - 15 >= 0 && um + 15 <= W;
        float pv[4] = {0.f, 0.f, 0.f, 0.f}, dsv[4] = {0.f, 0.f, 0.f, 0.f};
        if (any) {
          const float4 lse4 = *reinterpret_cast<const float4*>(&sLse[sl][16 * mb + 4 * gq]);
          const float4 del4 = *reinterpret_cast<const float4*>(&sDelta[sl][16 * mb + 4 * gq]);
          const float lsev[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
          const float delv[4] = {del4.x, del4.y, del4.z, del4.w};
          const int tb = q0 + 16 * mb + 4 * gq + tkey;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = S[mb][r] * p.scale_log2 - lsev[r];
            if (!full) x = (unsigned)(tb + r) <= (unsigned)W ? x : -INFINITY;
            pv[r] = fast_exp2(x);
            dsv[r] = pv[r] * (dP[mb][r] - delv[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pP[mb >> 1][(mb & 1) * 4 + r] = Elem<T>::from_float(pv[r]);
          pS[mb >> 1][(mb & 1) * 4 + r] = Elem<T>::from_float(dsv[r]);
        }
      }
      // dS^T into this visit's buffer: the visit before last read the same
      // buffer for its dQ, and every wave finished that before it passed the
      // previous visit's barrier
      T* dst = sdSt[vpar];
      vpar ^= 1;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 v = __builtin_bit_cast(u32x4, pS[s2]);
        T* base = dst + 16 * w * TROW;
        *reinterpret_cast<u32x2*>(base + ds_off[s2][0]) = u32x2{v[0], v[1]};
        *reinterpret_cast<u32x2*>(base + ds_off[s2][1]) = u32x2{v[2], v[3]};
      }
      // dV^T += dO^T P, dK^T += Q^T dS  (skip 32-row halves whose P is zero)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int um0 = u0 + 32 * s2;  // blocks mb = 2 s2, 2 s2 + 1: t in [um0 - 15, um0 + 31]
        if (um0 + 31 < 0 || um0 - 15 > W) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          dVa[db] = mfma16(tr_pair(tO + 32 * s2 * TROW + tr_off[db]), pP[s2], dVa[db]);
          dKa[db] = mfma16(tr_pair(tQ + 32 * s2 * TROW + tr_off[db]), pS[s2], dKa[db]);
        }
      }
      __syncthreads();  // dS^T complete
      // dQ rows 16 wr .. 16 wr + 15, head-dim half wd, += dS K over the 128 keys
      const int ud = q0 + 16 * wr + g.diag - kv0;  // t of (row 16 wr, key 0)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int uk = ud - 32 * ks;  // rows +0..15, keys +0..31: t in [uk - 31, uk + 15]
        if (uk + 15 < 0 || uk - 31 > W) continue;
        const V8 as = tr_pair(dst + 32 * ks * TROW + tr_off_q);
        dQa[k][0] = mfma16(as, tr_pair(sK + 32 * ks * TROW + tr_off_k0), dQa[k][0]);
        dQa[k][1] = mfma16(as, tr_pair(sK + 32 * ks * TROW + tr_off_k1), dQa[k][1]);
      }
    }

    // q-tiles whose last visitor in this chunk was this step
#pragma unroll
    for (int k = 0; k < NACT; ++k)
      if (k < nit && min(g.kv_last(qlo + k), j1 - 1) == j) retire(qlo + k, dQa[k]);
    // dK / dV of this step (zeros if it visited nothing)
    if (keyl < s.cap_kv) {
      T* dkr = static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, h, keyl);
      T* dvr = static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, h, keyl);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        T kx[4], vx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          kx[r] = Elem<T>::from_float(p.scale * dKa[db][r]);
          vx[r] = Elem<T>::from_float(dVa[db][r]);
        }
        *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, kx);
        *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, vx);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) dVa[db] = dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    __syncthreads();  // ring slots of retired tiles and sK are free
    if (has_next) {
      if (pf_n > 0) store_q_tile(pf_lo, pf[0]);
      if (pf_n > 1) store_q_tile(pf_lo + 1, pf[1]);
      if (pf_n > 0) loaded_hi = max(loaded_hi, pf_lo + pf_n);
      store_k_rows();
      vB[0] = vBn[0];
      vB[1] = vBn[1];
    }
  }

  // ---- relay: boundary q-tiles this chunk joined after another chunk -------
  if (RELAY && j0 < g.n_kv_tiles) {
    for (int i = g.q_lo(j0); i < g.n_q_tiles && i < g.q_hi(j0); ++i) {
      const int first = g.kv_first(i) / p.chunk;
      if (first >= chunk) break;  // kv_first is nondecreasing in i
      const int turn = chunk - first, nv = g.kv_last(i) / p.chunk - first + 1;
      int* semp = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
      if (tid == 0) {
        int spins = 0;
        while (__hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != turn) {
          if (++spins > a.spin_limit) {  // watchdog: never hang the device
            atomicAdd(&a.ctl[1], 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = i * kTile + 16 * wr + 4 * gq + r;
        if (qi >= s.cap_q) continue;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float* ap = acc_ptr(i, r, e);
          const float mine = a.dq_stash[ap - a.dq_acc];
          if (turn < nv - 1) {
            __hip_atomic_fetch_add(ap, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            const float old = __hip_atomic_fetch_add(ap, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            dqp[elem_off(p, p.sdq, b, s.row0_q, h, qi) + 16 * (2 * wd + e) + c] =
                Elem<T>::from_float(p.scale * (old + mine));
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0 && turn < nv - 1)
        __hip_atomic_store(semp, turn + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_bwd_stream(const BwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hq * a.p.n_chunks;
  if (n == 0) return hipSuccess;
  if (a.dtype == 0) {
    if (a.deterministic)
      hipLaunchKernelGGL((bwd_stream_kernel<__bf16, true>), dim3(n), dim3(NTHR), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<__bf16, false>), dim3(n), dim3(NTHR), 0, st, a);
  } else {
    if (a.deterministic)
      hipLaunchKernelGGL((bwd_stream_kernel<_Float16, true>), dim3(n), dim3(NTHR), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<_Float16, false>), dim3(n), dim3(NTHR), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace swa
