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
// while the current step computes; one block of 4 waves runs per CU.
//
// Per visit (q-tile i of 64 rows, kv-step of 128 keys; wave w owns keys
// 32w .. 32w + 31 as two 16-key blocks kb):
//   S, dP  = Q_i K^T, dO_i V^T   A: Q / dO rows (LDS), B: the wave's K / V rows
//   P, dS  = exp2(S c - LSE_i), P (dP - delta_i)           (fp32, masked)
//   dV^T  += dO_i^T P,  dK^T += Q_i^T dS                   A: transposed reads
//   dQ_i  += dS K                                           A: dS^T, B: K^T
// All products are v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 accumulate).  A
// wave skips the 16 x 16 blocks the mask hides entirely, and evaluates the
// mask only in blocks it cuts.
//
// LDS tiles are 64 elements (128 bytes) per row, unpadded, with the 16-byte
// chunks of row r permuted by XOR with f(r) = 2 (r mod 4) + (r / 4 mod 2):
// 8 consecutive rows then put one chunk column on 8 distinct chunk slots
// (conflict-free 16-byte row reads) and 4 aligned rows put 2 adjacent chunks
// on 8 distinct slots (conflict-free transposed reads).
// Transposed operands use ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element (i % 4) of lanes i / 4 + 4e (e = 0..3), so a lane
// pointing at row r0 + i / 4, column c0 + 4 (i % 4) receives rows
// r0 .. r0 + 3 of column c0 + i.
#include "kernels.h"

namespace swa {

namespace {

constexpr int SD = 64;     // head dim
constexpr int STEP = 128;  // keys per kv-step
constexpr int NSLOT = 6;   // ring slots (active q-tiles <= 5 for W <= 128)
constexpr int TROW = 64;   // elements per LDS tile row (128 bytes)

typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
// element offset of (row r, 16-byte chunk ch) in a swizzled tile
__device__ __forceinline__ int tile_off(int r, int ch) { return r * TROW + ((ch ^ swz(r)) << 3); }

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
// r0 + 16 + 4g + (e - 4) of one column, from a precomputed lane offset.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 tr_pair(const T* p) {
  const u32x2 lo = ld_tr4(p);
  const u32x2 hi = ld_tr4(p + 16 * TROW);
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(typename Elem<T>::vec8, r);
}

}  // namespace

template <typename T, bool RELAY>
__global__ __launch_bounds__(kThreads, 1) void bwd_stream_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  __shared__ __align__(16) T sQ[NSLOT][kTile * TROW];
  __shared__ __align__(16) T sdO[NSLOT][kTile * TROW];
  __shared__ __align__(16) float sLse[NSLOT][kTile];
  __shared__ __align__(16) float sDelta[NSLOT][kTile];
  __shared__ __align__(16) T sK[STEP * TROW];
  __shared__ __align__(16) T sdSt[STEP * TROW];  // dS^T [key][q]
  __shared__ int sTicket;

  const Problem& p = a.p;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;

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
  int tr_off[4];  // transposed read: row 4 gq + c / 4, column 16 db + 4 (c % 4)
  {
    const int r = 4 * gq + (c >> 2), f = swz(r);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      tr_off[db] = r * TROW + (((2 * db + ((c & 3) >> 1)) ^ f) << 3) + 4 * (c & 1);
  }
  const int tr_off_w = (4 * gq + (c >> 2)) * TROW +
                       (((2 * w + ((c & 3) >> 1)) ^ swz(4 * gq + (c >> 2))) << 3) + 4 * (c & 1);
  int ds_off[2][2];  // dS^T write: row 32w + 16kb + c, q 32 s2 + 16 hf + 4 gq
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      ds_off[s2][hf] = c * TROW + (((4 * s2 + 2 * hf + (gq >> 1)) ^ swz(c)) << 3) + 4 * (gq & 1);

  // ---- loaders ------------------------------------------------------------
  V8 kB[2][2], vB[2][2], kBn[2][2], vBn[2][2];
  auto load_kv_regs = [&](int j, V8 (&kx)[2][2], V8 (&vx)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = j * STEP + 32 * w + 16 * kb + c;
      const bool ok = key < s.len_kv;
      const int64_t ko = elem_off(p, p.sk, b, s.row0_kv, h, ok ? key : 0);
      const int64_t vo = elem_off(p, p.sv, b, s.row0_kv, h, ok ? key : 0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kx[kb][ks] = ok ? gld8(kp + ko + 32 * ks + 8 * gq) : zero8;
        vx[kb][ks] = ok ? gld8(vp + vo + 32 * ks + 8 * gq) : zero8;
      }
    }
  };
  V8 ktn[4];
  auto load_k_rows = [&](int j) {
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int r = (tid >> 3) + 32 * ps, ch = tid & 7, key = j * STEP + r;
      ktn[ps] = key < s.len_kv ? gld8(kp + elem_off(p, p.sk, b, s.row0_kv, h, key) + 8 * ch) : zero8;
    }
  };
  auto store_k_rows = [&]() {
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int r = (tid >> 3) + 32 * ps, ch = tid & 7;
      *reinterpret_cast<V8*>(&sK[tile_off(r, ch)]) = ktn[ps];
    }
  };
  struct QRegs {
    V8 q[2], o[2];
    float lse, delta;
  };
  auto load_q_tile = [&](int i, QRegs& r) {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int row = (tid >> 3) + 32 * ps, ch = tid & 7, qi = i * kTile + row;
      if (qi < s.len_q) {
        r.q[ps] = gld8(qp + elem_off(p, p.sq, b, s.row0_q, h, qi) + 8 * ch);
        r.o[ps] = gld8(dop + elem_off(p, p.sdo, b, s.row0_q, h, qi) + 8 * ch);
      } else {
        r.q[ps] = zero8;
        r.o[ps] = zero8;
      }
    }
    if (tid < kTile) {
      const int qi = i * kTile + tid;
      if (qi < s.len_q) {
        const int64_t si = s.stat0 + h * s.stat_hs + qi;
        r.lse = a.lse[si] * kLog2e;
        r.delta = a.delta[si];
      } else {
        r.lse = INFINITY;  // exp2(x - inf) = 0: padding rows carry no weight
        r.delta = 0.f;
      }
    }
  };
  auto store_q_tile = [&](int i, const QRegs& r) {
    const int sl = i % NSLOT;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int row = (tid >> 3) + 32 * ps, ch = tid & 7;
      *reinterpret_cast<V8*>(&sQ[sl][tile_off(row, ch)]) = r.q[ps];
      *reinterpret_cast<V8*>(&sdO[sl][tile_off(row, ch)]) = r.o[ps];
    }
    if (tid < kTile) {
      sLse[sl][tid] = r.lse;
      sDelta[sl][tid] = r.delta;
    }
  };

  // ---- accumulators -------------------------------------------------------
  f32x4 dQa[NSLOT][4];         // dQ[q = 16w + 4gq + r][d = 16db + c] per ring slot
  f32x4 dVa[2][4], dKa[2][4];  // dV^T / dK^T[d = 16db + 4gq + r][key = 32w + 16kb + c]
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl)
#pragma unroll
    for (int db = 0; db < 4; ++db) dQa[sl][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < 4; ++db) dVa[kb][db] = dKa[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- dQ of a retiring q-tile ------------------------------------------------
  auto acc_ptr = [&](int i, int r, int db) -> float* {
    const int qi = i * kTile + 16 * w + 4 * gq + r;
    return a.dq_acc + (s.stat0 + h * s.stat_hs + qi) * SD + 16 * db + c;
  };
  auto retire = [&](int i, f32x4 (&acc)[4]) {  // block-uniform arguments
    const int first = g.kv_first(i) / p.chunk, last = g.kv_last(i) / p.chunk;
    if (first == last) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = i * kTile + 16 * w + 4 * gq + r;
        if (qi >= s.cap_q) continue;
        T* row = dqp + elem_off(p, p.sdq, b, s.row0_q, h, qi);
#pragma unroll
        for (int db = 0; db < 4; ++db) row[16 * db + c] = Elem<T>::from_float(p.scale * acc[db][r]);
      }
    } else if (!RELAY) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * w + 4 * gq + r < s.len_q)
#pragma unroll
          for (int db = 0; db < 4; ++db) unsafeAtomicAdd(acc_ptr(i, r, db), acc[db][r]);
    } else if (first == chunk) {
      // first visiting chunk of a boundary tile: turn 0, no wait
      int* semp = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * w + 4 * gq + r < s.cap_q)
#pragma unroll
          for (int db = 0; db < 4; ++db)
            __hip_atomic_exchange(acc_ptr(i, r, db), acc[db][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(semp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // a later turn: stash the partial; it is added in turn order once this
      // chunk has finished its own kv-steps
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i * kTile + 16 * w + 4 * gq + r < s.cap_q)
#pragma unroll
          for (int db = 0; db < 4; ++db) a.dq_stash[acc_ptr(i, r, db) - a.dq_acc] = acc[db][r];
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- prologue -------------------------------------------------------------
  load_kv_regs(j0, kB, vB);
  load_k_rows(j0);
  store_k_rows();
  int loaded_hi = g.q_lo(j0);  // the ring holds q-tiles [.., loaded_hi)
  QRegs pf[2];
  int pf_lo = 0, pf_n = 0;

  for (int j = j0; j < j1; ++j) {
    const int qlo = g.q_lo(j), nit = g.n_iters(j), qhi = qlo + nit;
    if (loaded_hi < qlo) loaded_hi = qlo;
    for (; loaded_hi < qhi; ++loaded_hi) {  // chunk start and gaps only
      QRegs t;
      load_q_tile(loaded_hi, t);
      store_q_tile(loaded_hi, t);
    }
    __syncthreads();  // ring and sK ready

    const bool has_next = j + 1 < j1;
    if (has_next) {
      load_kv_regs(j + 1, kBn, vBn);
      load_k_rows(j + 1);
      const int nlo = g.q_lo(j + 1), nhi = nlo + g.n_iters(j + 1);
      pf_lo = max(loaded_hi, nlo);
      pf_n = max(0, min(2, nhi - pf_lo));
      if (pf_n > 0) load_q_tile(pf_lo, pf[0]);
      if (pf_n > 1) load_q_tile(pf_lo + 1, pf[1]);
    }

    const int kv0 = j * STEP;
    // t(row, key) = row + diag - key; visible iff 0 <= t <= W.  A key past
    // the sequence is pushed out of every window through its lane base.
    int tkey[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kv0 + 32 * w + 16 * kb + c;
      tkey[kb] = key < s.len_kv ? g.diag - key : -(1 << 29);
    }
    const bool keys_ok = kv0 + STEP <= s.len_kv;  // no key past the sequence

#pragma unroll 1
    for (int i = qlo; i < qhi; ++i) {
      const int sl = i % NSLOT, q0 = i * kTile;
      const T* tQ = sQ[sl];
      const T* tO = sdO[sl];
      // wave-uniform t of (row q0, key kv0 + 32w): block (kb, mb) spans t in
      // [u - 15, u + 15] with u = u00 + 16 mb - 16 kb
      const int u00 = q0 + g.diag - (kv0 + 32 * w);
      // S and dP, skipping blocks the mask hides
      f32x4 S[2][4], dP[2][4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) S[kb][mb] = dP[kb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int um = u00 + 16 * mb;
        const bool any0 = um + 15 >= 0 && um - 15 <= W;            // kb = 0
        const bool any1 = um - 16 + 15 >= 0 && um - 16 - 15 <= W;  // kb = 1
        if (!any0 && !any1) continue;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const V8 aq = *reinterpret_cast<const V8*>(tQ + 16 * mb * TROW + rd_off[ks]);
          const V8 ao = *reinterpret_cast<const V8*>(tO + 16 * mb * TROW + rd_off[ks]);
          if (any0) {
            S[0][mb] = mfma16(aq, kB[0][ks], S[0][mb]);
            dP[0][mb] = mfma16(ao, vB[0][ks], dP[0][mb]);
          }
          if (any1) {
            S[1][mb] = mfma16(aq, kB[1][ks], S[1][mb]);
            dP[1][mb] = mfma16(ao, vB[1][ks], dP[1][mb]);
          }
        }
      }
      // P and dS in the accumulator layout (rows 16mb + 4gq + r)
      V8 pP[2][2], pS[2][2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const float4 lse4 = *reinterpret_cast<const float4*>(&sLse[sl][16 * mb + 4 * gq]);
        const float4 del4 = *reinterpret_cast<const float4*>(&sDelta[sl][16 * mb + 4 * gq]);
        const float lsev[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
        const float delv[4] = {del4.x, del4.y, del4.z, del4.w};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int um = u00 + 16 * mb - 16 * kb;
          const bool any = um + 15 >= 0 && um - 15 <= W;
          const bool full = keys_ok && um - 15 >= 0 && um + 15 <= W;
          const int tb = q0 + 16 * mb + 4 * gq + tkey[kb];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float pv = 0.f, dsv = 0.f;
            if (any) {
              float x = S[kb][mb][r] * p.scale_log2 - lsev[r];
              if (!full) x = (unsigned)(tb + r) <= (unsigned)W ? x : -INFINITY;
              pv = fast_exp2(x);
              dsv = pv * (dP[kb][mb][r] - delv[r]);
            }
            pP[kb][mb >> 1][(mb & 1) * 4 + r] = Elem<T>::from_float(pv);
            pS[kb][mb >> 1][(mb & 1) * 4 + r] = Elem<T>::from_float(dsv);
          }
        }
      }
      __syncthreads();  // the previous visit's dQ reads of dS^T are done
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x4 v = __builtin_bit_cast(u32x4, pS[kb][s2]);
          T* base = sdSt + (32 * w + 16 * kb) * TROW;
          *reinterpret_cast<u32x2*>(base + ds_off[s2][0]) = u32x2{v[0], v[1]};
          *reinterpret_cast<u32x2*>(base + ds_off[s2][1]) = u32x2{v[2], v[3]};
        }
      // dV^T += dO^T P, dK^T += Q^T dS  (skip k-steps whose P / dS are zero)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bool use[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int um0 = u00 + 32 * s2 - 16 * kb, um1 = um0 + 16;
          use[kb] = (um0 + 15 >= 0 && um0 - 15 <= W) || (um1 + 15 >= 0 && um1 - 15 <= W);
        }
        if (!use[0] && !use[1]) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const V8 ao = tr_pair(tO + 32 * s2 * TROW + tr_off[db]);
          const V8 aq = tr_pair(tQ + 32 * s2 * TROW + tr_off[db]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (use[kb]) {
              dVa[kb][db] = mfma16(ao, pP[kb][s2], dVa[kb][db]);
              dKa[kb][db] = mfma16(aq, pS[kb][s2], dKa[kb][db]);
            }
        }
      }
      __syncthreads();  // dS^T complete
      // dQ rows 16w .. 16w + 15 of q-tile i += dS K over the step's 128 keys
      const int ud = q0 + 16 * w + g.diag - kv0;  // t of (row 16w, key 0)
      f32x4 dqv[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) dqv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int uk = ud - 32 * ks;  // rows +0..15, keys +0..31: t in [uk - 31, uk + 15]
        if (uk + 15 < 0 || uk - 31 > W) continue;
        const V8 as = tr_pair(sdSt + 32 * ks * TROW + tr_off_w);
#pragma unroll
        for (int db = 0; db < 4; ++db) dqv[db] = mfma16(as, tr_pair(sK + 32 * ks * TROW + tr_off[db]), dqv[db]);
      }
      // add into the slot's register accumulator (a static index per case)
      switch (sl) {
#define SWA_ACC(k)                                                           \
  case k:                                                                    \
    _Pragma("unroll") for (int db = 0; db < 4; ++db) dQa[k][db] += dqv[db]; \
    break;
        SWA_ACC(0) SWA_ACC(1) SWA_ACC(2) SWA_ACC(3) SWA_ACC(4) SWA_ACC(5)
#undef SWA_ACC
      }
    }

    // q-tiles whose last visitor in this chunk was this step
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      const int i = qlo + ((sl - qlo % NSLOT) + NSLOT) % NSLOT;
      if (i < qhi && min(g.kv_last(i), j1 - 1) == j) retire(i, dQa[sl]);
    }
    // dK / dV of this step (zeros if it visited nothing)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kv0 + 32 * w + 16 * kb + c;
      if (key < s.cap_kv) {
        T* dkr = static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, h, key);
        T* dvr = static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, h, key);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          T kx[4], vx[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kx[r] = Elem<T>::from_float(p.scale * dKa[kb][db][r]);
            vx[r] = Elem<T>::from_float(dVa[kb][db][r]);
          }
          *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, kx);
          *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, vx);
        }
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) dVa[kb][db] = dKa[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    __syncthreads();  // ring slots of retired tiles and sK are free
    if (has_next) {
      if (pf_n > 0) store_q_tile(pf_lo, pf[0]);
      if (pf_n > 1) store_q_tile(pf_lo + 1, pf[1]);
      if (pf_n > 0) loaded_hi = max(loaded_hi, pf_lo + pf_n);
      store_k_rows();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          kB[kb][ks] = kBn[kb][ks];
          vB[kb][ks] = vBn[kb][ks];
        }
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
        const int qi = i * kTile + 16 * w + 4 * gq + r;
        if (qi >= s.cap_q) continue;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          float* ap = acc_ptr(i, r, db);
          const float mine = a.dq_stash[ap - a.dq_acc];
          if (turn < nv - 1) {
            __hip_atomic_fetch_add(ap, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            const float old = __hip_atomic_fetch_add(ap, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            dqp[elem_off(p, p.sdq, b, s.row0_q, h, qi) + 16 * db + c] = Elem<T>::from_float(p.scale * (old + mine));
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
      hipLaunchKernelGGL((bwd_stream_kernel<__bf16, true>), dim3(n), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<__bf16, false>), dim3(n), dim3(kThreads), 0, st, a);
  } else {
    if (a.deterministic)
      hipLaunchKernelGGL((bwd_stream_kernel<_Float16, true>), dim3(n), dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<_Float16, false>), dim3(n), dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace swa
