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
// One kv-step of 128 keys runs in two phases with one barrier between them.
//
// Phase 1 (per wave, no barrier): wave w owns keys 16w .. 16w + 15 and walks
// only the 16-row query blocks its window band reaches -- rows
// [key - diag, key + W - diag] of its keys, at most 10 blocks for W <= 128,
// the same count for every wave -- two blocks at a time:
//   S, dP  = Q K^T, dO V^T        A: Q / dO rows (LDS), B: K / V rows (regs)
//   P, dS  = exp2(S c - LSE), P (dP - delta)          (fp32, masked)
//   dV^T  += dO^T P,  dK^T += Q^T dS                  A: transposed LDS reads
// and writes dS^T into its own LDS band: 16 keys x 12 block positions, where
// position 1 + n holds the wave's n-th block and positions 0 and 11 (and
// any position past its last block) hold zeros.
//
// Phase 2 (after the barrier): wave (r, h) = (w mod 4, w / 4) owns rows
// 16 r .. 16 r + 15 of every q-tile the step feeds and head-dim half h, and
// accumulates dQ^T += K^T dS^T over the key pairs whose bands reach those
// rows; the band's zero positions stand in for blocks outside a band, so
// no lane ever branches on the mask.
//
// All products are v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 accumulate).
//
// LDS tiles of Q, dO and K are 64 elements (128 bytes) per row, unpadded,
// with the 16-byte chunks of row r permuted by XOR with (r mod 8).
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT): 16-byte row reads are
// conflict-free in any layout, and this permutation also makes the
// transposed reads conflict-free (a plain 128-byte pitch costs 4x).  Band
// rows are 208 elements apart (416 bytes): the 8 rows one half-wave's
// transposed read touches then fall on 8 disjoint groups of 8 banks.
// Transposed operands use ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element (i % 4) of lanes i / 4 + 4e (e = 0..3), so a lane
// pointing at row r0 + i / 4, column c0 + 4 (i % 4) receives rows
// r0 .. r0 + 3 of column c0 + i.
#include "kernels.h"

namespace swa {

namespace {

constexpr int SD = 64;        // head dim
constexpr int STEP = 128;     // keys per kv-step
constexpr int NSLOT = 5;      // ring slots = most q-tiles one kv-step feeds
constexpr int NACT = 5;       // most q-tiles one kv-step visits (W <= 128)
constexpr int TROW = 64;      // elements per LDS tile row (128 bytes)
constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;
constexpr int NPAIR = 5;      // block pairs a band holds
constexpr int BPOS = 2 * NPAIR + 2;  // band block positions, guards included
constexpr int BP = 208;       // band row pitch (elements), >= 16 * BPOS

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

// 8 contraction values for lane (c, g) from two transposed reads: e < 4 from
// the read at p0, e >= 4 from the read at p1.
template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 tr_two(const T* p0, const T* p1) {
  const u32x2 lo = ld_tr4(p0);
  const u32x2 hi = ld_tr4(p1);
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(typename Elem<T>::vec8, r);
}

template <typename T>
__device__ __forceinline__ u32x2 pack4(float x0, float x1, float x2, float x3) {
  T v[4] = {Elem<T>::from_float(x0), Elem<T>::from_float(x1), Elem<T>::from_float(x2),
            Elem<T>::from_float(x3)};
  return __builtin_bit_cast(u32x2, v);
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
  __shared__ __align__(16) T sBand[NWAVE][16 * BP];  // dS^T [key][block position, row]
  __shared__ int sTicket;

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (scalar)
  const int wr = w & 3, wd = w >> 2;                        // phase 2: rows 16 wr, head-dim half wd

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

  // bands start (and their guard positions stay) zero
  for (int e = tid; e < NWAVE * 16 * BP / 8; e += NTHR) reinterpret_cast<V8*>(&sBand[0][0])[e] = zero8;

  // ---- per-lane LDS offsets (elements) --------------------------------------
  int rd_off[2];  // row read of a 16-row block: row c, chunk 4 ks + gq
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off[ks] = tile_off(c, 4 * ks + gq);
  int tr_off[4];  // transposed read of a 16-row block, columns 16 db ..
#pragma unroll
  for (int db = 0; db < 4; ++db) tr_off[db] = tr_lane_off(c, gq, db);
  // K^T columns of this wave's dQ half (kept out of a runtime-indexed array,
  // which the compiler would place in scratch memory)
  const int tr_off_k0 = tr_lane_off(c, gq, 2 * wd), tr_off_k1 = tr_lane_off(c, gq, 2 * wd + 1);
  const int band_wr = c * BP + 4 * gq;                         // dS^T write: key c, rows 4 gq ..
  const int band_rd = (4 * gq + (c >> 2)) * BP + 4 * (c & 3);  // transposed read
  T* const myband = sBand[w];

  // ---- loaders ------------------------------------------------------------
  // K and V rows of the wave's 16 keys in the MFMA B layout (key c, head-dim
  // 32 ks + 8 gq ..); the K rows are also this wave's share of the LDS K
  // tile.  Rows past the sequence are clamped to a valid row and zeroed
  // when the registers are taken into use.
  V8 kB[2], vB[2], kBn[2], vBn[2];
  auto load_kv = [&](int j, V8 (&kx)[2], V8 (&vx)[2]) {
    const int key = clampi(j * STEP + 16 * w + c, 0, max(s.cap_kv - 1, 0));
    const int64_t ko = elem_off(p, p.sk, b, s.row0_kv, h, key);
    const int64_t vo = elem_off(p, p.sv, b, s.row0_kv, h, key);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kx[ks] = gld8(kp + ko + 32 * ks + 8 * gq);
      vx[ks] = gld8(vp + vo + 32 * ks + 8 * gq);
    }
  };
  auto take_kv = [&](int j, const V8 (&kx)[2], const V8 (&vx)[2]) {
    const bool ok = j * STEP + 16 * w + c < s.len_kv;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kB[ks] = ok ? kx[ks] : zero8;
      vB[ks] = ok ? vx[ks] : zero8;
    }
  };
  struct QRegs {
    V8 q, o;
    float lse, delta;
    int tile;
  };
  // only called for q-tiles the schedule visits, so the sequence has rows
  auto load_q_tile = [&](int i, QRegs& r) {
    r.tile = i;
    const int row = tid >> 3, ch = tid & 7, qi = min(i * kTile + row, s.len_q - 1);
    r.q = gld8(qp + elem_off(p, p.sq, b, s.row0_q, h, qi) + 8 * ch);
    r.o = gld8(dop + elem_off(p, p.sdo, b, s.row0_q, h, qi) + 8 * ch);
    if (tid < kTile) {
      const int64_t si = s.stat0 + h * s.stat_hs + min(i * kTile + tid, s.len_q - 1);
      r.lse = a.lse[si];
      r.delta = a.delta[si];
    }
  };
  auto store_q_tile = [&](const QRegs& r) {
    const int sl = r.tile % NSLOT, row = tid >> 3, ch = tid & 7;
    const bool ok = r.tile * kTile + row < s.len_q;
    *reinterpret_cast<V8*>(&sQ[sl][tile_off(row, ch)]) = ok ? r.q : zero8;
    *reinterpret_cast<V8*>(&sdO[sl][tile_off(row, ch)]) = ok ? r.o : zero8;
    if (tid < kTile) {
      const bool okr = r.tile * kTile + tid < s.len_q;
      // exp2(x - inf) = 0: padding rows carry no weight
      sLse[sl][tid] = okr ? r.lse * kLog2e : INFINITY;
      sDelta[sl][tid] = okr ? r.delta : 0.f;
    }
  };

  // ---- accumulators -------------------------------------------------------
  // dQ^T of q-tile q_lo(j) + k in dQa[k][e]: head-dim 16 (2 wd + e) + 4 gq + r,
  // row 16 wr + c; shifted down when q_lo advances between kv-steps
  f32x4 dQa[NACT][2];
  f32x4 dVa[4], dKa[4];  // dV^T / dK^T[d = 16db + 4gq + r][key = 16w + c]
#pragma unroll
  for (int k = 0; k < NACT; ++k) dQa[k][0] = dQa[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) dVa[db] = dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- dQ of a retiring q-tile ------------------------------------------------
  auto q_row = [&](int i) { return i * kTile + 16 * wr + c; };
  auto acc_ptr = [&](int i, int e) -> float* {  // 4 consecutive head-dim values
    return a.dq_acc + (s.stat0 + h * s.stat_hs + q_row(i)) * SD + 16 * (2 * wd + e) + 4 * gq;
  };
  auto retire = [&](int i, f32x4 (&acc)[2]) {  // block-uniform arguments
    const int first = g.kv_first(i) / p.chunk, last = g.kv_last(i) / p.chunk;
    const int qi = q_row(i);
    if (first == last) {
      if (qi < s.cap_q) {
        T* row = dqp + elem_off(p, p.sdq, b, s.row0_q, h, qi) + 32 * wd + 4 * gq;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          *reinterpret_cast<u32x2*>(row + 16 * e) =
              pack4<T>(p.scale * acc[e][0], p.scale * acc[e][1], p.scale * acc[e][2], p.scale * acc[e][3]);
      }
    } else if (!RELAY) {
      if (qi < s.len_q)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) unsafeAtomicAdd(acc_ptr(i, e) + r, acc[e][r]);
    } else if (first == chunk) {
      // first visiting chunk of a boundary tile: turn 0, no wait
      int* semp = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles + i;
      if (qi < s.cap_q)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            __hip_atomic_exchange(acc_ptr(i, e) + r, acc[e][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(semp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // a later turn: stash the partial; it is added in turn order once this
      // chunk has finished its own kv-steps
      if (qi < s.cap_q)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          *reinterpret_cast<f32x4*>(a.dq_stash + (acc_ptr(i, e) - a.dq_acc)) = acc[e];
    }
    acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- band geometry ----------------------------------------------------------
  // 16-row blocks that keys kv0 + 16 v .. + 15 see: rows t = row + diag - key
  // in [0, W]; clipped to the step's q-tiles; empty past the keys.
  auto band_lo = [&](int kv0, int v, int qlo) {
    return max(floor_div(kv0 + 16 * v - g.diag, 16), 4 * qlo);
  };
  auto band_hi = [&](int kv0, int v, int qhi) {
    if (kv0 + 16 * v >= s.len_kv) return INT32_MIN / 2;
    return min(floor_div(kv0 + 16 * v + 15 + W - g.diag, 16), 4 * qhi - 1);
  };

  // ---- prologue -------------------------------------------------------------
  load_kv(j0, kBn, vBn);
  take_kv(j0, kBn, vBn);
  int loaded_hi = g.q_lo(j0);  // the ring holds q-tiles [.., loaded_hi)
  int acc_lo = g.q_lo(j0);     // q-tile held in dQa[0]
  QRegs pf[2];

  for (int j = j0; j < j1; ++j) {
    const int qlo = g.q_lo(j), nit = min(g.n_iters(j), NACT), qhi = qlo + nit;
    if (loaded_hi < qlo) loaded_hi = qlo;
    for (; loaded_hi < qhi; ++loaded_hi) {  // chunk start and gaps only
      QRegs t;
      load_q_tile(loaded_hi, t);
      store_q_tile(t);
    }
    __syncthreads();  // T: ring ready; sK and the bands are free
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<V8*>(&sK[tile_off(16 * w + c, 4 * ks + gq)]) = kB[ks];
    for (; acc_lo < qlo; ++acc_lo) {  // realign dQa[0] with q_lo(j)
#pragma unroll
      for (int k = 0; k + 1 < NACT; ++k) {
        dQa[k][0] = dQa[k + 1][0];
        dQa[k][1] = dQa[k + 1][1];
      }
      dQa[NACT - 1][0] = dQa[NACT - 1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // prefetch of the next kv-step: K / V rows and its new q-tiles
    const bool has_next = j + 1 < j1;
    int pf_n = 0;
    if (has_next) {
      load_kv(j + 1, kBn, vBn);
      const int nlo = g.q_lo(j + 1), nhi = nlo + min(g.n_iters(j + 1), NACT);
      const int pf_lo = max(loaded_hi, nlo);
      pf_n = max(0, min(2, nhi - pf_lo));
      if (pf_n > 0) load_q_tile(pf_lo, pf[0]);
      if (pf_n > 1) load_q_tile(pf_lo + 1, pf[1]);
    }

    // ---- phase 1: this wave's band --------------------------------------------
    const int kv0 = j * STEP;
    // t(row, key) = row + diag - key; visible iff 0 <= t <= W.  A key past
    // the sequence is pushed out of every window through its lane base.
    const int keyl = kv0 + 16 * w + c;
    const int tkey = keyl < s.len_kv ? g.diag - keyl : -(1 << 29);
    const int blo = band_lo(kv0, w, qlo), bhi = band_hi(kv0, w, qhi);
    const int npairs = min(max(bhi - blo + 2, 0) >> 1, NPAIR);
    for (int pr = 0; pr < npairs; ++pr) {
      const int b0 = blo + 2 * pr;
      const bool has1 = b0 + 1 <= bhi;
      const int b1 = has1 ? b0 + 1 : b0;  // a valid block either way
      const int sl0 = (b0 >> 2) % NSLOT, sl1 = (b1 >> 2) % NSLOT;
      const T* q0 = sQ[sl0] + 16 * (b0 & 3) * TROW;
      const T* o0 = sdO[sl0] + 16 * (b0 & 3) * TROW;
      const T* q1 = sQ[sl1] + 16 * (b1 & 3) * TROW;
      const T* o1 = sdO[sl1] + 16 * (b1 & 3) * TROW;
      f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, D0 = S0, S1 = S0, D1 = S0;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        S0 = mfma16(*reinterpret_cast<const V8*>(q0 + rd_off[ks]), kB[ks], S0);
        D0 = mfma16(*reinterpret_cast<const V8*>(o0 + rd_off[ks]), vB[ks], D0);
      }
      if (has1) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          S1 = mfma16(*reinterpret_cast<const V8*>(q1 + rd_off[ks]), kB[ks], S1);
          D1 = mfma16(*reinterpret_cast<const V8*>(o1 + rd_off[ks]), vB[ks], D1);
        }
      }
      float pv[8], dsv[8];
      {
        const int r0 = 16 * (b0 & 3) + 4 * gq, r1 = 16 * (b1 & 3) + 4 * gq;
        const float4 lse0 = *reinterpret_cast<const float4*>(&sLse[sl0][r0]);
        const float4 del0 = *reinterpret_cast<const float4*>(&sDelta[sl0][r0]);
        const float4 lse1 = *reinterpret_cast<const float4*>(&sLse[sl1][r1]);
        const float4 del1 = *reinterpret_cast<const float4*>(&sDelta[sl1][r1]);
        const float lsev[8] = {lse0.x, lse0.y, lse0.z, lse0.w, lse1.x, lse1.y, lse1.z, lse1.w};
        const float delv[8] = {del0.x, del0.y, del0.z, del0.w, del1.x, del1.y, del1.z, del1.w};
        const float sv[8] = {S0[0], S0[1], S0[2], S0[3], S1[0], S1[1], S1[2], S1[3]};
        const float dv[8] = {D0[0], D0[1], D0[2], D0[3], D1[0], D1[1], D1[2], D1[3]};
        const int tb0 = 16 * b0 + 4 * gq + tkey;
        // block 1 is masked out entirely when it is past the band
        const int tb1 = has1 ? 16 * b1 + 4 * gq + tkey : -(1 << 29);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = (r < 4 ? tb0 : tb1) + (r & 3);
          const float x = sv[r] * p.scale_log2 - lsev[r];
          pv[r] = (unsigned)t <= (unsigned)W ? fast_exp2(x) : 0.f;
          dsv[r] = pv[r] * (dv[r] - delv[r]);
        }
      }
      const u32x2 p0 = pack4<T>(pv[0], pv[1], pv[2], pv[3]), p1 = pack4<T>(pv[4], pv[5], pv[6], pv[7]);
      const u32x2 s0 = pack4<T>(dsv[0], dsv[1], dsv[2], dsv[3]);
      const u32x2 s1 = pack4<T>(dsv[4], dsv[5], dsv[6], dsv[7]);
      const V8 pP = __builtin_bit_cast(V8, u32x4{p0[0], p0[1], p1[0], p1[1]});
      const V8 pS = __builtin_bit_cast(V8, u32x4{s0[0], s0[1], s1[0], s1[1]});
      // dS^T of blocks b0, b1 at band positions 2 pr + 1, 2 pr + 2
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 1)) = s0;
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 2)) = s1;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dVa[db] = mfma16(tr_two(o0 + tr_off[db], o1 + tr_off[db]), pP, dVa[db]);
        dKa[db] = mfma16(tr_two(q0 + tr_off[db], q1 + tr_off[db]), pS, dKa[db]);
      }
    }
    for (int pr = npairs; pr < NPAIR; ++pr) {  // positions past the band
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 1)) = u32x2{0u, 0u};
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 2)) = u32x2{0u, 0u};
    }

    __syncthreads();  // A: bands and sK complete; ring slots of tiles before q_lo(j + 1) free
    if (pf_n > 0) store_q_tile(pf[0]);
    if (pf_n > 1) store_q_tile(pf[1]);
    loaded_hi += pf_n;

    // ---- phase 2: dQ^T += K^T dS^T ------------------------------------------
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int wa = 2 * ks, wb = 2 * ks + 1;
      const int lo_a = band_lo(kv0, wa, qlo), hi_a = band_hi(kv0, wa, qhi);
      const int lo_b = band_lo(kv0, wb, qlo), hi_b = band_hi(kv0, wb, qhi);
      if (hi_a < lo_a && hi_b < lo_b) continue;
      const T* kr = sK + 32 * ks * TROW;
      const V8 kt0 = tr_two(kr + tr_off_k0, kr + 16 * TROW + tr_off_k0);
      const V8 kt1 = tr_two(kr + tr_off_k1, kr + 16 * TROW + tr_off_k1);
#pragma unroll
      for (int k = 0; k < NACT; ++k) {
        if (k >= nit) break;
        const int bb = 4 * (qlo + k) + wr;
        if (!((bb >= lo_a && bb <= hi_a) || (bb >= lo_b && bb <= hi_b))) continue;
        const int pa = clampi(bb - lo_a + 1, 0, BPOS - 1), pb = clampi(bb - lo_b + 1, 0, BPOS - 1);
        const V8 st = tr_two(sBand[wa] + band_rd + 16 * pa, sBand[wb] + band_rd + 16 * pb);
        dQa[k][0] = mfma16(kt0, st, dQa[k][0]);
        dQa[k][1] = mfma16(kt1, st, dQa[k][1]);
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
        *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * gq) =
            pack4<T>(p.scale * dKa[db][0], p.scale * dKa[db][1], p.scale * dKa[db][2], p.scale * dKa[db][3]);
        *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * gq) = pack4<T>(dVa[db][0], dVa[db][1], dVa[db][2], dVa[db][3]);
      }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) dVa[db] = dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (has_next) take_kv(j + 1, kBn, vBn);
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
      const int qi = q_row(i);
      if (qi < s.cap_q) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float* ap = acc_ptr(i, e);
          const f32x4 mine = *reinterpret_cast<const f32x4*>(a.dq_stash + (ap - a.dq_acc));
          float out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float old = __hip_atomic_fetch_add(ap + r, mine[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            out[r] = p.scale * (old + mine[r]);
          }
          if (turn == nv - 1)
            *reinterpret_cast<u32x2*>(dqp + elem_off(p, p.sdq, b, s.row0_q, h, qi) + 16 * (2 * wd + e) + 4 * gq) =
                pack4<T>(out[0], out[1], out[2], out[3]);
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
