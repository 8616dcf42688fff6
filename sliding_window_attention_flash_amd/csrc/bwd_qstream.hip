// bwd_qstream: the backward for short windows at head_dim 128 (GQA or MHA)
// in one pass over query rows (gfx950).
//
// The rows of a 32-row q-step see at most 32 + W keys, four 32-key tiles for
// W <= 96: kv-tiles i + d - 3 .. i + d for q-step i, with d = diag / 32 (the
// plan takes this kernel only when diag is a multiple of 32, causal with no
// right band, W <= 96, dense sequences).  One block of 8 waves (one
// per CU) walks a chunk of consecutive q-steps of one (sequence, kv head);
// for each q-step it takes the G query heads of the group in turn, one step
// each.  The four kv-tiles of the window stay in a ring: K and V rows in
// registers (B operands of S = Q K^T and dP = dO V^T), K in LDS (A operand of
// dQ^T = K^T dS^T), and their dK^T / dV^T accumulate in registers across
// every q-step and head that sees them.  So Q, dO and O are read once, each
// step's dQ is complete within the step, and each kv-tile's dK / dV leave
// once the window has passed it.
//
// Waves: wave w owns keys 16 (w % 2) .. + 15 of ring slot w / 2 (slot of
// kv-tile j: j mod 4).  A step s (q-step i, head h), with its Q / dO / O
// rows already in LDS buffer s mod 4:
//   T  this wave's loads of step s + 1's rows have landed; barrier; at a
//      q-step's first head the slot entering the ring stores its K rows to
//      LDS.
//   1  every wave, for its 16 keys and the 32 rows: S = Q K^T, dP = dO V^T,
//      P = exp2(S c - LSE), dS = P (dP - delta) (masked), dV^T += dO^T P,
//      dK^T += Q^T dS, dS^T to LDS.
//   A  barrier: dS^T complete.
//   2  after a q-step's last head the oldest slot's waves retire their
//      kv-tile and load the entering one; every wave forms delta of step
//      s + 1's rows, computes 16 rows x 32 head-dim columns of dQ, starts
//      the loads of step s + 3 (straight into LDS buffer (s + 3) mod 4),
//      puts its dQ block into the step's LDS tile and last stores 4 whole
//      rows of the previous step's tile, so that those loads and that store
//      are the only operations the wait before the next barrier T leaves in
//      flight.
// The kv-tiles a chunk shares with its neighbours leave as fp32 partial
// sums; bwd_qstream_fix adds the two sides in a fixed order, so the whole
// pass is bitwise repeatable.
//
// All products are v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 accumulate),
// with the lane layouts and swizzled 128-wide LDS rows of the per-tile
// kernels.

#include "kernels.h"
#include "tiles.h"

namespace swa {

namespace {

constexpr int QD = 128;              // head dim
constexpr int QNS = QD / 32;         // k-steps over the head dim
constexpr int QNDB = QD / 16;        // 16-column blocks of the head dim
constexpr int QCH = QD / 8;          // 16-byte chunks per row
constexpr int QR = 32;               // rows of a q-step
constexpr int QK = 32;               // keys of a ring tile
constexpr int QSLOT = 4;             // ring tiles (W <= 96)
constexpr int QWAVE = 2 * QSLOT;     // 16 keys per wave
constexpr int QTHR = 64 * QWAVE;
constexpr int QROWS = QR * QD;       // elements of a step's Q (or dO, O) rows
constexpr int DSP = QR + 8;          // dS^T row pitch (elements): 80 bytes
constexpr int QPART = QK * 2 * QD;   // floats of one kv-tile's dK / dV partial
constexpr int QPIECES = 3 * QROWS * 2 / 1024;  // 1 KB pieces of a step's Q, dO, O
constexpr int kWaitVm4 = 0xF74;      // s_waitcnt vmcnt(4) (no LDS / export wait)
constexpr int kWaitVm0 = 0xF70;      // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0)

static_assert(QPIECES % QWAVE == 0, "a step's rows stream in whole pieces per wave");
static_assert(QPIECES / QWAVE == 3, "the wait at a step's top leaves the last step's 3 pieces and 1 store in flight");
static_assert(QR * QCH == QTHR, "each thread stores one 16-byte chunk of a step's dQ (4 whole rows per wave)");

// A barrier for LDS only: this wave's LDS accesses are complete, then
// s_barrier.  (__syncthreads also orders global memory, which here would
// make every barrier wait for the rows streaming in for later steps.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
}

// Sum over the 16 lanes of a row (DPP: swaps within quads, then the mirrors
// of each half-row and of the row).
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}
static_assert(QSLOT * QK >= QR + 96, "the ring holds the keys of a q-step for W <= 96");

}  // namespace

template <typename T>
__global__ __launch_bounds__(QTHR, 1) void bwd_qstream_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  // Per step buffer (four, used in turn; separately named, so that reading
  // one is no reason to wait for the loads streaming into another): Q then
  // dO rows, O rows, and row statistics (LSE in log2 units, then delta).
  // The ring's K tiles; dS^T [key][row].
  __shared__ __align__(16) T sQO0[2 * QROWS];
  __shared__ __align__(16) T sQO1[2 * QROWS];
  __shared__ __align__(16) T sQO2[2 * QROWS];
  __shared__ __align__(16) T sQO3[2 * QROWS];
  __shared__ __align__(16) T sO0[QROWS];
  __shared__ __align__(16) T sO1[QROWS];
  __shared__ __align__(16) T sO2[QROWS];
  __shared__ __align__(16) T sO3[QROWS];
  __shared__ __align__(16) float sLD0[2 * QR];
  __shared__ __align__(16) float sLD1[2 * QR];
  __shared__ __align__(16) float sLD2[2 * QR];
  __shared__ __align__(16) float sLD3[2 * QR];
  __shared__ __align__(16) T sK[QSLOT * QK * QD];
  __shared__ __align__(16) T sdSt[QSLOT * QK * DSP];
  // dQ of a step on its way out (two, used in turn): the 8 waves' blocks
  // meet here so that each wave stores 4 whole rows
  __shared__ __align__(16) T sDQ0[QROWS];
  __shared__ __align__(16) T sDQ1[QROWS];

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = w >> 1, wk = w & 1;
  if (blockIdx.x == 0 && tid < 2) a.ctl[tid] = 0;  // no relay runs: no ticket, no expiry
  const int nch = p.qs_nch, C = p.qs_chunk, G = p.G;
  const int chunk = blockIdx.x % nch, bh = blockIdx.x / nch;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const Seq s = load_seq(p, b);
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, 1, p.window, 0, QR, QK);
  const int nqt = g.n_q_tiles, nkt = g.n_kv_tiles;
  const int i0 = chunk * C, i1 = min(i0 + C, nqt);
  if (i0 >= i1) return;
  const int dq = g.diag / QK;  // the plan checked diag % 32 == 0
  const int W = p.window;      // 0 <= W <= 96
  // Row 0 of this (sequence, kv head) in K, V, dK, dV, and of this
  // sequence in dQ, with the row (and dQ's head) strides: formed once, so
  // that the loop keeps a few scalars instead of every tensor's strides.
  const T* const k_row0 = static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, hk, 0);
  const T* const v_row0 = static_cast<const T*>(a.v) + elem_off(p, p.sv, b, s.row0_kv, hk, 0);
  T* const dk_row0 = static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, hk, 0);
  T* const dv_row0 = static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, hk, 0);
  T* const dq_row0 = static_cast<T*>(a.dq) + elem_off(p, p.sdq, b, s.row0_q, 0, 0);
  const int64_t k_rs = p.sk[2], v_rs = p.sv[2], dk_rs = p.sdk[2], dv_rs = p.sdv[2], dq_rs = p.sdq[2],
                dq_hs = p.sdq[1];
  const float* const lse0p = a.lse + s.stat0;
  // kv-tile in ring slot sl while q-step i runs: the one of i + dq - 3 ..
  // i + dq congruent to sl mod 4 (outside [0, nkt): a hole)
  auto slot_tile = [&](int sl, int i) { return i + dq - 3 + ((sl - (i + dq - 3)) & 3); };

  V8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = Elem<T>::from_float(0.f);

  // per-lane LDS offsets (elements), as in the per-tile kernels
  int rd_off[QNS], tr_off[QNDB];
#pragma unroll
  for (int st = 0; st < QNS; ++st) rd_off[st] = toff<QD>(c, 4 * st + gq);
#pragma unroll
  for (int db = 0; db < QNDB; ++db) tr_off[db] = troff<QD>(c, gq, db);
  // dS^T: this lane's key row of its slot, and the transposed read of phase 2
  // (lane c of a 16-lane group points at key 4 gq + c / 4, rows 4 (c % 4) ..;
  // it receives keys 4 gq .. + 3 of row c)
  T* const my_ds = sdSt + (slot * QK + 16 * wk + c) * DSP + 4 * gq;
  int ds_rd = (4 * gq + (c >> 2)) * DSP + 4 * (c & 3);
  int kst_off[QNS];  // this lane's K chunks in its slot's LDS tile
#pragma unroll
  for (int st = 0; st < QNS; ++st) kst_off[st] = toff<QD>(16 * wk + c, 4 * st + gq);
  int fd_row = tid >> 4, fd_off = toff<QD>(tid >> 4, tid & 15);  // delta: row and chunk of this lane
  int g4 = 4 * gq, lq = l;

  // ---- the ring: this wave's 16 keys of its slot's kv-tile -------------------
  V8 kB[QNS], vB[QNS];
  f32x4 dK[QNDB], dV[QNDB];
  int my_j = -1;  // kv-tile held (wave-uniform)
  auto load_keys = [&](int j) {
    my_j = j;
    const int key = j * QK + 16 * wk + c;
    const bool ok = j >= 0 && j < nkt && key < s.len_kv;
    const int kr = clampi(key, 0, max(s.len_kv - 1, 0));
    const T* krow = row_at(k_row0, kr, k_rs) + 8 * gq;
    const T* vrow = row_at(v_row0, kr, v_rs) + 8 * gq;
#pragma unroll
    for (int st = 0; st < QNS; ++st) {
      kB[st] = ok ? ld8(krow + 32 * st) : zero8;
      vB[st] = ok ? ld8(vrow + 32 * st) : zero8;
    }
#pragma unroll
    for (int db = 0; db < QNDB; ++db) dK[db] = dV[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_k_rows = [&]() {  // this wave's K rows into its slot's LDS tile
    T* kt = sK + slot * QK * QD;
#pragma unroll
    for (int st = 0; st < QNS; ++st) *reinterpret_cast<V8*>(&kt[kst_off[st]]) = kB[st];
  };
  // dK = scale dS^T Q, dV = P^T dO of kv-tile my_j: straight out when every
  // q-step that sees it is in this chunk, else as one side's fp32 partial
  auto retire = [&]() {
    const int j = my_j;
    if (j < 0 || j >= nkt) return;
    const int key = j * QK + 16 * wk + c;
    const int lo = g.q_lo(j), hi = lo + g.n_iters(j);
    if (lo >= i0 && hi <= i1) {
      if (key < s.cap_kv) {
        T* dkp = row_at(dk_row0, key, dk_rs) + 4 * gq;
        T* dvp = row_at(dv_row0, key, dv_rs) + 4 * gq;
#pragma unroll
        for (int db = 0; db < QNDB; ++db) {
          T kx[4], vx[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kx[r] = Elem<T>::from_float(p.scale * dK[db][r]);
            vx[r] = Elem<T>::from_float(dV[db][r]);
          }
          *reinterpret_cast<u32x2*>(dkp + 16 * db) = __builtin_bit_cast(u32x2, kx);
          *reinterpret_cast<u32x2*>(dvp + 16 * db) = __builtin_bit_cast(u32x2, vx);
        }
      }
    } else {
      // boundary k between chunks k - 1 and k: tile t = j - (k C + dq - 3)
      // (0 .. 2); side 0 from the earlier chunk, 1 from the later
      const int later = lo < i0;
      const int k = later ? chunk : chunk + 1;
      const int t = j - (k * C + dq - 3);
      float* part = a.dq_acc + ((((int64_t)bh * nch + k) * 3 + t) * 2 + later) * QPART + (16 * wk + c) * 2 * QD;
#pragma unroll
      for (int db = 0; db < QNDB; ++db) {
        *reinterpret_cast<f32x4*>(part + 16 * db + 4 * gq) = dK[db];
        *reinterpret_cast<f32x4*>(part + QD + 16 * db + 4 * gq) = dV[db];
      }
    }
  };

  // ---- a step's rows -------------------------------------------------------
  // Q / dO / O of (q-step i, head h): 24 pieces of 1 KB (4 rows each), 3 per
  // wave, straight into LDS; lane l fills bytes 16 l of a piece: row
  // 4 pr + l / 16, stored chunk l % 16, which holds logical chunk
  // (l % 16) ^ tsw(row).  Rows past the sequence repeat its last row.
  // A wave's pieces always come from the same tensors: their sequence base
  // and strides are picked once, by value (a pointer into the kernel
  // arguments chosen at run time would cost a scalar load, and a wait on
  // every outstanding LDS access, per piece and step).
  constexpr int QPW = QPIECES / QWAVE;  // pieces per wave
  const T* pc_base[QPW];
  int64_t pc_hs[QPW], pc_rs[QPW];
#pragma unroll
  for (int k = 0; k < QPW; ++k) {
    const int ten = (QPW * w + k) >> 3;
    const T* base = static_cast<const T*>(ten == 0 ? a.q : (ten == 1 ? a.dO : a.o));
    const int64_t s0 = ten == 0 ? p.sq[0] : (ten == 1 ? p.sdo[0] : p.so[0]);
    pc_hs[k] = ten == 0 ? p.sq[1] : (ten == 1 ? p.sdo[1] : p.so[1]);
    pc_rs[k] = ten == 0 ? p.sq[2] : (ten == 1 ? p.sdo[2] : p.so[2]);
    pc_base[k] = base + (p.layout == LAYOUT_THD ? s.row0_q * pc_rs[k] : (int64_t)b * s0);
  }
  auto stream_rows = [&](int i, int h, T* qo, T* ob) {
#pragma unroll
    for (int k = 0; k < QPW; ++k) {
      const int pc = QPW * w + k, ten = pc >> 3, pr = pc & 7;
      const int row = 4 * pr + (l >> 4), ch = (l & 15) ^ tsw<QD>(row);
      const int gr = min(i * QR + row, s.len_q - 1);
      T* dst = ten == 2 ? ob : qo + ten * QROWS;
      ld16_to_lds(row_at(pc_base[k] + h * pc_hs[k], gr, pc_rs[k]) + 8 * ch, dst + pr * 512);
    }
  };
  auto load_lse = [&](int i, int h) {  // wave 0, lane l < 32: row l
    return lse0p[h * s.stat_hs + min(i * QR + (l & 31), s.len_q - 1)];
  };
  // With a sink: wave 0 adds the step's 32 terms exp(sink_h - LSE) delta
  // (zero past the sequence: LSE +inf there, delta 0) in a fixed order and
  // writes the step's dSink partial
  // (lane g of every wave holds the group's g-th sink logit in log2 units;
  // the plan takes this kernel with a sink only for groups of up to 64 heads)
  const float sink_l = p.has_sink && l < G ? a.sink[hk * G + l] * kLog2e : 0.f;
  auto sink_partial = [&](int i, int g, const float* ld) {
    const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sink_l), g));
    const int h = hk * G + g;
    float t = lq < QR ? fast_exp2(s2 - ld[lq]) * ld[QR + lq] : 0.f;
#pragma unroll
    for (int off = QR / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off);
    if (lq == 0) a.sink_part[((int64_t)h * p.B + b) * p.sink_tiles + i] = t;
  };
  auto store_lse = [&](int i, float v, float* ld) {
    if (w == 0 && lq < QR) ld[lq] = i * QR + lq < s.len_q ? v * kLog2e : INFINITY;  // padding rows: P = 0
  };
  // delta of the step's rows from its dO (in qo) and O (in ob): 16 lanes per
  // row, one 16-byte chunk each
  auto form_delta = [&](int i, const T* qo, const T* ob, float* ld) {
    const int row = fd_row, ch = tid & 15;
    const V8 x = *reinterpret_cast<const V8*>(&qo[QROWS + fd_off]);
    const V8 y = *reinterpret_cast<const V8*>(&ob[fd_off]);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += Elem<T>::to_float(x[k]) * Elem<T>::to_float(y[k]);
    acc = row16_sum(acc);
    if (ch == 0) ld[QR + row] = i * QR + row < s.len_q ? acc : 0.f;
  };

  // Mask: t = row + diag - key must lie in [0, W]; a key past the sequence
  // is pushed out of reach through its lane term, and rows past the
  // sequence carry LSE = +inf.
  const unsigned trange = (unsigned)W;

  // Phase 1 for this wave's keys: the 32 rows of q-step i in (qo, ld).
  // Both 16-row blocks are computed (the mask zeroes what no row sees), so
  // the products form one straight run, with each operand read one product
  // ahead; a hole only writes zeros into its dS^T (phase 2 reads every
  // slot).
  auto phase1 = [&](int i, const T* qo, const float* ld) {
    const int j = my_j;
    if (j < 0 || j >= nkt) {
      const u32x2 z = {0u, 0u};
      *reinterpret_cast<u32x2*>(my_ds) = z;
      *reinterpret_cast<u32x2*>(my_ds + 16) = z;
      return;
    }
    const T* sQ = qo;
    const T* sdO = qo + QROWS;
    const int key = j * QK + 16 * wk + c;
    const int tkey = key < s.len_kv ? g.diag - key : -(1 << 30);  // t = row + tkey
    const int q0 = i * QR;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 S[2] = {zero4, zero4}, dP[2] = {zero4, zero4};
    V8 aq[2][2], ao[2][2];  // [k-step parity][16-row block]: one k-step ahead
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      aq[0][mb] = *reinterpret_cast<const V8*>(&sQ[16 * mb * QD + rd_off[0]]);
      ao[0][mb] = *reinterpret_cast<const V8*>(&sdO[16 * mb * QD + rd_off[0]]);
    }
#pragma unroll
    for (int st = 0; st < QNS; ++st) {
      if (st + 1 < QNS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          aq[(st + 1) & 1][mb] = *reinterpret_cast<const V8*>(&sQ[16 * mb * QD + rd_off[st + 1]]);
          ao[(st + 1) & 1][mb] = *reinterpret_cast<const V8*>(&sdO[16 * mb * QD + rd_off[st + 1]]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        S[mb] = mfma16(aq[st & 1][mb], kB[st], S[mb]);
        dP[mb] = mfma16(ao[st & 1][mb], vB[st], dP[mb]);
      }
    }
    V8 to[2], tq[2];  // the transposed operands, one 16-column block ahead
    to[0] = trpair(&sdO[tr_off[0]], &sdO[16 * QD + tr_off[0]]);
    tq[0] = trpair(&sQ[tr_off[0]], &sQ[16 * QD + tr_off[0]]);
    V8 pP, pS;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&ld[16 * mb + g4]);
      const f32x4 del4 = *reinterpret_cast<const f32x4*>(&ld[QR + 16 * mb + g4]);
      const int tb = q0 + 16 * mb + 4 * gq + tkey;
      T sk[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = S[mb][r] * p.scale_log2 - lse4[r];
        asm("" : "+v"(x));
        const float pv = fast_exp2((unsigned)(tb + r) <= trange ? x : -INFINITY);
        const float dsv = pv * (dP[mb][r] - del4[r]);
        sk[r] = Elem<T>::from_float(dsv);
        pP[mb * 4 + r] = Elem<T>::from_float(pv);
        pS[mb * 4 + r] = sk[r];
      }
      // dS^T [key][row] for the dQ of phase 2 (zeros where unseen)
      *reinterpret_cast<u32x2*>(my_ds + 16 * mb) = __builtin_bit_cast(u32x2, sk);
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the 32 rows
#pragma unroll
    for (int db = 0; db < QNDB; ++db) {
      if (db + 1 < QNDB) {
        to[(db + 1) & 1] = trpair(&sdO[tr_off[db + 1]], &sdO[16 * QD + tr_off[db + 1]]);
        tq[(db + 1) & 1] = trpair(&sQ[tr_off[db + 1]], &sQ[16 * QD + tr_off[db + 1]]);
      }
      dV[db] = mfma16(to[db & 1], pP, dV[db]);
      dK[db] = mfma16(tq[db & 1], pS, dK[db]);
    }
  };

  // Phase 2: dQ^T of rows 16 rb .. + 15 of q-step i, head h, head-dim
  // columns 32 dq4 .. + 31, over the ring's tiles that see the rows
  const int rb = w & 1, dq4 = w >> 1;
  int tr_dq[2] = {troff<QD>(c, gq, 2 * dq4), troff<QD>(c, gq, 2 * dq4 + 1)};  // (dq4 varies by wave)
  // The lane offsets above are made opaque at the top of every step: left
  // loop-invariant, the compiler would keep a precomputed copy of each for
  // every LDS buffer of the unrolled loop (dozens of registers) instead of
  // folding the buffer into the instructions' offset field.
  auto refresh_offsets = [&]() {
#pragma unroll
    for (int st = 0; st < QNS; ++st) {
      asm volatile("" : "+v"(rd_off[st]));
      asm volatile("" : "+v"(kst_off[st]));
    }
#pragma unroll
    for (int db = 0; db < QNDB; ++db) asm volatile("" : "+v"(tr_off[db]));
    asm volatile("" : "+v"(tr_dq[0]), "+v"(tr_dq[1]), "+v"(ds_rd), "+v"(fd_row), "+v"(fd_off), "+v"(g4), "+v"(lq));
  };
  auto phase2_dq = [&](f32x4 (&dQt)[2]) {
    dQt[0] = dQt[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // every slot (its dS^T is zero where its keys do not see these rows, and
    // a hole's K rows are zeros); slot m + 1's operands are read while slot
    // m's products run
    V8 as[2], ak[2][2];
    auto read = [&](int m, int x) {
      const T* dsb = sdSt + m * QK * DSP + 16 * rb + ds_rd;
      as[x] = trpair(dsb, dsb + 16 * DSP);
      const T* kt = sK + m * QK * QD;
#pragma unroll
      for (int e = 0; e < 2; ++e) ak[x][e] = trpair(&kt[tr_dq[e]], &kt[16 * QD + tr_dq[e]]);
    };
    read(0, 0);
#pragma unroll
    for (int m = 0; m < QSLOT; ++m) {
      if (m + 1 < QSLOT) read(m + 1, (m + 1) & 1);
#pragma unroll
      for (int e = 0; e < 2; ++e) dQt[e] = mfma16(ak[m & 1][e], as[m & 1], dQt[e]);
    }
  };
  // dQ leaves through a step's LDS tile: each wave writes its 16 rows x 32
  // head-dim columns (16-byte chunk k of row r stored at chunk k ^ (r mod 16),
  // so that the 8-byte writes of 16 lanes fall on distinct chunks and the row
  // reads of 16 on a whole row), and after the next barrier reads rows
  // 4 w .. 4 w + 3 back and stores them whole.  The store of every lane is
  // issued whatever the row (rows past the sequence's slots, and the step
  // before the chunk's first, write into the never-used partial slot of
  // chunk 0), so every step ends with the same loads and stores in flight.
  auto dq_tile_write = [&](T* tile, const f32x4 (&dQt)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      T x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = Elem<T>::from_float(p.scale * dQt[e][r]);
      const int k = 4 * dq4 + 2 * e + (gq >> 1);
      *reinterpret_cast<u32x2*>(&tile[(16 * rb + c) * QD + ((k ^ c) << 3) + 4 * (gq & 1)]) = __builtin_bit_cast(u32x2, x);
    }
  };
  auto dq_tile_read = [&](const T* tile) {
    const int r = 4 * w + (l >> 4), k = l & 15;
    return *reinterpret_cast<const V8*>(&tile[r * QD + ((k ^ (r & 15)) << 3)]);
  };
  auto dq_tile_store = [&](int i, int h, bool valid, const V8& x) {
    const int row = i * QR + 4 * w + (l >> 4), k = l & 15;
    T* dst = (valid && row < s.cap_q ? row_at(dq_row0 + h * dq_hs, row, dq_rs) : reinterpret_cast<T*>(a.dq_acc)) + 8 * k;
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4*>(dst));
  };

  // ---- kv-tiles no chunk's ring holds: zeros ----------------------------------
  {
    const int jhi = chunk == 0 ? min(max(dq - 3, 0), nkt) : 0;     // before the first window
    const int klo = i1 == nqt ? min(max(nqt + dq, 0), nkt) : nkt;  // after the last
    for (int pass = 0; pass < 2; ++pass) {
      const int r0 = (pass == 0 ? 0 : klo) * QK;
      const int r1 = min((pass == 0 ? jhi : nkt) * QK, s.cap_kv);
      for (int e = tid; e < (r1 - r0) * QCH; e += QTHR) {
        const int key = r0 + e / QCH, ch = e % QCH;
        st8(static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, hk, key) + 8 * ch, zero8);
        st8(static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, hk, key) + 8 * ch, zero8);
      }
    }
  }

  // ---- prologue: the ring of q-step i0 and the rows of the first three steps ---
  int ci = i0, cg = 0;  // the current step
  auto next_of = [&](int& i, int& gg) {
    if (++gg == G) {
      gg = 0;
      ++i;
    }
  };
  load_keys(slot_tile(slot, i0));
  store_k_rows();
  stream_rows(i0, hk * G, sQO0, sO0);
  const float lse0 = w == 0 ? load_lse(i0, hk * G) : 0.f;
  float nlse = 0.f;  // wave 0: the LSE of the next step's rows
  {
    int i = i0, gg = 0;
    next_of(i, gg);
    if (i < i1) {
      stream_rows(i, hk * G + gg, sQO1, sO1);
      if (w == 0) nlse = load_lse(i, hk * G + gg);
    }
    next_of(i, gg);
    if (i < i1) stream_rows(i, hk * G + gg, sQO2, sO2);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  store_lse(i0, lse0, sLD0);
  form_delta(i0, sQO0, sO0, sLD0);
  int pi = i0, ph = 0;  // the previous step's q-step and head, whose dQ tile is pending
  bool pending = false;
  const T* last_tile = sDQ0;

  // One step: rows of (q-step ci, head hk G + cg) in buffer c; the next
  // step's rows are in buffer n (landed by barrier A), and the rows of the
  // step after the one after that start streaming into buffer n3 at the
  // end.  False after the chunk's last step.
  auto step = [&](const T* cqo, const float* cld, const T* nqo, const T* nob, float* nld, T* n3qo,
                  T* n3ob, T* dqw, const T* dqp) -> bool {
    int ni = ci, ng = cg;
    next_of(ni, ng);
    int ai = ni, ag = ng;  // step s + 2 (its LSE), then s + 3 (its rows)
    next_of(ai, ag);
    int bi = ai, bg = ag;
    next_of(bi, bg);
    const bool more = ni < i1, more2 = ai < i1;
    const int so = (ci + dq - 3) & 3;  // the oldest slot: its kv-tile leaves after this q-step
    // Everything this wave issued but the last 4 operations of the previous
    // step (the 3 loads of the rows of step s + 2, then its dQ store) has
    // completed: the rows of step s + 1, its own K / V rows, the earlier
    // stores and the LSE loads.
    refresh_offsets();
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    lds_barrier();  // T: this step's statistics are in, phase 2 of the last step is done
    if (cg == 0 && ci > i0 && slot == ((ci + dq) & 3)) store_k_rows();  // the slot entering at ci
    if (p.has_sink && w == 0) sink_partial(ci, cg, cld);
    phase1(ci, cqo, cld);
    lds_barrier();  // A: dS^T complete; everyone's rows of step s + 1 are in (since T)
    if (more) store_lse(ni, nlse, nld);
    if (more2 && w == 0) nlse = load_lse(ai, hk * G + ag);
    if (slot == so && ng == 0) {  // the last head of q-step ci: this slot's kv-tile is done
      retire();
      if (more) load_keys(ni + dq);
    }
    if (more) form_delta(ni, nqo, nob, nld);
    f32x4 dQt[2];
    phase2_dq(dQt);
    // (past the chunk's end: a copy of in-range rows into the free buffer, so
    // that every step ends with the same 3 loads in flight)
    stream_rows(bi, hk * G + bg, n3qo, n3ob);
    // the previous step's dQ rows (its tile is complete since barrier T),
    // then this step's tile, then the store
    const V8 prev = dq_tile_read(dqp);
    dq_tile_write(dqw, dQt);
    dq_tile_store(pi, ph, pending, prev);
    pi = ci;
    ph = hk * G + cg;
    pending = true;
    last_tile = dqw;
    ci = ni;
    cg = ng;
    return more;
  };
  while (step(sQO0, sLD0, sQO1, sO1, sLD1, sQO3, sO3, sDQ0, sDQ1) &&
         step(sQO1, sLD1, sQO2, sO2, sLD2, sQO0, sO0, sDQ1, sDQ0) &&
         step(sQO2, sLD2, sQO3, sO3, sLD3, sQO1, sO1, sDQ0, sDQ1) &&
         step(sQO3, sLD3, sQO0, sO0, sLD0, sQO2, sO2, sDQ1, sDQ0)) {
  }
  // the last step's dQ tile
  lds_barrier();
  dq_tile_store(pi, ph, true, dq_tile_read(last_tile));
  // the three newer slots of the last q-step still hold kv-tiles
  if (slot != ((i1 - 1 + dq - 3) & 3)) retire();
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no LDS write outlives the block
}

// The kv-tiles two neighbouring chunks share: dK = scale (earlier + later),
// dV = earlier + later, in that order.  One block per (sequence, kv head,
// chunk boundary, tile).
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_qstream_fix_kernel(BwdArgs a) {
  const Problem& p = a.p;
  const int nch = p.qs_nch, C = p.qs_chunk;
  int L = blockIdx.x;
  const int t = L % 3;
  L /= 3;
  const int k = L % (nch - 1) + 1, bh = L / (nch - 1);
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const Seq s = load_seq(p, b);
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, 1, p.window, 0, QR, QK);
  const int j = k * C + g.diag / QK - 3 + t;
  if (j < 0 || j >= g.n_kv_tiles) return;
  const int lo = g.q_lo(j), hi = lo + g.n_iters(j);
  if (!(lo < k * C && k * C < hi)) return;
  const float* e0 = a.dq_acc + ((((int64_t)bh * nch + k) * 3 + t) * 2 + 0) * QPART;
  const float* e1 = e0 + QPART;
  for (int e = threadIdx.x; e < QPART / 4; e += kThreads) {
    const int key = j * QK + e / (2 * QD / 4), col = (e % (2 * QD / 4)) * 4;
    if (key >= s.cap_kv) continue;
    const f32x4 x = *reinterpret_cast<const f32x4*>(e0 + 4 * e);
    const f32x4 y = *reinterpret_cast<const f32x4*>(e1 + 4 * e);
    const bool isk = col < QD;
    const float f = isk ? p.scale : 1.f;
    T v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = Elem<T>::from_float(f * (x[r] + y[r]));
    T* out = isk ? static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, hk, key) + col
                 : static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, hk, key) + (col - QD);
    *reinterpret_cast<u32x2*>(out) = __builtin_bit_cast(u32x2, v);
  }
}

hipError_t launch_bwd_qstream(const BwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hkv * a.p.qs_nch;
  if (n == 0) return hipSuccess;
  if (a.dtype == 0)
    hipLaunchKernelGGL((bwd_qstream_kernel<__bf16>), dim3(n), dim3(QTHR), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_qstream_kernel<_Float16>), dim3(n), dim3(QTHR), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.p.qs_nch < 2) return e;
  const int nf = a.p.B * a.p.Hkv * (a.p.qs_nch - 1) * 3;
  if (a.dtype == 0)
    hipLaunchKernelGGL((bwd_qstream_fix_kernel<__bf16>), dim3(nf), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_qstream_fix_kernel<_Float16>), dim3(nf), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace swa
