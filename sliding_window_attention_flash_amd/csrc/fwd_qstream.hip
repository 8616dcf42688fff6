// fwd_qstream: the window-trimmed forward for short windows at head_dim 128
// with query-head groups of a multiple of 8, in one pass over query rows
// (gfx950).
//
// Source: cudnn-frontend PR #866 "frost(sdpa): bound the SM80 backward q-loop
// by the sliding window ...", Problem section (the forward trims its kv range
// by the window); cudnn-frontend PR #557 "... sink-token gradients ...",
// Summary (a per-head sink logit joins each row's softmax denominator).
//
// The rows of a 32-row q-step i see only keys of the 32-key kv-tiles
// i + d - NS + 1 .. i + d, with d = diag / 32 and NS = ceil(W / 32) + 1 (at
// most 4 for W <= 96; the plan takes this kernel only for causal masks with
// no right band, diag a multiple of 32 and dense sequences).  One block of 8
// waves (one per CU) walks a chunk of consecutive q-steps of one (sequence,
// kv head).  Those kv-tiles stay in an 8-slot LDS ring (tile j in slot
// j mod 8) that every query head of the group reads: each q-step adds one
// tile, loaded into registers during the previous q-step and written to its
// slot at the step's top.  Wave w owns the query heads w, w + 8, .. of the
// group; for each q-step and head it computes
//   S^T = K Q^T over the NS tiles   A: K rows from the ring, B: the Q rows,
//                                   loaded straight into registers while the
//                                   previous (q-step, head) step computed;
//   the softmax of each row at once (every key the row sees is in the ring:
//   max, exp2, sum; the sink joins the max and the denominator);
//   O^T = V^T P^T                   A: transposed reads of the ring's V
//                                   tiles, B: P^T from the S^T accumulators;
// and stores O (through a per-wave LDS tile, so that each store writes four
// whole rows) and the row LSE.  Rows past the sequence repeat its last row,
// so every lane issues the same stores (identical values to the same
// address) and the memory operations in flight at a step's top are always
// the same: the previous step's 9 stores.
//
// All products are v_mfma_f32_16x16x32 (bf16 / f16 in, fp32 accumulate),
// with the lane layouts and swizzled 128-wide LDS rows of the other kernels.

#include "kernels.h"
#include "tiles.h"

namespace swa {

namespace {

constexpr int FD = 128;         // head dim
constexpr int FNS = FD / 32;    // k-steps over the head dim
constexpr int FNDB = FD / 16;   // 16-column blocks of the head dim
constexpr int FCH = FD / 8;     // 16-byte chunks per row
constexpr int FR = 32;          // rows of a q-step
constexpr int FK = 32;          // keys of a ring tile
constexpr int FRING = 8;        // ring slots (NS + 1 <= 5 in use)
constexpr int FWAVE = 8;
constexpr int FTHR = 64 * FWAVE;
constexpr int FTILE = FK * FD;  // elements of a K (or V) tile
// s_waitcnt vmcnt(9): everything but the last 9 vector-memory operations
// (the previous step's 8 O stores and its LSE store) has completed
constexpr int kWaitVm9 = 0xF79;
constexpr int FOST = 16 * FD;   // elements of a wave's O staging tile (16 rows)
static_assert(FTHR * 8 == FTILE, "each thread stages one 16-byte chunk of a K and a V tile");

// A barrier for LDS only: this wave's LDS accesses are complete, then
// s_barrier (the loads streaming in for later steps are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

}  // namespace

template <typename T, int NS>
__global__ __launch_bounds__(FTHR, 1) void fwd_qstream_kernel(FwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  __shared__ __align__(16) T sK[FRING * FTILE];
  __shared__ __align__(16) T sV[FRING * FTILE];
  __shared__ __align__(16) T sO[FWAVE * FOST];  // per wave: 16 rows of O on their way out

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = p.qs_nch, C = p.qs_chunk, G = p.G, HPW = p.G / FWAVE;
  const int chunk = blockIdx.x % nch, bh = blockIdx.x / nch;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const Seq s = load_seq(p, b);
  const int nqt = (s.len_q + FR - 1) / FR;
  const int i0 = chunk * C, i1 = min(i0 + C, nqt);
  if (i0 >= i1) return;
  // diag >= 0 and a multiple of 32, len_q and len_kv > 0 (checked by the plan)
  const int diag = p.bottom_right ? s.len_kv - s.len_q : 0;
  const int dq = diag / FK;
  const int W = p.window;  // 0 <= W <= 96

  // ---- the ring ----------------------------------------------------------------
  // Thread tid stages row tid / 16 of a tile, stored chunk tid % 16, which
  // holds logical chunk (tid % 16) ^ tsw(row).  Keys outside the sequence
  // (and tiles before it) repeat a valid row: finite values that the mask
  // gives zero weight.
  const int st_row = tid / FCH, st_off = st_row * FD + 8 * (tid % FCH);
  const int st_ch = (tid % FCH) ^ tsw<FD>(st_row);
  const T* const k_row0 = static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, hk, 0) + 8 * st_ch;
  const T* const v_row0 = static_cast<const T*>(a.v) + elem_off(p, p.sv, b, s.row0_kv, hk, 0) + 8 * st_ch;
  const int64_t k_rs = p.sk[2], v_rs = p.sv[2];
  V8 stK, stV;
  auto stage = [&](int j) {
    const int kr = clampi(j * FK + st_row, 0, s.len_kv - 1);
    stK = ld8(row_at(k_row0, kr, k_rs));
    stV = ld8(row_at(v_row0, kr, v_rs));
  };
  auto write_staged = [&](int j) {
    const int sl = j & (FRING - 1);
    *reinterpret_cast<V8*>(&sK[sl * FTILE + st_off]) = stK;
    *reinterpret_cast<V8*>(&sV[sl * FTILE + st_off]) = stV;
  };

  // ---- Q rows, O rows, LSE ------------------------------------------------------
  const T* const q_b = static_cast<const T*>(a.q) + elem_off(p, p.sq, b, s.row0_q, 0, 0) + 8 * gq;
  T* const o_b = static_cast<T*>(a.o) + elem_off(p, p.so, b, s.row0_q, 0, 0);
  const int64_t q_hs = p.sq[1], q_rs = p.sq[2], o_hs = p.so[1], o_rs = p.so[2];
  float* const lse_b = a.lse + s.stat0;
  // B operand of S^T: lane (c, g) holds Q[row 16 rb + c][32 kst + 8 g .. + 7];
  // two buffers, the next step's rows loading while this one computes
  V8 qX[2][FNS], qY[2][FNS];
  auto load_q = [&](int i, int h, V8 (&qB)[2][FNS]) {
    const T* qh = q_b + h * q_hs;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const T* qr = row_at(qh, min(i * FR + 16 * rb + c, s.len_q - 1), q_rs);
#pragma unroll
      for (int kst = 0; kst < FNS; ++kst) qB[rb][kst] = ld8(qr + 32 * kst);
    }
  };
  // lane l < HPW holds the sink logit (log2 units) of head w + 8 l of the group
  const float sink_l = p.has_sink && l < HPW ? a.sink[hk * G + w + FWAVE * l] * kLog2e : -INFINITY;

  // lane offsets into a tile (elements)
  int rd_off[FNS], tr_off[FNDB];
#pragma unroll
  for (int kst = 0; kst < FNS; ++kst) rd_off[kst] = toff<FD>(c, 4 * kst + gq);
#pragma unroll
  for (int db = 0; db < FNDB; ++db) tr_off[db] = troff<FD>(c, gq, db);

  // ---- prologue: the ring of q-step i0 but its newest tile, which is staged ----
  for (int t = 0; t + 1 < NS; ++t) {
    const int j = i0 + dq - NS + 1 + t;
    stage(j);
    write_staged(j);
  }
  stage(i0 + dq);
  int ci = i0, hh = 0;  // the current step: q-step ci, head w + 8 hh of the group
  load_q(ci, hk * G + w, qX);
  __builtin_amdgcn_s_waitcnt(0);

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // One step (q-step ci, head w + 8 hh) with its rows in qB, the next step's
  // rows loading into qN; false after the chunk's last step.
  auto step = [&](const V8 (&qB)[2][FNS], V8 (&qN)[2][FNS]) -> bool {
    // (the lane offsets are made opaque each step: left loop-invariant, the
    // compiler keeps a precomputed copy of each for every ring slot)
#pragma unroll
    for (int kst = 0; kst < FNS; ++kst) asm volatile("" : "+v"(rd_off[kst]));
#pragma unroll
    for (int db = 0; db < FNDB; ++db) asm volatile("" : "+v"(tr_off[db]));
    // the Q rows of this step and the staged tile have landed
    __builtin_amdgcn_s_waitcnt(kWaitVm9);
    if (hh == 0) {
      // the tile entering at q-step ci; its slot last held tile ci + dq - 8,
      // which no wave has read since q-step ci - 5
      write_staged(ci + dq);
      lds_barrier();
      if (ci + 1 < i1) stage(ci + 1 + dq);
    }
    const int h = hk * G + w + FWAVE * hh;
    int ni = ci, nh = hh + 1;
    if (nh == HPW) {
      nh = 0;
      ++ni;
    }
    const bool more = ni < i1;
    if (more) load_q(ni, hk * G + w + FWAVE * nh, qN);
    const int jb = ci + dq - NS + 1;  // the ring's oldest tile for this q-step

    // S^T [key][row] for the NS tiles: [tile][16-key half][16-row block]
    f32x4 S[NS][2][2];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const T* kt = sK + ((jb + t) & (FRING - 1)) * FTILE;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        V8 ka[FNS];
#pragma unroll
        for (int kst = 0; kst < FNS; ++kst) ka[kst] = *reinterpret_cast<const V8*>(&kt[16 * kh * FD + rd_off[kst]]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          S[t][kh][rb] = mfma16(ka[0], qB[rb][0], zero4);
#pragma unroll
          for (int kst = 1; kst < FNS; ++kst) S[t][kh][rb] = mfma16(ka[kst], qB[rb][kst], S[t][kh][rb]);
        }
      }
    }

    // Mask: row r sees key k when 0 <= r + diag - k <= W and k < len_kv,
    // i.e. lo <= r + diag - k <= W with lo = max(0, r + diag - len_kv + 1).
    // Lane term A = r + diag - lo - 4 g; the element (tile j, half kh,
    // register e) holds key 32 j + 16 kh + 4 g + e and is visible when
    // (unsigned)(A - 32 j - 16 kh - e) <= W - lo.  Tiles before the
    // sequence (j < 0) are masked whole.
    int A[2];
    unsigned rg[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = min(ci * FR + 16 * rb + c, s.len_q - 1);
      const int lo = max(0, row + diag - s.len_kv + 1);
      const int span = W - lo;
      A[rb] = span < 0 ? -(1 << 30) : row + diag - lo - 4 * gq;
      rg[rb] = span < 0 ? 0u : (unsigned)span;
    }
    float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int j = jb + t;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int kt = j * FK + 16 * kh;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int ub = j < 0 ? -(1 << 30) : A[rb] - kt;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = (unsigned)(ub - e) <= rg[rb] ? S[t][kh][rb][e] : -INFINITY;
            S[t][kh][rb][e] = x;
            mx[rb] = fmaxf(mx[rb], x);
          }
        }
      }
    }
    // the row max over the 4 lanes holding it; with the sink (log2 units)
    const float snk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sink_l), hh));
    float mref[2], lsum[2];
    V8 bP[2][NS];  // B operand of O^T: P^T of 32 keys (tile t) x 16 rows
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float m = fmaxf(col4_max(mx[rb]) * p.scale_log2, snk);  // the scale is > 0
      mref[rb] = m == -INFINITY ? 0.f : m;  // a row that sees nothing keeps zeros
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = fast_exp2(__builtin_fmaf(S[t][kh][rb][e], p.scale_log2, -mref[rb]));
            rs += pv;
            bP[rb][t][4 * kh + e] = Elem<T>::from_float(pv);
          }
      lsum[rb] = col4_sum(rs) + fast_exp2(snk - mref[rb]);  // exp2(-inf) = 0 without a sink
    }

    // O^T [head dim][row] = V^T P^T over the NS tiles
    f32x4 O[FNDB][2];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const T* vt = sV + ((jb + t) & (FRING - 1)) * FTILE;
#pragma unroll
      for (int db = 0; db < FNDB; ++db) {
        const V8 va = trpair(&vt[tr_off[db]], &vt[16 * FD + tr_off[db]]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) O[db][rb] = mfma16(va, bP[rb][t], t == 0 ? zero4 : O[db][rb]);
      }
    }

    // O = O^T / denominator (a row with neither a visible key nor a sink
    // gets O = 0 and LSE = -inf), then LSE
    // Each 16-row block goes through the wave's LDS tile (16-byte chunk k of
    // row r stored at chunk k ^ r: the 8-byte writes of 32 lanes and the
    // row reads of 16 fall on distinct banks), so that every store writes
    // four whole rows.
    T* const oh = o_b + h * o_hs;
    float lse_v[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bool live = lsum[rb] > 0.f;
      const float inv = live ? 1.f / lsum[rb] : 0.f;
      lse_v[rb] = live ? (mref[rb] + __log2f(lsum[rb])) * kLn2 : -INFINITY;
#pragma unroll
      for (int db = 0; db < FNDB; ++db) {
        T ox[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ox[e] = Elem<T>::from_float(O[db][rb][e] * inv);
        // row c, head-dim 16 db + 4 g: chunk 2 db + g / 2, half g % 2
        *reinterpret_cast<u32x2*>(&sO[w * FOST + c * FD + (((2 * db + (gq >> 1)) ^ c) << 3) + 4 * (gq & 1)]) =
            __builtin_bit_cast(u32x2, ox);
      }
#pragma unroll
      for (int ps = 0; ps < 4; ++ps) {
        const int r = 4 * ps + (l >> 4), k = l & 15;
        const V8 x = *reinterpret_cast<const V8*>(&sO[w * FOST + r * FD + ((k ^ r) << 3)]);
        // (non-temporal: O is not read again here; 2% faster at c4)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x),
                                    reinterpret_cast<u32x4*>(row_at(oh, min(ci * FR + 16 * rb + r, s.len_q - 1), o_rs) + 8 * k));
      }
    }
    {
      // lane (c, g) writes row 16 (g mod 2) + c (lanes g and g + 2 the same value)
      const int rb = gq & 1;
      lse_b[h * s.stat_hs + min(ci * FR + 16 * rb + c, s.len_q - 1)] = rb ? lse_v[1] : lse_v[0];
    }
    ci = ni;
    hh = nh;
    return more;
  };
  while (step(qX, qY) && step(qY, qX)) {
  }
}

hipError_t launch_fwd_qstream(const FwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hkv * a.p.qs_nch;
  if (n == 0) return hipSuccess;
  // tiles the rows of a q-step see: ceil(W / 32) + 1 (the plan checked W <= 96)
  const int ns = (a.p.window + FK - 1) / FK + 1;
  if (a.p.window < 0 || ns > 4) return hipErrorInvalidValue;
#define SWA_FWD_QS(T, N) hipLaunchKernelGGL((fwd_qstream_kernel<T, N>), dim3(n), dim3(FTHR), 0, st, a)
  if (a.dtype == 0) {
    switch (ns) {
      case 1: SWA_FWD_QS(__bf16, 1); break;
      case 2: SWA_FWD_QS(__bf16, 2); break;
      case 3: SWA_FWD_QS(__bf16, 3); break;
      default: SWA_FWD_QS(__bf16, 4); break;
    }
  } else {
    switch (ns) {
      case 1: SWA_FWD_QS(_Float16, 1); break;
      case 2: SWA_FWD_QS(_Float16, 2); break;
      case 3: SWA_FWD_QS(_Float16, 3); break;
      default: SWA_FWD_QS(_Float16, 4); break;
    }
  }
#undef SWA_FWD_QS
  return hipGetLastError();
}

}  // namespace swa
