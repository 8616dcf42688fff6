// Window-trimmed forward of the sliding-window attention (gfx950): O and the
// row log-sum-exp that the backward consumes.
//
// Source: cudnn-frontend PR #866 "frost(sdpa): bound the SM80 backward q-loop
// by the sliding window ...", Problem section: the forward already limits its
// kv range by the window.  Here a q-tile walks exactly its visitor range
// [kv_first, kv_last] of kv-tiles (the same schedule the backward uses).
// Sinks: cudnn-frontend PR #557 "... sink-token gradients ...", Summary: the
// per-head sink logit joins each row's softmax denominator.
//
// One block (4 waves) per (run of p.fwd_tiles consecutive q-tiles, query
// head, sequence); each wave owns 16 query rows of the current q-tile, kept
// in registers as the B operand of S^T = K Q^T (keys on the MFMA rows,
// queries on the columns).  The online softmax runs per column (one query
// row per lane column, its 16 keys spread over 4 lanes x 4 registers).
// O^T += V^T P^T takes V^T from transposed reads of the V tile and P^T
// straight from the accumulator, so each lane ends with 4 consecutive
// head-dim values of one row and O leaves as 8-byte stores.  K and V are
// double-buffered in swizzled LDS and the next pair's tiles (and, across a
// q-tile boundary, the next q-tile's rows) load while the current pair
// computes.  Accumulation in fp32, exp2 with log2(e) folded into the scale;
// a wave skips the 16-key blocks its rows cannot see.
#include "kernels.h"
#include "tiles.h"

namespace swa {

template <typename T, int D, bool RUN>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 2) void fwd_kernel(FwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  constexpr int NS = D / 32, NDB = D / 16;
  constexpr int CH = D / 8, RPP = kThreads / CH, NPASS = kTile / RPP;
  // K / V double buffer as two arrays (K tile, then V tile): every access
  // names its array, so the compiler sees that reads of one buffer need not
  // wait for the loads streaming into the other
  __shared__ __align__(16) T sKV0[2 * kTile * D];
  __shared__ __align__(16) T sKV1[2 * kTile * D];

  const Problem& p = a.p;
  const int tid = threadIdx.x, l = tid & 63, c = l & 15, gq = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // block -> (kv head, sequence, run of q-tiles, head within the group),
  // kv-head-major with runs descending, as in the q-major dQ pass
  const int nruns = (p.n_q_tiles + p.fwd_tiles - 1) / p.fwd_tiles;
  int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = L % p.G;
  L /= p.G;
  const int run = nruns - 1 - L % nruns;
  L /= nruns;
  const int b = L % p.B, hk = L / p.B, h = hk * p.G + hg;
  const Seq s = load_seq(p, b);
  const int ia = run * p.fwd_tiles;
  const int ib = min(ia + p.fwd_tiles, (s.cap_q + kTile - 1) / kTile);  // q-tiles holding slot rows
  if (ia >= ib) return;
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, p.causal, p.window, p.right, kTile, kTile);

  // running max (log2 units) and denominator of this lane's row; the sink
  // starts them at exp2(sink - m) = 1
  const float m0 = p.has_sink ? a.sink[h] * kLog2e : -INFINITY;
  const float l0 = p.has_sink ? 1.f : 0.f;
  float m = m0, lsum = l0;
  f32x4 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // O = O^T / denominator and LSE of row 16 w + c of q-tile i; a row past
  // the sequence, or with neither a visible key nor a sink, gets O = 0 and
  // LSE = -inf.  Rows past the slot are not stored.
  T* op = static_cast<T*>(a.o);
  auto finish = [&](int i) {
    const int row = i * kTile + 16 * w + c;
    if (row >= s.cap_q) return;
    const bool live = row < s.len_q && lsum > 0.f;
    const float inv = live ? 1.f / lsum : 0.f;
    T* orow = op + elem_off(p, p.so, b, s.row0_q, h, row) + 4 * gq;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      T ox[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ox[r] = Elem<T>::from_float(O[db][r] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * db) = __builtin_bit_cast(u32x2, ox);
    }
    if (gq == 0) a.lse[s.stat0 + h * s.stat_hs + row] = live ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
  };
  // q-tiles no kv-tile visits
  for (int i = ia; i < ib; ++i)
    if (g.n_visitors(i) == 0) finish(i);
  auto next_visited = [&](int i) {
    while (i < ib && g.n_visitors(i) == 0) ++i;
    return i;
  };
  int ci = next_visited(ia);  // current pair (ci, cj)
  if (ci >= ib) return;
  int cj = g.kv_first(ci);

  // Q rows of a visited q-tile (len_q > 0); rows past the sequence repeat
  // its last row and are dropped at the end
  V8 qB[NS], nqB[NS];
  const T* q0h = static_cast<const T*>(a.q) + elem_off(p, p.sq, b, s.row0_q, h, 0) + 8 * gq;
  auto load_q = [&](int i, V8* qv) {
    const int qr = min(i * kTile + 16 * w + c, s.len_q - 1);
    const T* qrow = row_at(q0h, qr, p.sq[2]);
#pragma unroll
    for (int st = 0; st < NS; ++st) qv[st] = ld8(qrow + 32 * st);
  };
  // K / V staging (a visited kv-tile: len_kv > 0); rows past the sequence
  // repeat its last key (finite values; the mask gives them zero weight).
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

  int rd_off[NS], tr_off[NDB];
#pragma unroll
  for (int st = 0; st < NS; ++st) rd_off[st] = toff<D>(c, 4 * st + gq);
#pragma unroll
  for (int db = 0; db < NDB; ++db) tr_off[db] = troff<D>(c, gq, db);

  // Mask: with t = row + diag - key, visible iff 0 <= t - tlo <= trange
  // (tlo = -R if causal, thi = W if windowed), and the key lies inside the
  // sequence.
  const int tlo = p.causal ? -p.right : -(1 << 28), thi = p.window >= 0 ? p.window : (1 << 28);
  const unsigned trange = (unsigned)(thi - tlo);

  load_q(ci, qB);
  load_kv(cj, sKV0, sKV0 + kTile * D);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // One pair: reads the tiles in (cK, cV) and streams the next pair's into
  // (nK, nV), which were last read before the previous barrier.  False once
  // the run is done.
  auto step = [&](const T* cK, const T* cV, T* nK, T* nV) -> bool {
    int ni = ci, nj = cj + 1;
    if (nj > g.kv_last(ci)) {
      ni = RUN ? next_visited(ci + 1) : ib;
      nj = ni < ib ? g.kv_first(ni) : 0;
    }
    const bool more = ni < ib;
    if (more) {
      load_kv(nj, nK, nV);
      if (RUN && ni != ci) load_q(ni, nqB);
    }
    const int kv0 = cj * kTile;
    const int kvn = s.len_kv - kv0;                           // keys of this tile inside the sequence
    const int u0 = ci * kTile + 16 * w + g.diag - tlo - kv0;  // t - tlo at (row 16 w, key kv0)
    const int tq = u0 + c - 4 * gq;                           // t - tlo at (row, key kv0 + 4 gq), minus 16 nb + r

    f32x4 St[4];
    bool live[4];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int um = u0 - 16 * nb;  // the block spans t - tlo in [um - 15, um + 15]
      live[nb] = um + 15 >= 0 && um - 15 <= (int)trange && 16 * nb < kvn;
      if (!live[nb]) {
        St[nb] = zero4;
        continue;
      }
      // the first product starts from a literal zero accumulator
      St[nb] = mfma16(*reinterpret_cast<const V8*>(&cK[16 * nb * D + rd_off[0]]), qB[0], zero4);
#pragma unroll
      for (int st = 1; st < NS; ++st)
        St[nb] = mfma16(*reinterpret_cast<const V8*>(&cK[16 * nb * D + rd_off[st]]), qB[st], St[nb]);
    }
    // masked logits (log2 units) and the tile's row max over the 4 lanes
    // sharing a column.  Where the wave's 16 rows see all 64 keys the mask
    // drops out.
    const bool full = u0 >= 63 && u0 + 15 <= (int)trange && kvn >= kTile;
    float x[4][4];
    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[nb][r] = St[nb][r] * p.scale_log2;
          mx = fmaxf(mx, x[nb][r]);
        }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = St[nb][r] * p.scale_log2;
          asm("" : "+v"(v));
          const bool vis = live[nb] && (unsigned)(tq - 16 * nb - r) <= trange && 16 * nb + 4 * gq + r < kvn;
          x[nb][r] = vis ? v : -INFINITY;
          mx = fmaxf(mx, x[nb][r]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float mref = mnew == -INFINITY ? 0.f : mnew;  // a row with nothing yet keeps zeros
    const float alpha = fast_exp2(m - mref);
    V8 bP[2];
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = fast_exp2(x[nb][r] - mref);
        rs += pv;
        bP[nb >> 1][(nb & 1) * 4 + r] = Elem<T>::from_float(pv);
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    lsum = lsum * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[db] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (!live[2 * ks] && !live[2 * ks + 1]) continue;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        O[db] = mfma16(trpair(&cV[32 * ks * D + tr_off[db]], &cV[(32 * ks + 16) * D + tr_off[db]]), bP[ks], O[db]);
    }
    if (ni != ci) {  // q-tile ci is complete
      finish(ci);
      m = m0;
      lsum = l0;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (RUN && more) {
#pragma unroll
        for (int st = 0; st < NS; ++st) qB[st] = nqB[st];
      }
    }
    if (!more) return false;
    // the next tiles (and the next q-tile's rows, if this pair ended one)
    // have landed, and (cK, cV) are free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ci = ni;
    cj = nj;
    return true;
  };
  while (step(sKV0, sKV0 + kTile * D, sKV1, sKV1 + kTile * D) &&
         step(sKV1, sKV1 + kTile * D, sKV0, sKV0 + kTile * D)) {
  }
}

template <typename T, int D>
static void fwd_td(const FwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hq * ((a.p.n_q_tiles + a.p.fwd_tiles - 1) / a.p.fwd_tiles);
  if (a.p.fwd_tiles > 1)
    hipLaunchKernelGGL((fwd_kernel<T, D, true>), dim3(n), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, false>), dim3(n), dim3(kThreads), 0, st, a);
}

// the q-major forward for short windows at head_dim 128 (fwd_qstream.hip)
hipError_t launch_fwd_qstream(const FwdArgs& a, hipStream_t st);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.p.n_q_tiles == 0) return hipSuccess;
  if (a.p.qstream) return launch_fwd_qstream(a, st);
  if (a.dtype == 0) {
    if (a.p.D == 64) fwd_td<__bf16, 64>(a, st);
    else fwd_td<__bf16, 128>(a, st);
  } else {
    if (a.p.D == 64) fwd_td<_Float16, 64>(a, st);
    else fwd_td<_Float16, 128>(a, st);
  }
  return hipGetLastError();
}

}  // namespace swa
