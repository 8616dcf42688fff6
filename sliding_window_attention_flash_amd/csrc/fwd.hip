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
// One block (4 waves) per (q-tile of 64 rows, query head, sequence); each
// wave owns 16 query rows, kept in registers as the B operand of
// S^T = K Q^T (keys on the MFMA rows, queries on the columns).  The online
// softmax runs per column; O^T += V^T P^T takes P^T straight from the
// accumulator.  Accumulation in fp32, exp2 with log2(e) folded into the
// scale.
#include "kernels.h"

namespace swa {

template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 fld8(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::vec8*>(p);
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::vec8 flds_pair4(const T* p) {
  typedef typename Elem<T>::vec8 V8;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
  u32x4 r = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(V8, r);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  constexpr int NS = D / 32, NDB = D / 16;
  constexpr int LDR = D + 8, LDT = kTile + 8;
  constexpr int CH = D / 8, RPP = kThreads / CH, NPASS = kTile / RPP;
  __shared__ __align__(16) T sK[kTile * LDR];
  __shared__ __align__(16) T sVt[D * LDT];

  const Problem& p = a.p;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;
  const Seq s = load_seq(p, b);
  const int q0 = i * kTile;
  if (q0 >= s.cap_q) return;
  SeqSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, p.causal, p.window, p.right, kTile, kTile);
  const int hk = h / p.G;
  const int qrow = q0 + 16 * w + c;
  const T* qp = static_cast<const T*>(a.q);
  const T* kp = static_cast<const T*>(a.k);
  const T* vp = static_cast<const T*>(a.v);

  V8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = Elem<T>::from_float(0.f);
  V8 qB[NS];
  {
    const bool ok = qrow < s.len_q;
    const int64_t qo = elem_off(p, p.sq, b, s.row0_q, h, ok ? qrow : 0);
#pragma unroll
    for (int st = 0; st < NS; ++st) qB[st] = ok ? fld8(qp + qo + 32 * st + 8 * gq) : zero8;
  }

  float m = -INFINITY, lsum = 0.f;  // running max (log2 units) and sum
  if (p.has_sink) {
    m = a.sink[h] * kLog2e;
    lsum = 1.f;
  }
  f32x4 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int jlo = g.kv_first(i), nv = g.n_visitors(i);
  for (int jt = jlo; jt < jlo + nv; ++jt) {
    const int kv0 = jt * kTile;
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = tid / CH + ps * RPP, ch = tid % CH, kk = kv0 + r;
      V8 kx = zero8, vx = zero8;
      if (kk < s.len_kv) {
        kx = fld8(kp + elem_off(p, p.sk, b, s.row0_kv, hk, kk) + 8 * ch);
        vx = fld8(vp + elem_off(p, p.sv, b, s.row0_kv, hk, kk) + 8 * ch);
      }
      *reinterpret_cast<V8*>(&sK[r * LDR + 8 * ch]) = kx;
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(8 * ch + e) * LDT + r] = vx[e];
    }
    __syncthreads();

    f32x4 St[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      St[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st)
        St[mb] = mfma16(*reinterpret_cast<const V8*>(&sK[(16 * mb + c) * LDR + 32 * st + 8 * gq]),
                        qB[st], St[mb]);
    }
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 16 * mb + 4 * gq + r;
        const float t = visible(g, qrow, key) ? St[mb][r] * p.scale_log2 : -INFINITY;
        x[4 * mb + r] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    V8 pB[2];
    float rs = 0.f;
    if (mnew == -INFINITY) {
      pB[0] = zero8;
      pB[1] = zero8;
    } else {
      const float alpha = fast_exp2(m - mnew);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = fast_exp2(x[4 * mb + r] - mnew);
          rs += pv;
          pB[mb >> 1][(mb & 1) * 4 + r] = Elem<T>::from_float(pv);
        }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      lsum = lsum * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[db] *= alpha;
      m = mnew;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        O[db] = mfma16(flds_pair4(&sVt[(16 * db + c) * LDT + 32 * s2 + 4 * gq]), pB[s2], O[db]);
  }

  if (qrow >= s.cap_q) return;
  const bool live = qrow < s.len_q && lsum > 0.f;
  const float inv = live ? 1.f / lsum : 0.f;
  T* op = static_cast<T*>(a.o) + elem_off(p, p.so, b, s.row0_q, h, qrow);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    T ox[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ox[r] = Elem<T>::from_float(O[db][r] * inv);
    *reinterpret_cast<u32x2*>(op + 16 * db + 4 * gq) = __builtin_bit_cast(u32x2, ox);
  }
  if (gq == 0)
    a.lse[s.stat0 + h * s.stat_hs + qrow] = live ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

template <typename T>
static hipError_t fwd_t(const FwdArgs& a, hipStream_t st) {
  dim3 grid(a.p.n_q_tiles, a.p.Hq, a.p.B);
  if (a.p.D == 64)
    hipLaunchKernelGGL((fwd_kernel<T, 64>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, 128>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.p.n_q_tiles == 0) return hipSuccess;
  return a.dtype == 0 ? fwd_t<__bf16>(a, st) : fwd_t<_Float16>(a, st);
}

}  // namespace swa
