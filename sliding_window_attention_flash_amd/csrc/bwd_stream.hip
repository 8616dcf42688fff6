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
//   P, dS  = exp2(S c - LSE), P (dP - delta)          (fp32, masked; dP
//          accumulates from -delta, which the ring stores negated)
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
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT, one access pattern at a time):
// 16-byte row reads are conflict-free in any layout, and this permutation
// also makes the transposed reads conflict-free (a plain 128-byte pitch
// costs 4x).  Band rows are 208 elements apart (416 bytes), each group of 4
// rows 8 bytes further than the one before, which takes the dS^T writes
// from 4-way to conflict-free (see band_wr).  The whole kernel still
// records about 2.6M conflict cycles per launch at batch 2, 16 heads,
// S = 32768 (about 5% of its LDS instruction cycles); which accesses they
// come from is not pinned down.
// Transposed operands use ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element (i % 4) of lanes i / 4 + 4e (e = 0..3), so a lane
// pointing at row r0 + i / 4, column c0 + 4 (i % 4) receives rows
// r0 .. r0 + 3 of column c0 + i.
#include <type_traits>

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
constexpr int BSH = 4;        // extra offset (elements) per 4-row group of a band
constexpr int BAND = 16 * BP + 4 * BSH;  // elements of one wave's band

static_assert(STEP == StreamSched::kStep && kTile == StreamSched::kTileQ,
              "the kernel's kv-step and q-tile are the shift forms' tiles");
static_assert(NACT >= (STEP + 128) / 64 + 1, "a kv-step feeds at most ceil((128 + W) / 64) + 1 q-tiles, W <= 128");
static_assert(2 * NPAIR >= (16 + 128 + 15) / 16 + 1, "a 16-key band spans at most 10 16-row blocks, W <= 128");
static_assert(BAND % 8 == 0, "bands are cleared in 16-byte vectors");

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
  typedef T t2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const t2 a = __builtin_convertvector(f2{x0, x1}, t2), b = __builtin_convertvector(f2{x2, x3}, t2);
  return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// LDS byte addresses.  Reads through an explicit 32-bit address let the
// compiler fold constant displacements into the instruction's offset field.
typedef __attribute__((address_space(3))) unsigned char lds_byte;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_byte*)p;
}
template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t a) {
  return *(const __attribute__((address_space(3))) V*)(uintptr_t)a;
}
__device__ __forceinline__ u32x2 lds_tr4(uint32_t a) {
  v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(uintptr_t)a);
  return __builtin_bit_cast(u32x2, v);
}
// Agent-coherent 16-byte store and load of fp32 partial sums through a raw
// buffer resource with cache policy sc1: for each of the four words, the
// same visibility across the XCDs' L2 caches as a relaxed agent-scope
// atomic store or load (which compile to single-word sc1 stores and loads),
// in one instruction per lane.  Offsets are bytes from the resource base;
// the buffer unit drops stores at or past its size and reads zeros there.
constexpr int kAgentCoherent = 16;  // CPol::SC1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(float* base, int64_t bytes) {
  const int n = (int)min<int64_t>(bytes, INT32_MAX);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, n, 0x00020000);
}
__device__ __forceinline__ void st_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kAgentCoherent);
}
__device__ __forceinline__ f32x4 ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAgentCoherent));
}

// a value the compiler must keep in a register as computed (no re-derivation)
__device__ __forceinline__ uint32_t pin(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

}  // namespace

template <typename T, bool RELAY, bool DELTA>
__global__ __launch_bounds__(NTHR, 1) void bwd_stream_kernel(BwdArgs a) {
  typedef typename Elem<T>::vec8 V8;
  // The ring is a circle of NRB 16-row blocks: row r of q-tile t is row
  // r mod 16 of block (4 t + r / 16) mod NRB.  All Q blocks, then all dO
  // blocks (QO_DO bytes further); LSE, then delta (LD_DL bytes further).
  constexpr int NRB = 4 * NSLOT;
  __shared__ __align__(16) T sRing[2][NRB][16 * TROW];
  __shared__ __align__(16) float sLD[2][NRB][16];
  __shared__ __align__(16) T sK[STEP * TROW];
  __shared__ __align__(16) T sBand[NWAVE][BAND];  // dS^T [key][block position, row]
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
  // The window-bounded schedule at this kernel's fixed tiles (q-tiles of 64
  // rows, kv-steps of 128 keys, causal, no right band; the plan selects this
  // kernel only then), in the shift form of swa_sched.h.
  StreamSched g;
  g.init(s.len_q, s.len_kv, p.bottom_right, p.window);
  const int n_cap_steps = (s.cap_kv + STEP - 1) / STEP;
  const int j0 = chunk * p.chunk;
  if (j0 >= n_cap_steps) return;
  const int j1 = min(j0 + p.chunk, n_cap_steps);
  const int W = p.window;
  const int diag = g.diag, nqt = g.n_q_tiles, nkt = g.n_kv_tiles;
  auto q_lo = [&](int j) { return g.q_lo(j); };
  auto q_hi = [&](int j) { return g.q_hi(j); };
  auto n_iters = [&](int j) { return g.n_iters(j); };
  auto kv_first = [&](int i) { return g.kv_first(i); };
  auto kv_last = [&](int i) { return g.kv_last(i); };

  // (b, h) bases; row r of a tensor is at base + r * row stride
  const T* qb = static_cast<const T*>(a.q) + elem_off(p, p.sq, b, s.row0_q, h, 0);
  const T* kb = static_cast<const T*>(a.k) + elem_off(p, p.sk, b, s.row0_kv, h, 0);
  const T* vb = static_cast<const T*>(a.v) + elem_off(p, p.sv, b, s.row0_kv, h, 0);
  const T* dob = static_cast<const T*>(a.dO) + elem_off(p, p.sdo, b, s.row0_q, h, 0);
  const T* ob = static_cast<const T*>(a.o) + elem_off(p, p.so, b, s.row0_q, h, 0);  // DELTA
  T* dqb = static_cast<T*>(a.dq) + elem_off(p, p.sdq, b, s.row0_q, h, 0);
  T* dkb = static_cast<T*>(a.dk) + elem_off(p, p.sdk, b, s.row0_kv, h, 0);
  T* dvb = static_cast<T*>(a.dv) + elem_off(p, p.sdv, b, s.row0_kv, h, 0);
  const int rs_q = (int)p.sq[2], rs_k = (int)p.sk[2], rs_v = (int)p.sv[2], rs_do = (int)p.sdo[2];
  const int rs_o = (int)p.so[2];
  const int rs_dq = (int)p.sdq[2], rs_dk = (int)p.sdk[2], rs_dv = (int)p.sdv[2];
  const float* lseb = a.lse + s.stat0 + h * s.stat_hs;
  const float* deltab = a.delta + s.stat0 + h * s.stat_hs;
  float* accb = a.dq_acc + (s.stat0 + h * s.stat_hs) * SD;
  // this (b, h)'s rows of the accumulator, for the relay's coherent accesses
  const __amdgpu_buffer_rsrc_t accr = coherent_rsrc(accb, (int64_t)s.cap_q * SD * sizeof(float));
  float* stashb = a.dq_stash + (s.stat0 + h * s.stat_hs) * SD;
  // unordered mode: q-tile i's fp32 partial sum sits in a 64-row slot of its
  // own (stream_slot), lane-contiguous: element (wave w, e, r) of lane l at
  // ((2 w + e) 4 + r) 64 + l, so one atomic instruction adds into 256
  // contiguous bytes (measured 3.5x cheaper than 16 rows x 4 words)
  float* slotb = a.dq_acc + stream_slot(p, s, b, h, 0) * (kTile * SD);
  const int slot_lane = 4 * 64 * 2 * w + l;
  int* semb = a.sem + ((int64_t)b * p.Hq + h) * p.n_q_tiles;
  V8 zero8;
#pragma unroll
  for (int e = 0; e < 8; ++e) zero8[e] = Elem<T>::from_float(0.f);

  // ---- per-lane LDS offsets (elements) --------------------------------------
  int rd_off[2];  // row read of a 16-row block: row c, chunk 4 ks + gq
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off[ks] = tile_off(c, 4 * ks + gq);
  // the same in bytes, for the explicit-address reads of the ring
  uint32_t rd_off_b[2], tr_off_b[4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) rd_off_b[ks] = rd_off[ks] * sizeof(T);
#pragma unroll
  for (int db = 0; db < 4; ++db) tr_off_b[db] = tr_lane_off(c, gq, db) * sizeof(T);
  const uint32_t ld_off_b = 4 * gq * sizeof(float);  // LSE / delta of rows 4 gq ..
  const uint32_t ring_q = lds_addr(&sRing[0][0][0]), ring_ld = lds_addr(&sLD[0][0][0]);
  // K^T columns of this wave's dQ half (kept out of a runtime-indexed array,
  // which the compiler would place in scratch memory)
  const int tr_off_k0 = tr_lane_off(c, gq, 2 * wd), tr_off_k1 = tr_lane_off(c, gq, 2 * wd + 1);
  // Band row r starts at r BP + BSH (r / 4) elements.  8-byte LDS accesses
  // are served 16 lanes at a time over 32 banks (SQ_LDS_BANK_CONFLICT: a
  // plain 416-byte pitch costs 4x on the dS^T writes, a shift of rows
  // 8 .. 15 alone 2x): 8 bytes per 4-row group put the 16 rows of a
  // write's lane group on distinct bank pairs, while the 4 rows of a
  // transposed read's lane group keep disjoint 32-byte spans.
  const int band_wr = c * BP + BSH * (c >> 2) + 4 * gq;  // dS^T write: key c, rows 4 gq ..
  const int band_rd_row = 4 * gq + (c >> 2);
  const int band_rd = band_rd_row * BP + BSH * (band_rd_row >> 2) + 4 * (c & 3);  // transposed read
  T* const myband = sBand[w];
  const uint32_t band0 = lds_addr(&sBand[0][0]);

  // ---- loaders ------------------------------------------------------------
  // K and V rows of the wave's 16 keys in the MFMA B layout (key c, head-dim
  // 32 ks + 8 gq ..); the K rows are also this wave's share of the LDS K
  // tile.  Rows past the sequence are clamped to a valid row and zeroed
  // when the registers are taken into use.
  V8 kB[2], vB[2], kBn[2], vBn[2];
  auto load_kv = [&](int j, V8 (&kx)[2], V8 (&vx)[2]) {
    const int key = clampi(j * STEP + 16 * w + c, 0, max(s.cap_kv - 1, 0));
    const T* kr = kb + (int64_t)key * rs_k + 8 * gq;
    const T* vr = vb + (int64_t)key * rs_v + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      kx[ks] = gld8(kr + 32 * ks);
      vx[ks] = gld8(vr + 32 * ks);
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
    V8 q, o, x;  // x: O rows (DELTA, staged synchronously)
    float lse, delta;
    int tile;
  };
  // Thread tid holds 16 bytes (chunk tid % 8) of row tid / 8 of a q-tile.
  // DELTA: delta of each row (rowsum of dO * O) is formed here from the
  // thread's chunks, joined over the 8 lanes of the row; 0 past the
  // sequence.
  auto put_delta = [&](int tile, const V8& dov, const V8& xv) {
    const int row = tid >> 3, mb = (tile % NSLOT) * 4;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += Elem<T>::to_float(dov[e]) * Elem<T>::to_float(xv[e]);
    // the 8 lanes of the row by DPP (no LDS traffic): swaps within quads,
    // then each half-row's mirror, which pairs the two quads
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0xB1, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x4E, 0xF, 0xF, false));
    acc += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, acc), 0x141, 0xF, 0xF, false));
    if ((tid & 7) == 0) sLD[1][mb + (row >> 4)][row & 15] = tile * kTile + row < s.len_q ? -acc : 0.f;
  };
  auto load_o_rows = [&](int i) {
    const int row = tid >> 3, ch = tid & 7, qi = min(i * kTile + row, s.len_q - 1);
    return gld8(ob + (int64_t)qi * rs_o + 8 * ch);
  };
  // only called for q-tiles the schedule visits, so the sequence has rows;
  // with_o: also the O rows (DELTA), for a tile staged right away
  auto load_q_tile = [&](int i, QRegs& r, bool with_o) {
    r.tile = i;
    const int row = tid >> 3, ch = tid & 7, qi = min(i * kTile + row, s.len_q - 1);
    r.q = gld8(qb + (int64_t)qi * rs_q + 8 * ch);
    r.o = gld8(dob + (int64_t)qi * rs_do + 8 * ch);
    if (DELTA && with_o) r.x = load_o_rows(i);
    if (tid < kTile) {
      const int si = min(i * kTile + tid, s.len_q - 1);
      r.lse = lseb[si];
      if (!DELTA) r.delta = deltab[si];
    }
  };
  auto store_q_tile = [&](const QRegs& r, bool with_o) {
    const int mb = (r.tile % NSLOT) * 4, row = tid >> 3, ch = tid & 7;  // first block of the tile
    const bool ok = r.tile * kTile + row < s.len_q;
    *reinterpret_cast<V8*>(&sRing[0][mb + (row >> 4)][tile_off(row & 15, ch)]) = ok ? r.q : zero8;
    *reinterpret_cast<V8*>(&sRing[1][mb + (row >> 4)][tile_off(row & 15, ch)]) = ok ? r.o : zero8;
    if (tid < kTile) {
      const bool okr = r.tile * kTile + tid < s.len_q;
      // exp2(x - inf) = 0: padding rows carry no weight
      sLD[0][mb + (tid >> 4)][tid & 15] = okr ? r.lse * kLog2e : INFINITY;
      if (!DELTA) sLD[1][mb + (tid >> 4)][tid & 15] = okr ? -r.delta : 0.f;
    }
    if (DELTA && with_o) put_delta(r.tile, r.o, r.x);
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
  auto acc_off = [&](int i, int e) {  // 4 consecutive head-dim values
    return (int64_t)q_row(i) * SD + 16 * (2 * wd + e) + 4 * gq;
  };
  // a q-tile is visited by the kv-steps [kv_first, kv_last]; this chunk runs
  // the steps [j0, j1)
  auto retire = [&](int i, f32x4 (&acc)[2]) {  // block-uniform arguments
    const bool earlier = kv_first(i) < j0, later = kv_last(i) >= j1;
    const int qi = q_row(i);
    if (!earlier && !later) {
      if (qi < s.cap_q) {
        T* row = dqb + (int64_t)qi * rs_dq + 32 * wd + 4 * gq;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          *reinterpret_cast<u32x2*>(row + 16 * e) =
              pack4<T>(p.scale * acc[e][0], p.scale * acc[e][1], p.scale * acc[e][2], p.scale * acc[e][3]);
      }
    } else if (!RELAY) {
      float* slot = slotb + (int64_t)i * (kTile * SD) + slot_lane;
      if (qi < s.len_q)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) unsafeAtomicAdd(slot + (4 * e + r) * 64, acc[e][r]);
      // The visiting chunk whose adds complete last converts the tile: every
      // thread waits for its agent-scope atomics, then one thread counts the
      // chunk in; the chunk that completes the count reads the sums back
      // with agent-scope loads (coherent across XCDs).
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) sTicket = __hip_atomic_fetch_add(semb + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int nv = kv_last(i) / p.chunk - kv_first(i) / p.chunk + 1;
      if (sTicket == nv - 1 && qi < s.cap_q) {
        T* row = dqb + (int64_t)qi * rs_dq + 32 * wd + 4 * gq;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = p.scale * __hip_atomic_load(slot + (4 * e + r) * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          *reinterpret_cast<u32x2*>(row + 16 * e) = pack4<T>(v[0], v[1], v[2], v[3]);
        }
      }
    } else if (!earlier) {
      // first visiting chunk of a boundary tile: turn 0, no wait; the
      // partial leaves with agent-coherent stores, whose completion the
      // wait below observes before the turn is released
      if (qi < s.cap_q)
#pragma unroll
        for (int e = 0; e < 2; ++e) st_coherent(accr, (uint32_t)acc_off(i, e) * sizeof(float), acc[e]);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) __hip_atomic_store(semb + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // a later turn: stash the partial; it is added in turn order once this
      // chunk has finished its own kv-steps
      if (qi < s.cap_q)
#pragma unroll
        for (int e = 0; e < 2; ++e) *reinterpret_cast<f32x4*>(stashb + acc_off(i, e)) = acc[e];
    }
    acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- prologue -------------------------------------------------------------
  load_kv(j0, kBn, vBn);
  int loaded_hi = q_lo(j0);  // the ring holds q-tiles [.., loaded_hi)
  {
    // the first kv-step's q-tiles: all loads (K / V's too) issued before
    // the first store
    const int n0 = min(n_iters(j0), NACT);
    QRegs t0[NACT];
#pragma unroll
    for (int k = 0; k < NACT; ++k)
      if (k < n0) load_q_tile(loaded_hi + k, t0[k], true);
    // While they are in flight: the bands start (and their guard positions
    // stay) zero, and so does the ring, so that a ring slot read before any
    // tile was staged in it holds finite values (see the pair geometry).
    for (int e = tid; e < NWAVE * BAND / 8; e += NTHR) reinterpret_cast<V8*>(&sBand[0][0])[e] = zero8;
    for (int e = tid; e < 2 * NRB * 16 * TROW / 8; e += NTHR) reinterpret_cast<V8*>(&sRing[0][0][0])[e] = zero8;
    for (int e = tid; e < 2 * NRB * 16 / 4; e += NTHR)
      reinterpret_cast<f32x4*>(&sLD[0][0][0])[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NACT; ++k)
      if (k < n0) store_q_tile(t0[k], true);
    loaded_hi += n0;
  }
  take_kv(j0, kBn, vBn);
  int acc_lo = q_lo(j0);     // q-tile held in dQa[0]
  QRegs pf[2];

  for (int j = j0; j < j1; ++j) {
    const int qlo = q_lo(j), nit = min(n_iters(j), NACT), qhi = qlo + nit;
    if (loaded_hi < qlo) loaded_hi = qlo;
    for (; loaded_hi < qhi; ++loaded_hi) {  // chunk start and gaps only
      QRegs t;
      load_q_tile(loaded_hi, t, true);
      store_q_tile(t, true);
    }
    __syncthreads();  // T: ring ready; sK and the bands are free
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) *reinterpret_cast<V8*>(&sK[tile_off(16 * w + c, 4 * ks + gq)]) = kB[ks];
    // realign dQa[0] with q_lo(j): q_lo advances by two q-tiles per step
    // except where it is clamped at the sequence start, so the shift is a
    // block-uniform 2 (plain register moves) or, once per sequence, 1
    auto shift_acc = [&](auto by) {
      constexpr int SH = decltype(by)::value;
#pragma unroll
      for (int k = 0; k < NACT; ++k)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          dQa[k][e] = k + SH < NACT ? dQa[min(k + SH, NACT - 1)][e] : f32x4{0.f, 0.f, 0.f, 0.f};
    };
    while (acc_lo < qlo) {
      if (qlo - acc_lo >= 2) {
        shift_acc(std::integral_constant<int, 2>());
        acc_lo += 2;
      } else {
        shift_acc(std::integral_constant<int, 1>());
        acc_lo += 1;
      }
    }

    // Prefetch of the next kv-step -- its K / V rows and new q-tiles -- is
    // issued over the first pairs of phase 1, and this step's dK / dV are
    // stored over phase 2: every CU runs the same step pattern, so memory
    // traffic issued in bursts at fixed points of the step would reach the
    // memory system from all of them at once.
    const bool has_next = j + 1 < j1;
    int pf_n = 0, pf_lo = 0;
    if (has_next) {
      const int nlo = q_lo(j + 1), nhi = nlo + min(n_iters(j + 1), NACT);
      pf_lo = max(loaded_hi, nlo);
      pf_n = max(0, min(2, nhi - pf_lo));
    }
    auto issue_pf = [&](int m) {
      if (m == 0 && has_next) load_kv(j + 1, kBn, vBn);
      if (m == 1 && pf_n > 0) load_q_tile(pf_lo, pf[0], false);
      if (m == 2 && pf_n > 1) load_q_tile(pf_lo + 1, pf[1], false);
    };

    // ---- phase 1: this wave's band --------------------------------------------
    const int kv0 = j * STEP;
    // t(row, key) = row + diag - key; visible iff 0 <= t <= W.  A key past
    // the sequence is pushed out of every window through its lane base.
    const int keyl = kv0 + 16 * w + c;
    const int tkey = keyl < s.len_kv ? diag - keyl : -(1 << 29);
    // 16-row blocks this wave's keys see (StreamSched::band_lo / band_hi)
    const int blo = g.band_lo(kv0 + 16 * w), bhi = g.band_hi(kv0 + 16 * w, qhi);
    const int npairs = nit == 0 || bhi < 0 ? 0 : min(max(bhi - blo + 2, 0) >> 1, NPAIR);
    struct PairSD {
      f32x4 S0, D0, S1, D1;
    };
    // Pair pr holds the band's blocks blo + 2 pr and blo + 2 pr + 1; block
    // blo + n sits at ring position (mlo + n) mod NRB.  A block before row 0
    // (only at a sequence start) or past bhi is masked out entirely; the
    // ring slot it reads holds finite values -- zeros from the kernel start
    // or rows staged earlier -- so its masked products add exact zeros.
    const int mlo = ((blo % NRB) + NRB) % NRB;
    auto ring_pos = [&](int n) {  // n < 2 NPAIR <= NRB
      const int m = mlo + n;
      return m >= NRB ? m - NRB : m;
    };
    // LDS byte addresses of ring block m (Q; the dO rows are QO_DO bytes
    // further) and of its LSE values (delta: LD_DL bytes further)
    constexpr uint32_t QO_DO = NRB * 16 * TROW * sizeof(T), LD_DL = NRB * 16 * sizeof(float);
    auto blk_addr = [&](int m) { return ring_q + (uint32_t)m * (16 * TROW * sizeof(T)); };
    auto ld_addr = [&](int m) { return ring_ld + (uint32_t)m * (16 * sizeof(float)); };
    // S = Q K^T and dP = dO V^T of both blocks
    auto stage_sdp = [&](int pr) {
      const int m0 = ring_pos(2 * pr), m1 = ring_pos(2 * pr + 1);
      const uint32_t a0 = blk_addr(m0), a1 = blk_addr(m1);
      PairSD r;
      // Wave priority 1 over each run of products: of a SIMD's two waves,
      // the one with MFMAs ready issues first while the other's softmax
      // fills the gaps (c3 main kernel -1.5%)
      __builtin_amdgcn_s_setprio(1);
      r.S0 = r.S1 = f32x4{0.f, 0.f, 0.f, 0.f};
      // dP starts from -delta of its rows, so that it leaves as dP - delta
      r.D0 = lds_ld<f32x4>(pin(ld_addr(m0) + ld_off_b) + LD_DL);
      r.D1 = lds_ld<f32x4>(pin(ld_addr(m1) + ld_off_b) + LD_DL);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint32_t x0 = pin(a0 + rd_off_b[ks]), x1 = pin(a1 + rd_off_b[ks]);
        r.S0 = mfma16(lds_ld<V8>(x0), kB[ks], r.S0);
        r.D0 = mfma16(lds_ld<V8>(x0 + QO_DO), vB[ks], r.D0);
        r.S1 = mfma16(lds_ld<V8>(x1), kB[ks], r.S1);
        r.D1 = mfma16(lds_ld<V8>(x1 + QO_DO), vB[ks], r.D1);
      }
      __builtin_amdgcn_s_setprio(0);
      return r;
    };
    // P, dS, the band write and dV^T += dO^T P, dK^T += Q^T dS
    auto stage_grad = [&](int pr, const PairSD& r) {
      const int b0 = blo + 2 * pr, m0 = ring_pos(2 * pr), m1 = ring_pos(2 * pr + 1);
      const bool has0 = b0 >= 0, has1 = b0 + 1 >= 0 && b0 + 1 <= bhi;
      const uint32_t a0 = blk_addr(m0), a1 = blk_addr(m1);
      const uint32_t l0 = pin(ld_addr(m0) + ld_off_b), l1 = pin(ld_addr(m1) + ld_off_b);
      const f32x4 lse0 = lds_ld<f32x4>(l0), lse1 = lds_ld<f32x4>(l1);
      const float lsev[8] = {lse0[0], lse0[1], lse0[2], lse0[3], lse1[0], lse1[1], lse1[2], lse1[3]};
      const float sv[8] = {r.S0[0], r.S0[1], r.S0[2], r.S0[3], r.S1[0], r.S1[1], r.S1[2], r.S1[3]};
      const float dv[8] = {r.D0[0], r.D0[1], r.D0[2], r.D0[3], r.D1[0], r.D1[1], r.D1[2], r.D1[3]};
      const int tb0 = has0 ? 16 * b0 + 4 * gq + tkey : -(1 << 29);
      const int tb1 = has1 ? 16 * (b0 + 1) + 4 * gq + tkey : -(1 << 29);
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (e < 4 ? tb0 : tb1) + (e & 3);
        // masked elements take exp2(-inf) = 0.  The empty asm makes x opaque
        // so that the compiler keeps a select instead of branching around
        // the LSE read and the multiply-add.
        float x = sv[e] * p.scale_log2 - lsev[e];
        asm("" : "+v"(x));
        pv[e] = fast_exp2((unsigned)t <= (unsigned)W ? x : -INFINITY);
        dsv[e] = pv[e] * dv[e];  // (dv: dP - delta)
      }
      const u32x2 p0 = pack4<T>(pv[0], pv[1], pv[2], pv[3]), p1 = pack4<T>(pv[4], pv[5], pv[6], pv[7]);
      const u32x2 s0 = pack4<T>(dsv[0], dsv[1], dsv[2], dsv[3]);
      const u32x2 s1 = pack4<T>(dsv[4], dsv[5], dsv[6], dsv[7]);
      const V8 pP = __builtin_bit_cast(V8, u32x4{p0[0], p0[1], p1[0], p1[1]});
      const V8 pS = __builtin_bit_cast(V8, u32x4{s0[0], s0[1], s1[0], s1[1]});
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint32_t y0 = pin(a0 + tr_off_b[db]), y1 = pin(a1 + tr_off_b[db]);
        const u32x2 o_lo = lds_tr4(y0 + QO_DO), o_hi = lds_tr4(y1 + QO_DO);
        const u32x2 q_lo = lds_tr4(y0), q_hi = lds_tr4(y1);
        dVa[db] = mfma16(__builtin_bit_cast(V8, u32x4{o_lo[0], o_lo[1], o_hi[0], o_hi[1]}), pP, dVa[db]);
        dKa[db] = mfma16(__builtin_bit_cast(V8, u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}), pS, dKa[db]);
      }
      __builtin_amdgcn_s_setprio(0);
      // dS^T of blocks b0, b1 at band positions 2 pr + 1, 2 pr + 2 (after the
      // pair's ring reads, which the stores would otherwise hold back)
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 1)) = s0;
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 2)) = s1;
    };
    // Software pipeline: the products of pair pr + 1 are issued in the same
    // straight-line block as the softmax and gradients of pair pr.
    PairSD sdp[2];
    if (npairs > 0) sdp[0] = stage_sdp(0);
#pragma unroll
    for (int pr = 0; pr < NPAIR; ++pr) {
      if (pr >= npairs) break;
      if (pr < 3) issue_pf(pr);
      if (pr + 1 < npairs) {
        sdp[(pr + 1) & 1] = stage_sdp(pr + 1);
        stage_grad(pr, sdp[pr & 1]);
      } else {
        stage_grad(pr, sdp[pr & 1]);
      }
    }
    for (int m = max(npairs, 0); m < 3; ++m) issue_pf(m);
    for (int pr = npairs; pr < NPAIR; ++pr) {  // positions past the band
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 1)) = u32x2{0u, 0u};
      *reinterpret_cast<u32x2*>(myband + band_wr + 16 * (2 * pr + 2)) = u32x2{0u, 0u};
    }

    __syncthreads();  // A: bands and sK complete; ring slots of tiles before q_lo(j + 1) free
    // Everything prefetched is taken into use here, before this step issues
    // any global store: vector-memory operations complete in order, so a
    // wait placed after the stores would also wait for their write-back.
    // The loads were issued before phase 1 and the last stores before that,
    // so this wait is normally free; it also tells the compiler that no load
    // is outstanding past this point.
    __builtin_amdgcn_s_waitcnt(0);
    if (pf_n > 0) store_q_tile(pf[0], false);
    if (pf_n > 1) store_q_tile(pf[1], false);
    loaded_hi += pf_n;
    // DELTA: the prefetched tiles' O rows load over phase 2; their delta is
    // formed at the end of the step, before the next one reads it
    V8 xo[2];
    if (DELTA && pf_n > 0) xo[0] = load_o_rows(pf_lo);
    if (DELTA && pf_n > 1) xo[1] = load_o_rows(pf_lo + 1);
    if (has_next) take_kv(j + 1, kBn, vBn);  // kB / vB of step j are no longer read

    // dK / dV of this step (zeros if it visited nothing) are complete after
    // this wave's phase 1; head-dim block db is stored in phase-2 round db
    auto store_dkdv = [&](int db) {
      if (keyl < s.cap_kv) {
        T* dkr = dkb + (int64_t)keyl * rs_dk;
        T* dvr = dvb + (int64_t)keyl * rs_dv;
        *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * gq) =
            pack4<T>(p.scale * dKa[db][0], p.scale * dKa[db][1], p.scale * dKa[db][2], p.scale * dKa[db][3]);
        *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * gq) = pack4<T>(dVa[db][0], dVa[db][1], dVa[db][2], dVa[db][3]);
      }
      dVa[db] = dKa[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // ---- phase 2: dQ^T += K^T dS^T ------------------------------------------
    // Wave v's band starts at block L + v (L = (kv0 - diag) / 16) and spans
    // nb = H - L + 1 blocks, so row block bb = 4 (q_lo + k) + wr sits at
    // position pa = 4 k - 2 ks + c0 of wave 2 ks and pb = pa - 1 of wave
    // 2 ks + 1, with c0 = wr + 1 + 4 q_lo - L; the pair of waves is active iff
    // 1 <= pa <= nb + 1.  Positions of clipped or missing blocks hold zeros,
    // so the positions are compile-time offsets from one per-wave address.
    {
      const int nb = g.dq_nb(j), c0 = g.dq_c0(j, wr);
      const uint32_t bbase = pin(band0 + band_rd * sizeof(T) + 32 * c0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        store_dkdv(ks);
        // the active k, klo <= k <= khi: 0 <= 4 k - 2 ks + c0 - 1 <= nb and
        // k < nit, as a bit mask
        const int klo = g.dq_klo(c0, ks), khi = g.dq_khi(c0, nb, ks, nit);
        const unsigned act = khi < klo ? 0u : ((2u << khi) - 1u) & ~((1u << klo) - 1u);
        if (act == 0u) continue;
        const T* kr = sK + 32 * ks * TROW;
        const V8 kt0 = tr_two(kr + tr_off_k0, kr + 16 * TROW + tr_off_k0);
        const V8 kt1 = tr_two(kr + tr_off_k1, kr + 16 * TROW + tr_off_k1);
#pragma unroll
        for (int k = 0; k < NACT; ++k) {
          if (!((act >> k) & 1u)) continue;
          const uint32_t ya = bbase + (uint32_t)(2 * ks * BAND * sizeof(T)) + 32 * (4 * k - 2 * ks);
          const u32x2 lo = lds_tr4(ya), hi = lds_tr4(ya + BAND * sizeof(T) - 32);
          const V8 st = __builtin_bit_cast(V8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          dQa[k][0] = mfma16(kt0, st, dQa[k][0]);
          dQa[k][1] = mfma16(kt1, st, dQa[k][1]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }

    // q-tiles whose last visitor in this chunk was this step (all of them
    // at the chunk's or the sequence's last step; StreamSched::n_retire)
    const int nret = j + 1 == j1 || j + 1 >= nkt ? nit : min(g.n_retire(j), nit);
#pragma unroll
    for (int k = 0; k < NACT; ++k)
      if (k < nret) retire(qlo + k, dQa[k]);
    if (DELTA) {
      // each thread reads back the dO chunk it staged
      const int row = tid >> 3, ch = tid & 7;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k >= pf_n) break;
        const int mb = ((pf_lo + k) % NSLOT) * 4;
        put_delta(pf_lo + k, *reinterpret_cast<const V8*>(&sRing[1][mb + (row >> 4)][tile_off(row & 15, ch)]),
                  xo[k]);
      }
    }
  }

  // ---- relay: boundary q-tiles this chunk joined after another chunk -------
  if (RELAY && j0 < nkt) {
    for (int i = q_lo(j0); i < nqt && i < q_hi(j0); ++i) {
      const int first = kv_first(i) / p.chunk;
      if (first >= chunk) break;  // kv_first is nondecreasing in i
      const int turn = chunk - first, nv = kv_last(i) / p.chunk - first + 1;
      int* semp = semb + i;
      if (tid == 0) {
        // a wait past the spin limit gives up so that the device never
        // hangs: it counts an expiry, and this turn then adds NaN, so the
        // q-tile's dQ comes out poisoned rather than out of order
        int spins = 0, expired = 0;
        while (__hip_atomic_load(semp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != turn + a.relay_bias) {
          if (++spins > a.spin_limit) {
            atomicAdd(&a.ctl[1], 1);
            expired = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        sTicket = expired;
      }
      __syncthreads();
      const bool expired = sTicket != 0;
      const int qi = q_row(i);
      if (qi < s.cap_q) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // the turn holds the tile alone: a coherent read of the running
          // sum, this chunk's add, and a coherent write for the next turn
          const uint32_t off = (uint32_t)acc_off(i, e) * sizeof(float);
          f32x4 mine = *reinterpret_cast<const f32x4*>(stashb + acc_off(i, e));
          if (expired) mine = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
          const f32x4 sum = ld_coherent(accr, off) + mine;
          if (turn < nv - 1)
            st_coherent(accr, off, sum);
          else
            *reinterpret_cast<u32x2*>(dqb + (int64_t)qi * rs_dq + 16 * (2 * wd + e) + 4 * gq) =
                pack4<T>(p.scale * sum[0], p.scale * sum[1], p.scale * sum[2], p.scale * sum[3]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0 && turn < nv - 1)
        __hip_atomic_store(semp, turn + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename T>
static void stream_t(const BwdArgs& a, int n, hipStream_t st) {
  if (a.p.stream_relay) {
    if (a.p.stream_delta)
      hipLaunchKernelGGL((bwd_stream_kernel<T, true, true>), dim3(n), dim3(NTHR), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<T, true, false>), dim3(n), dim3(NTHR), 0, st, a);
  } else {
    if (a.p.stream_delta)
      hipLaunchKernelGGL((bwd_stream_kernel<T, false, true>), dim3(n), dim3(NTHR), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_stream_kernel<T, false, false>), dim3(n), dim3(NTHR), 0, st, a);
  }
}

hipError_t launch_bwd_stream(const BwdArgs& a, hipStream_t st) {
  const int n = a.p.B * a.p.Hq * a.p.n_chunks;
  if (n == 0) return hipSuccess;
  if (a.dtype == 0)
    stream_t<__bf16>(a, n, st);
  else
    stream_t<_Float16>(a, n, st);
  return hipGetLastError();
}

}  // namespace swa
