// Window-bounded tile schedule of the sliding-window attention backward.
// Shared by the host plan and the device kernels (header-only, integer-only).
//
// Source: cudnn-frontend PR #866, "frost(sdpa): bound the SM80 backward
// q-loop by the sliding window ... + window-aware deterministic relay",
// commit message and "Change" section:
//   * the anchor of query row i is i (top-left) or i + diag with
//     diag = s_kv - s_q (bottom-right), in-sequence indices (per packed
//     sequence for THD);
//   * a kv-tile [kv_base, kv_base + tile_kv) is seen by no query whose
//     anchor exceeds kv_base + tile_kv - 1 + W, so the q-tile loop stops at
//     q_hi = ceil((kv_base + tile_kv + W - diag) / tile_q);
//   * the loop starts at the causal skip q_lo (not printed on the page: the
//     first q-tile holding a row whose anchor reaches kv_base);
//   * a kv-tile with no q-tile to visit stores dK = dV = 0;
//   * the ordered dQ relay counts a visitor's turn from the q-tile's first
//     visitor kv_first = max((q_row0 + diag - W) // tile_kv, 0).
// The window is inclusive: row i keeps keys with anchor(i) - j <= W.
// Right-band widening (cudnn-frontend PR #557, Summary, named there without
// a formula) is read as an inclusive right bound R on the causal mask: row i
// keeps keys j <= anchor(i) + R, so R = 0 is plain causal; it moves the
// causal skip q_lo and its inverse kv_last by R keys.
#pragma once

#if defined(__HIPCC__)
#define SWA_HD __host__ __device__ __forceinline__
#else
#define SWA_HD inline
#endif

namespace swa {

// Floor / ceiling division for a positive divisor and any-sign numerator
// (C's '/' truncates toward zero, the schedule needs floor and true ceil).
SWA_HD int floor_div(int a, int b) {
  int q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}
SWA_HD int ceil_div(int a, int b) { return -floor_div(-a, b); }
SWA_HD int imax(int a, int b) { return a > b ? a : b; }
SWA_HD int imin(int a, int b) { return a < b ? a : b; }

// Geometry of one (packed) sequence under one mask.
struct SeqSched {
  int len_q, len_kv;  // valid rows
  int diag;           // anchor offset: s_kv - s_q (bottom-right) or 0
  int tile_q, tile_kv;
  int causal;         // 1: keys after anchor + right are masked
  int window;         // < 0: no window; else inclusive left window W
  int right;          // causal only: inclusive right band R >= 0
  int n_q_tiles, n_kv_tiles;

  SWA_HD void init(int lq, int lkv, int bottom_right, int causal_, int window_, int right_,
                   int tq, int tkv) {
    len_q = lq;
    len_kv = lkv;
    diag = bottom_right ? lkv - lq : 0;
    tile_q = tq;
    tile_kv = tkv;
    causal = causal_;
    window = window_;
    right = causal_ ? right_ : 0;
    n_q_tiles = lq > 0 ? ceil_div(lq, tq) : 0;
    n_kv_tiles = lkv > 0 ? ceil_div(lkv, tkv) : 0;
  }

  // First q-tile that kv-tile j can feed: causal skip (the first row whose
  // anchor + R reaches kv-tile j's first key).
  SWA_HD int q_lo(int j) const {
    if (!causal) return 0;
    return imax(floor_div(j * tile_kv - diag - right, tile_q), 0);
  }
  // One past the last q-tile that kv-tile j can feed: window bound.
  SWA_HD int q_hi(int j) const {
    if (window < 0) return n_q_tiles;
    return imin(ceil_div(j * tile_kv + tile_kv + window - diag, tile_q), n_q_tiles);
  }
  SWA_HD int n_iters(int j) const {
    if (j < 0 || j >= n_kv_tiles) return 0;
    return imax(q_hi(j) - q_lo(j), 0);
  }
  // First kv-tile that visits q-tile i (inverse of the q_hi clamp).
  SWA_HD int kv_first(int i) const {
    if (window < 0) return 0;
    return imax(floor_div(i * tile_q + diag - window, tile_kv), 0);
  }
  // Last kv-tile that visits q-tile i (inverse of the q_lo clamp).
  SWA_HD int kv_last(int i) const {
    if (!causal) return n_kv_tiles - 1;
    return imin(ceil_div((i + 1) * tile_q + diag + right, tile_kv) - 1, n_kv_tiles - 1);
  }
  // Visitors of q-tile i form the contiguous range [kv_first, kv_last];
  // empty when i is past the valid rows or the range is inverted.
  SWA_HD int n_visitors(int i) const {
    if (i < 0 || i >= n_q_tiles) return 0;
    return imax(kv_last(i) - kv_first(i) + 1, 0);
  }
  // Relay turn of kv-tile j at q-tile i: its rank among i's visitors.
  SWA_HD int relay_turn(int i, int j) const { return j - kv_first(i); }
};

// Floor division by 2^k of any-sign numerators is an arithmetic right shift.
static_assert((-5 >> 1) == -3 && (-4 >> 2) == -1 && (5 >> 1) == 2, "arithmetic right shift");

// The schedule of the streaming kernel: SeqSched for a causal mask with a
// left window W >= 0 and no right band, at q-tiles of 64 rows and kv-steps
// of 128 keys, with each floor / ceiling division by those powers of two
// written as an arithmetic shift.  Plus the step-level quantities that
// kernel derives from it: which q-tiles a step retires and the 16-row query
// blocks each 16-key group of a step reaches (its band).
struct StreamSched {
  static constexpr int kTileQ = 64, kStep = 128, kBlock = 16;
  static constexpr int kQShift = 6, kStepShift = 7, kBlockShift = 4;
  static_assert((1 << kQShift) == kTileQ && (1 << kStepShift) == kStep && (1 << kBlockShift) == kBlock,
                "shift forms of the tile sizes");
  int len_q, len_kv, diag, window, n_q_tiles, n_kv_tiles;

  SWA_HD void init(int lq, int lkv, int bottom_right, int window_) {
    len_q = lq;
    len_kv = lkv;
    diag = bottom_right ? lkv - lq : 0;
    window = window_;
    n_q_tiles = lq > 0 ? (lq + kTileQ - 1) >> kQShift : 0;
    n_kv_tiles = lkv > 0 ? (lkv + kStep - 1) >> kStepShift : 0;
  }
  // SeqSched::q_lo / q_hi / n_iters / kv_first / kv_last at these tiles
  SWA_HD int q_lo(int j) const { return imax((j * kStep - diag) >> kQShift, 0); }
  SWA_HD int q_hi(int j) const { return imin(-((diag - j * kStep - kStep - window) >> kQShift), n_q_tiles); }
  SWA_HD int n_iters(int j) const { return j < n_kv_tiles ? imax(q_hi(j) - q_lo(j), 0) : 0; }
  SWA_HD int kv_first(int i) const { return imax((i * kTileQ + diag - window) >> kStepShift, 0); }
  SWA_HD int kv_last(int i) const {
    return imin(-((-(i + 1) * kTileQ - diag) >> kStepShift) - 1, n_kv_tiles - 1);
  }
  // Below the sequence's last kv-step, kv_last(i) <= j exactly for
  // i < (128 (j + 1) - diag) / 64 (kv_last is nondecreasing in i), so the
  // q-tiles of step j whose last visitor is j are its first n_retire(j)
  // (clipped to [0, n_iters(j)] by the caller).
  SWA_HD int n_retire(int j) const { return ((kStep * (j + 1) - diag) >> kQShift) - q_lo(j); }
  // Band of the 16 keys kv0 .. kv0 + 15 (visible rows: 0 <= row + diag - key
  // <= W): the 16-row query blocks band_lo(kv0) .. band_hi(kv0, qhi), not
  // clipped below (blocks before row 0 may start a band), clipped above to
  // the step's q-tiles [.., qhi); empty (band_hi < 0) past the keys.
  SWA_HD int band_lo(int kv0) const { return (kv0 - diag) >> kBlockShift; }
  SWA_HD int band_hi(int kv0, int qhi) const {
    if (kv0 >= len_kv) return -(1 << 30);
    return imin((kv0 + kBlock - 1 + window - diag) >> kBlockShift, 4 * qhi - 1);
  }
  // The dQ products of step j read the bands back by 32-key group ks (the
  // bands of key groups 2 ks and 2 ks + 1).  Band of group v starts at block
  // band_lo(kv0) + v, so rows 16 wr .. 16 wr + 15 of the step's k-th q-tile
  // (block 4 (q_lo + k) + wr) sit at band position pa = 4 k - 2 ks + c0 of
  // group 2 ks and pa - 1 of group 2 ks + 1, with c0 = dq_c0(j, wr).  The
  // bands hold the blocks up to dq_nb(j) positions past their start, so the
  // group pair contributes for k in [dq_klo(c0, ks), dq_khi(c0, nb, ks, n)],
  // n the step's q-tile count: exactly 1 <= pa <= nb + 1 and k < n.
  SWA_HD int dq_c0(int j, int wr) const { return wr + 1 + 4 * q_lo(j) - band_lo(j * kStep); }
  SWA_HD int dq_nb(int j) const {
    return ((j * kStep + kBlock - 1 + window - diag) >> kBlockShift) - band_lo(j * kStep) + 1;
  }
  SWA_HD int dq_klo(int c0, int ks) const { return imax((2 * ks - c0 + 4) >> 2, 0); }
  SWA_HD int dq_khi(int c0, int nb, int ks, int n) const { return imin((nb + 1 + 2 * ks - c0) >> 2, n - 1); }
};

}  // namespace swa
