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

}  // namespace swa
