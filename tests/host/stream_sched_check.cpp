// Brute-force check (host only) of the streaming kernel's schedule, the
// shift forms of swa_sched.h's StreamSched, against the mask's definition
// and against the general SeqSched at the same tiles.  For random lengths,
// windows 0..128 and both anchors it checks:
//   * q_lo, q_hi, n_iters, kv_first, kv_last equal SeqSched's at q-tiles of
//     64 rows and kv-steps of 128 keys (causal, left window, no right band);
//   * a kv-step feeds at most 5 q-tiles (the kernel's register array);
//   * the q-tiles a step retires (n_retire, below the last step) are exactly
//     those whose last visitor it is, and every visited q-tile retires at
//     its last visitor;
//   * every visible (row, key) pair lies in a q-tile the key's step feeds,
//     in its 16-key group's band [band_lo, band_hi] (at most 10 blocks), and
//     in an active dQ round: dq_klo <= k <= dq_khi, with band positions
//     inside the 12 a band holds.
// Prints "stream sched: ok" and exits 0, or names the first failure.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "swa_sched.h"

using swa::SeqSched;
using swa::StreamSched;

static int fails = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      if (fails++ < 10) {                                 \
        std::printf("FAILED %s: ", #cond);                \
        std::printf(__VA_ARGS__);                         \
        std::printf("\n");                                \
      }                                                   \
    }                                                     \
  } while (0)

// the mask, written out: causal with an inclusive left window W
static bool visible(int lq, int lk, int diag, int W, int row, int key) {
  if (row < 0 || row >= lq || key < 0 || key >= lk) return false;
  const int a = row + diag;
  return key <= a && a - key <= W;
}

static void check_case(int lq, int lk, int W, int br) {
  StreamSched s;
  s.init(lq, lk, br, W);
  SeqSched g;
  g.init(lq, lk, br, 1, W, 0, 64, 128);
  CHECK(s.n_q_tiles == g.n_q_tiles && s.n_kv_tiles == g.n_kv_tiles, "lq %d lk %d", lq, lk);
  const int nq = s.n_q_tiles, nk = s.n_kv_tiles, diag = s.diag;
  for (int j = 0; j <= nk; ++j) {
    if (j < nk) {
      CHECK(s.q_lo(j) == g.q_lo(j), "q_lo(%d) lq %d lk %d W %d br %d", j, lq, lk, W, br);
      CHECK(s.q_hi(j) == g.q_hi(j), "q_hi(%d) lq %d lk %d W %d br %d", j, lq, lk, W, br);
    }
    CHECK(s.n_iters(j) == g.n_iters(j), "n_iters(%d) lq %d lk %d W %d br %d", j, lq, lk, W, br);
    CHECK(s.n_iters(j) <= 5, "n_iters(%d) = %d > 5", j, s.n_iters(j));
  }
  for (int i = 0; i < nq; ++i) {
    CHECK(s.kv_first(i) == g.kv_first(i), "kv_first(%d) lq %d lk %d W %d br %d", i, lq, lk, W, br);
    CHECK(s.kv_last(i) == g.kv_last(i), "kv_last(%d) lq %d lk %d W %d br %d", i, lq, lk, W, br);
  }
  // retirement
  for (int j = 0; j + 1 < nk; ++j) {
    const int lo = s.q_lo(j), n = s.n_iters(j);
    int r = s.n_retire(j);
    r = r < 0 ? 0 : (r > n ? n : r);
    for (int k = 0; k < n; ++k)
      CHECK((k < r) == (s.kv_last(lo + k) <= j), "retire j %d k %d lq %d lk %d W %d br %d", j, k, lq, lk, W, br);
  }
  for (int i = 0; i < nq; ++i) {
    if (s.kv_last(i) < s.kv_first(i)) continue;  // never visited
    const int j = s.kv_last(i);
    CHECK(i >= s.q_lo(j) && i < s.q_lo(j) + s.n_iters(j), "q-tile %d not fed by its last visitor %d", i, j);
    if (j + 1 < nk) {
      const int r = s.n_retire(j);
      CHECK(i - s.q_lo(j) < r, "q-tile %d not retired by its last visitor %d", i, j);
    }
  }
  // every visible pair: q-tile, band and dQ round
  for (int key = 0; key < lk; ++key) {
    const int j = key >> 7, kv0 = j * 128, v = (key - kv0) >> 4, ks = v >> 1;
    const int qlo = s.q_lo(j), n = s.n_iters(j), qhi = qlo + n;
    const int blo = s.band_lo(kv0 + 16 * v), bhi = s.band_hi(kv0 + 16 * v, qhi);
    const int nb = s.dq_nb(j);
    CHECK(nb + 1 <= 11, "dq_nb(%d) = %d", j, nb);
    if (bhi >= blo) CHECK(bhi - blo + 1 <= 10, "band of %d blocks", bhi - blo + 1);
    const int rlo = key - diag, rhi = key - diag + W;
    for (int row = rlo < 0 ? 0 : rlo; row <= rhi && row < lq; ++row) {
      if (!visible(lq, lk, diag, W, row, key)) continue;
      const int i = row >> 6, k = i - qlo, wr = (row & 63) >> 4, bb = row >> 4;
      CHECK(k >= 0 && k < n, "pair (%d, %d) outside step %d's q-tiles", row, key, j);
      CHECK(bb >= blo && bb <= bhi, "pair (%d, %d) outside its band [%d, %d]", row, key, blo, bhi);
      CHECK(bb - blo < 10, "pair (%d, %d) past the band's 10 blocks", row, key);
      const int c0 = s.dq_c0(j, wr);
      const int klo = s.dq_klo(c0, ks), khi = s.dq_khi(c0, nb, ks, n);
      CHECK(k >= klo && k <= khi, "pair (%d, %d): dQ round k %d not in [%d, %d]", row, key, k, klo, khi);
      const int pa = 4 * k - 2 * ks + c0;
      CHECK(pa == 1 + bb - (blo - (v & 1)), "band position %d of row block %d", pa, bb);
    }
  }
  // rounds never read outside a band's 12 positions
  for (int j = 0; j < nk; ++j)
    for (int wr = 0; wr < 4; ++wr)
      for (int ks = 0; ks < 4; ++ks) {
        const int c0 = s.dq_c0(j, wr), nb = s.dq_nb(j), n = s.n_iters(j);
        for (int k = s.dq_klo(c0, ks); k <= s.dq_khi(c0, nb, ks, n); ++k) {
          const int pa = 4 * k - 2 * ks + c0;
          CHECK(pa >= 1 && pa <= 11, "round j %d wr %d ks %d k %d reads position %d", j, wr, ks, k, pa);
        }
      }
}

int main() {
  std::mt19937 rng(2024);
  int cases = 0;
  const int fixed[][4] = {{256, 256, 64, 0}, {4096, 4096, 128, 0}, {300, 700, 100, 1}, {777, 777, 128, 1},
                          {1, 1, 0, 0},      {0, 5, 3, 0},         {5, 0, 3, 1},       {640, 700, 61, 1},
                          {130, 130, 0, 0},  {2048, 2048, 128, 0}, {333, 500, 128, 1}, {64, 1000, 128, 1}};
  for (auto& c : fixed) {
    check_case(c[0], c[1], c[2], c[3]);
    ++cases;
  }
  for (int t = 0; t < 3000; ++t) {
    const int lq = rng() % 1200, lk = rng() % 1200, W = rng() % 129, br = rng() % 2;
    // (bottom-right with s_q > s_kv occurs per sequence in the packed layout)
    check_case(lq, lk, W, br);
    ++cases;
  }
  if (fails) {
    std::printf("stream sched: %d failures over %d cases\n", fails, cases);
    return 1;
  }
  std::printf("stream sched: ok (%d cases)\n", cases);
  return 0;
}
