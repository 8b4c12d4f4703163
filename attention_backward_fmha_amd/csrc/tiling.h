// tiling.h -- mask geometry and tile ranges shared by the host plan and the kernels.
//
// One definition of "which query blocks does key tile j touch" serves the main kernel (which
// writes a dQ partial for every such block) and the reduction kernel (which sums exactly those
// partials), so the two can never disagree about which accumulator slots hold data.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define FMHA_HD __host__ __device__ inline
#else
#define FMHA_HD inline
#endif

namespace fmha {

// Key j is allowed for query i of a segment with lengths (lq, lk) iff 0 <= j < lk and
//   (left < 0 || j >= i + delta - left) && (right < 0 || j <= i + delta + right).
// Mask numbering: 0 none, 1 causal top-left, 2 causal bottom-right, 3 window (aligned like
// bottom-right causal).
struct MaskGeom {
  int64_t delta;
  int64_t left;
  int64_t right;
};

FMHA_HD MaskGeom mask_geom(int type, int window_left, int window_right, int64_t lq, int64_t lk) {
  MaskGeom g;
  g.delta = 0;
  g.left = -1;
  g.right = -1;
  if (type == 1) {
    g.right = 0;
  } else if (type == 2) {
    g.delta = lk - lq;
    g.right = 0;
  } else if (type == 3) {
    g.delta = lk - lq;
    g.left = window_left;
    g.right = window_right;
  }
  return g;
}

FMHA_HD bool pair_allowed(const MaskGeom& g, int64_t i, int64_t j, int64_t lq, int64_t lk) {
  if (i < 0 || i >= lq || j < 0 || j >= lk) return false;
  if (g.left >= 0 && j < i + g.delta - g.left) return false;
  if (g.right >= 0 && j > i + g.delta + g.right) return false;
  return true;
}

// Query rows that may attend to some key in [k0, k1] (inclusive, k1 < lk): [*lo, *hi]; empty
// when *lo > *hi.  Every key's row set is an interval shifted by one per key, so the union
// over the key range is one interval.
FMHA_HD void rows_for_keys(const MaskGeom& g, int64_t lq, int64_t k0, int64_t k1, int64_t* lo,
                           int64_t* hi) {
  int64_t a = 0, b = lq - 1;
  if (g.right >= 0) {
    const int64_t t = k0 - g.delta - g.right;
    a = t > a ? t : a;
  }
  if (g.left >= 0) {
    const int64_t t = k1 - g.delta + g.left;
    b = t < b ? t : b;
  }
  *lo = a;
  *hi = b;
}

// Query blocks [*qb_lo, *qb_hi] that key tile `tile` (keys [tile*tn, tile*tn + tn) clipped to
// lk) touches; empty when *qb_lo > *qb_hi.
FMHA_HD void qblocks_for_tile(const MaskGeom& g, int64_t lq, int64_t lk, int tile, int tm,
                              int tn, int64_t* qb_lo, int64_t* qb_hi) {
  const int64_t k0 = (int64_t)tile * tn;
  int64_t k1 = k0 + tn - 1;
  if (k1 > lk - 1) k1 = lk - 1;
  *qb_lo = 1;
  *qb_hi = 0;
  if (k0 > k1 || lq <= 0) return;
  int64_t lo, hi;
  rows_for_keys(g, lq, k0, k1, &lo, &hi);
  if (lo > hi) return;
  *qb_lo = lo / tm;
  *qb_hi = hi / tm;
}

// True when every (row, key) in rows [r0, r1] x keys [c0, c1] is allowed.
FMHA_HD bool block_full(const MaskGeom& g, int64_t lq, int64_t lk, int64_t r0, int64_t r1,
                        int64_t c0, int64_t c1) {
  if (r1 >= lq || c1 >= lk || r0 < 0 || c0 < 0) return false;
  if (g.left >= 0 && c0 < r1 + g.delta - g.left) return false;
  if (g.right >= 0 && c1 > r0 + g.delta + g.right) return false;
  return true;
}

// Allowed keys of row i (for FLOP accounting): count of j in [0, lk) passing the mask.
FMHA_HD int64_t keys_of_row(const MaskGeom& g, int64_t i, int64_t lk) {
  int64_t a = 0, b = lk - 1;
  if (g.left >= 0) {
    const int64_t t = i + g.delta - g.left;
    a = t > a ? t : a;
  }
  if (g.right >= 0) {
    const int64_t t = i + g.delta + g.right;
    b = t < b ? t : b;
  }
  return b >= a ? b - a + 1 : 0;
}

}  // namespace fmha
