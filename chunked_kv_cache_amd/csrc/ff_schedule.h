// Schedule of one attention call over n_wg persistent workgroups (one per
// CU), shared by the kernel, the merge kernel and the host-side checks.
// Plain integer arithmetic only; FF_HD marks the functions for both the
// device and the host compiler.
//
// Items run whole in full rounds (workgroup g takes item r*n_wg + g, so the
// workgroups of an XCD stream one head's K/V in lockstep).  The rem items of
// the last, partial round are cut along their key tiles into m = n_wg / rem
// levels and a remainder: level j is the tile range [F(j), F(j+1)) of every
// item, run by workgroups j*rem .. j*rem + rem-1 (again in lockstep, one item
// each); the remainders [F(m), ntiles) of all items, item-major, are cut into
// equal contiguous ranges for the n_wg - m*rem leftover workgroups, each of
// which runs several short pieces.  F(j) = j*rem*(ntiles + c)/n_wg with c =
// kPieceCost tiles, the cost of a piece's start and partial write, so that a
// level piece and a leftover range (with its pieces) take about as long.
// Every piece leaves a partial (O, m, l) in its own slot (level piece of
// workgroup g: slot g; remainder piece of item x in leftover range k: slot
// m*rem + x + k, below 2*n_wg) and the merge kernel combines an item's pieces
// in key order.
#pragma once

#include <cstdint>

#ifdef __HIPCC__
#define FF_HD __host__ __device__
#else
#define FF_HD
#endif

namespace ff {

constexpr int kPieceCost = 6;

struct LastRound {
  int full, rem, m, left, ntiles, n_wg;
  int fm;                          // F(m): first tile of the remainders
  int r;                           // remainder tiles per item
};

FF_HD inline int level_start(const LastRound& lr, int j) {
  if (j >= lr.m && lr.left == 0) return lr.ntiles;
  const int64_t f = int64_t(j) * lr.rem * (lr.ntiles + kPieceCost) / lr.n_wg;
  return f < lr.ntiles ? int(f) : lr.ntiles;
}

FF_HD inline LastRound last_round(int n_items, int ntiles, int n_wg) {
  LastRound lr;
  lr.full = n_items / n_wg;
  lr.rem = n_items % n_wg;
  lr.ntiles = ntiles;
  lr.n_wg = n_wg;
  lr.m = lr.rem ? n_wg / lr.rem : 0;
  lr.left = n_wg - lr.m * lr.rem;
  lr.fm = lr.rem ? level_start(lr, lr.m) : ntiles;
  lr.r = ntiles - lr.fm;
  return lr;
}

// Leftover range k in remainder units (rem * r of them).
FF_HD inline int64_t left_lo(const LastRound& lr, int k) {
  return int64_t(lr.rem) * lr.r * k / lr.left;
}

// The leftover range that holds remainder unit u.
FF_HD inline int left_of(const LastRound& lr, int64_t u) {
  int k = int(u * lr.left / (int64_t(lr.rem) * lr.r));
  while (k + 1 < lr.left && left_lo(lr, k + 1) <= u) ++k;
  while (k > 0 && left_lo(lr, k) > u) --k;
  return k;
}

// The pieces of workgroup g in order: whole items of the full rounds (slot
// -1), then its level piece or its leftover range.
struct PieceIter {
  int g, u = 0, k = 0;
  bool lev_todo = false;
  int64_t pos = 0, hi = 0;
  FF_HD PieceIter(const LastRound& lr, int g_) : g(g_) {
    lev_todo = lr.rem && g < lr.m * lr.rem;
    k = g - lr.m * lr.rem;
    if (lr.rem && !lev_todo && lr.r > 0) {
      pos = left_lo(lr, k);
      hi = left_lo(lr, k + 1);
    }
  }
  // Next piece: item, key tiles [t_begin, t_end), partial slot (or -1).
  // False when the workgroup has no more.
  FF_HD bool next(const LastRound& lr, int& item, int& t_begin, int& t_end, int& slot) {
    t_begin = 0;
    t_end = lr.ntiles;
    slot = -1;
    if (u < lr.full) {
      item = u * lr.n_wg + g;
      ++u;
      return true;
    }
    if (lev_todo) {
      lev_todo = false;
      const int j = g / lr.rem, x = g % lr.rem;
      t_begin = level_start(lr, j);
      t_end = level_start(lr, j + 1);
      if (t_begin >= t_end) return false;
      item = lr.full * lr.n_wg + x;
      slot = g;
      return true;
    }
    if (pos < hi) {
      const int x = int(pos / lr.r);
      const int64_t off = pos - int64_t(x) * lr.r;
      const int64_t end = (hi - int64_t(x) * lr.r) < lr.r ? (hi - int64_t(x) * lr.r) : int64_t(lr.r);
      t_begin = lr.fm + int(off);
      t_end = lr.fm + int(end);
      item = lr.full * lr.n_wg + x;
      slot = lr.m * lr.rem + x + k;
      pos = int64_t(x) * lr.r + end;
      return true;
    }
    return false;
  }
};

// Pieces of last-round item x for the merge, in key order: candidate n <
// merge_candidates() is the non-empty level n (slot n*rem + x) or leftover
// range k0 + n - m holding part of x's remainder (slot m*rem + x + k); an
// empty candidate gives -1.
struct MergeList {
  int x, k0 = 0, k1 = -1;
  FF_HD MergeList(const LastRound& lr, int x_) : x(x_) {
    if (lr.r > 0) {
      k0 = left_of(lr, int64_t(x) * lr.r);
      k1 = left_of(lr, int64_t(x) * lr.r + lr.r - 1);
    }
  }
  FF_HD int count(const LastRound& lr) const { return lr.m + (k1 - k0 + 1); }
  FF_HD int slot(const LastRound& lr, int n) const {
    if (n < lr.m) return level_start(lr, n) < level_start(lr, n + 1) ? n * lr.rem + x : -1;
    const int kk = k0 + (n - lr.m);
    return left_lo(lr, kk) < left_lo(lr, kk + 1) ? lr.m * lr.rem + x + kk : -1;
  }
};

}  // namespace ff
