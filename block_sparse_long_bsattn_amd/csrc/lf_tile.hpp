// Helpers shared by the Longformer forward and backward kernels.
//
// Windows ("Longformer: The Long-Document Transformer", §3.1 "Sliding Window" and
// "Dilated Sliding Window", Fig. 2(c)): with dilation d the window of token p holds
// the tokens p + k*(d+1) for k in [-w1, w1] (k in [-w1, 0] in the autoregressive
// mode of §4.1).  Tokens of one residue class modulo s = d + 1 only see their own
// class, so each class is a plain sliding window over its class indices
// (token = c + s * index), walked in 64-row class tiles (LfTileRef); the window is
// then the index difference range dlo <= i - j <= dhi.  The blocked window of the
// BigBird-ETC construction ("Big Bird", §2, App. E) is the other kind of LfWindow.
// Sequences need not fill their last 64-token tile: rows past the end are clamped
// on load and masked or skipped.
//
// Tiles whose rows are global tokens are gathered by index from the [n][d]
// tensors (d = 64, or 128 for the instances that take it).
#pragma once

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace bsattn {

// Segments of the global query rows (a global token attends to every token), per
// call: seg key tiles each, the largest power of two in kLfSeg..64 within the average
// work of one work-group slot (four per compute unit).  The segments run first on each
// XCD and so end within the run, while longer segments write and merge fewer fp32
// partials.  The work counted: every band item's window tiles and global tiles, and
// the global rows' tiles.
struct LfSeg {
  int seg, nseg;
};

inline LfSeg lf_row_seg(const lfattn_plan* P, int batch, int heads) {
  const int64_t bhn = (int64_t)batch * heads;
  const int64_t band_items = bhn / (P->heads > 0 ? P->heads : 1) * P->nct;
  const int64_t span = P->wb > 0 ? (int64_t)(2 * P->whalf + 1) * P->wb
                                 : (P->causal ? P->w1 + 1 : 2 * (int64_t)P->w1 + 1);
  const int64_t band_tiles = std::min<int64_t>(P->nt, (span + kBlock - 1) / kBlock + 1);
  const int64_t work = band_items * (band_tiles + P->ngt) + bhn * P->ngt * P->nt;
  const int64_t avg = work / (4 * (int64_t)(P->cus > 0 ? P->cus : 1));
  int seg = kLfSeg;
  while (seg < 64 && 2 * seg <= avg) seg *= 2;
  return LfSeg{seg, (P->nt + seg - 1) / seg};
}

// Segments of the columns of the key tiles holding global keys (every query tile
// sees a global key), per call: seg query tiles each, the smallest power of two in
// kLfSeg..64 above the average of those columns' tiles per work-group slot, and at
// most half a column.  They run in a kernel of their own; longer segments write and
// sum fewer fp32 partials.
inline LfSeg lf_col_seg(const lfattn_plan* P, int batch, int heads) {
  const int64_t periods = (int64_t)batch * heads / (P->heads > 0 ? P->heads : 1);
  const int64_t work = periods * (P->nct - P->nct_plain) * P->nt;
  const int64_t avg = work / (4 * (int64_t)(P->cus > 0 ? P->cus : 1));
  int seg = kLfSeg;
  while (seg < 64 && seg <= avg && 2 * seg < P->nt) seg *= 2;
  return LfSeg{seg, (P->nt + seg - 1) / seg};
}

// Two lists, n1 items and then n2: each XCD runs its eighth of the first list and
// then its eighth of the second, so that both kinds of item spread over all eight
// (eighths of the joined list would give the first XCDs only the first kind).
// Returns the item (the second list numbered from n1 on), or -1 for a work-group
// past the end of its XCD's share.  Grid: 8 * (ceil(n1/8) + ceil(n2/8)).
__device__ __forceinline__ int xcd_remap_two(int g, int n1, int n2) {
  const int p1 = (n1 + 7) / 8, p2 = (n2 + 7) / 8;
  const int x = g & 7, k = g >> 3;
  if (k < p1) {
    const int v = x * p1 + k;
    return v < n1 ? v : -1;
  }
  const int v = x * p2 + (k - p1);
  return v < n2 ? n1 + v : -1;
}

// Token behind row x of global tile gt: the (gt*64 + x)-th global token; rows past
// the last one repeat it (their keys or queries are masked out or not written).
__device__ __forceinline__ int global_token(const int32_t* gtok, int ng, int gt, int x) {
  return gtok[min(gt * kBlock + x, ng - 1)];
}

// gload_nat for a tile of global tokens, rows gathered from `base` ([n][D]).
template <int D>
__device__ __forceinline__ void gload_gather(TileRegsT<D>& r, const uint16_t* base,
                                             const int32_t* gtok, int ng, int gt, int tid) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  const int c = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
    r.v[u] = ldg16(base + (size_t)global_token(gtok, ng, gt, row + kRpp * u) * D + 8 * c);
}

// Token of row x of class tile t; rows past the class repeat its last token.
__device__ __forceinline__ int class_token(int c, int s, int t, int nc, int x) {
  return c + s * min(t * kBlock + x, nc - 1);
}

// gload_nat for class tile t: row x from token c + s*(64t + x) of `base` ([n][D]).
template <int D>
__device__ __forceinline__ void gload_class(TileRegsT<D>& r, const uint16_t* base, int c, int s,
                                            int t, int nc, int tid) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  const int k = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
    r.v[u] = ldg16(base + (size_t)class_token(c, s, t, nc, row + kRpp * u) * D + 8 * k);
}

// Bits [lo, hi] of a 64-bit word, clipped to [0, 63]; empty when hi < lo.
__device__ __forceinline__ uint64_t bit_range(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, kBlock - 1);
  if (hi < lo) return 0ull;
  return (~0ull >> (kBlock - 1 - hi)) & (~0ull << lo);
}

// Rows of class tile t that hold a token (class index below nc; nc > 64t).
__device__ __forceinline__ uint64_t valid_rows(int t, int nc) {
  const int m = nc - t * kBlock;
  return m >= kBlock ? ~0ull : (1ull << m) - 1;
}

// Word t of a read-only table, t the same in every lane, read as a scalar load
// (constant address space): it counts against the scalar/LDS counter, so waiting
// for it never waits for the vector loads in flight.
__device__ __forceinline__ uint64_t load_uniform_u64(const uint64_t* table, int t) {
  typedef const __attribute__((address_space(4))) uint64_t* ConstPtr;
  return ((ConstPtr)table)[t];
}

// Rows of class tile t that are global tokens.  Every lane of the wave must call
// it (a ballot, except for stride 1 where the natural tile mask is read).
__device__ __forceinline__ uint64_t class_gbits(const int32_t* gidx, const uint64_t* tile_gmask,
                                                int ng, int c, int s, int t, int nc, int lane) {
  if (ng == 0) return 0ull;
  if (s == 1) return load_uniform_u64(tile_gmask, t);
  const int i = t * kBlock + lane;
  return __ballot(i < nc && gidx[c + s * i] >= 0);
}

// class_gbits in two steps, for a loop that loads the word one iteration before it
// uses it: issue reads the per-lane data, done (called by every lane of the wave)
// turns it into the row bits.
struct ClassGBits {
  uint64_t w;   // stride 1: the tile's bit word
  int g;        // larger strides: this lane's row's index among the global tokens, or -1
};

__device__ __forceinline__ ClassGBits class_gbits_issue(const int32_t* gidx,
                                                        const uint64_t* tile_gmask, int ng,
                                                        int c, int s, int t, int nc, int lane) {
  ClassGBits r{0ull, -1};
  if (ng == 0) return r;
  if (s == 1) {
    r.w = load_uniform_u64(tile_gmask, t);
  } else {
    const int i = t * kBlock + lane;
    if (i < nc) r.g = gidx[c + s * i];
  }
  return r;
}

__device__ __forceinline__ uint64_t class_gbits_done(const ClassGBits& r, int ng, int s) {
  if (ng == 0) return 0ull;
  if (s == 1) return r.w;
  return __ballot(r.g >= 0);
}

// Which rows of global tile gt are global tokens that no tile of [lo, hi] in class
// (c, s) holds (inside, such a tile already counts them): bit x <-> row x.  Every
// lane of the wave must call it.
__device__ __forceinline__ uint64_t global_outside(const int32_t* gtok, int ng, int gt, int c,
                                                   int s, int lo, int hi, int lane) {
  const int j = gt * kBlock + lane;
  bool ok = false;
  if (j < ng) {
    const int rel = gtok[j] - c;
    int u = -1;   // tile within class c, -1 for another class
    if (s == 1)
      u = rel / kBlock;
    else if (rel >= 0 && rel % s == 0)
      u = rel / s / kBlock;
    ok = u < lo || u > hi;
  }
  return __ballot(ok);
}

// The window as a contiguous range per row, in class indices: the keys of row i and
// the rows whose window holds key j.  Both ends are non-decreasing in i (in j), so
// a tile's range runs from its first row's start to its last row's end.
//   relative (b == 0): i - j in [dlo, dhi] (sliding, dilated within a class, causal)
//   blocked  (b > 0): tokens from off on form blocks of b; a token of block k sees
//                     the tokens of blocks k - half .. k + half (the blocked window of
//                     "Big Bird", §2 and App. D, over the ordinary tokens of the ETC
//                     construction; tokens below off are global)
struct LfWindow {
  int dlo, dhi;
  int b, off, half;
  __device__ __forceinline__ void keys(int i, int& lo, int& hi) const {
    if (b == 0) {
      lo = i - dhi;
      hi = i - dlo;
    } else {
      const int k = (max(i, off) - off) / b;
      lo = off + b * (k - half);
      hi = off + b * (k + half + 1) - 1;
    }
  }
  __device__ __forceinline__ void rows(int j, int& lo, int& hi) const {
    if (b == 0) {
      lo = j + dlo;
      hi = j + dhi;
    } else {
      keys(j, lo, hi);   // the blocked window is symmetric
    }
  }
};

// The plan's window: relative (sliding, dilated, causal) or blocked (ETC).
inline LfWindow lf_window(const lfattn_plan* P) {
  LfWindow w;
  w.dlo = P->causal ? 0 : -P->w1;
  w.dhi = P->w1;
  w.b = P->wb;
  w.off = P->woff;
  w.half = P->whalf;
  return w;
}

// Key tiles holding a key in the window of some row of query tile t, among the
// ntc tiles of a class of nc indices.
__device__ __forceinline__ void band_keys(const LfWindow& w, int t, int nc, int ntc, int& lo,
                                          int& hi) {
  int a0, a1, b0, b1;
  w.keys(t * kBlock, a0, a1);
  w.keys(min(t * kBlock + kBlock - 1, nc - 1), b0, b1);
  lo = max(0, a0) / kBlock;
  hi = min(ntc - 1, b1 / kBlock);
}

// Query tiles holding a row whose window has a key of key tile u.
__device__ __forceinline__ void band_queries(const LfWindow& w, int u, int nc, int ntc, int& lo,
                                             int& hi) {
  int a0, a1, b0, b1;
  w.rows(u * kBlock, a0, a1);
  w.rows(min(u * kBlock + kBlock - 1, nc - 1), b0, b1);
  lo = max(0, a0) / kBlock;
  hi = min(ntc - 1, b1 / kBlock);
}

// Whether every (row of query tile tq, row of key tile tk) pair is in the window.
__device__ __forceinline__ bool tiles_in_window(const LfWindow& w, int tq, int tk) {
  // the first row's keys end earliest, the last row's keys start latest
  int a0, a1, b0, b1;
  w.keys(tq * kBlock, a0, a1);
  w.keys(tq * kBlock + kBlock - 1, b0, b1);
  return b0 <= tk * kBlock && a1 >= tk * kBlock + kBlock - 1;
}

// Sets score registers to -inf where `allowed` has no bit.  Register r of s0 holds
// tile row 8*(r/4) + 4*hl + r%4, of s1 that row + 32 (keys in the S^T layout of
// the forward and dQ kernels, queries in the S layout of the dK/dV kernel).
__device__ __forceinline__ void mask_rows(f32x16& s0, f32x16& s1, int hl, uint64_t allowed) {
  const uint64_t a = allowed >> (4 * hl);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int x = 8 * (r >> 2) + (r & 3);
    if (!((a >> x) & 1ull)) s0[r] = -INFINITY;
    if (!((a >> (32 + x)) & 1ull)) s1[r] = -INFINITY;
  }
}

}  // namespace bsattn
