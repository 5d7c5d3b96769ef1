// Arguments, work items and tile loads of the block-sparse backward kernels.
#pragma once

#include "attn_tile.hpp"
#include "internal.hpp"

namespace bsattn {
namespace bwd {

template <int D>
constexpr int kTileOf = kBlock * D;   // floats in one 64 x D partial tile

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* o_lo;   // bf16 rounding residual of O, or null
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dbuf;      // D [B*H*n]
  float* part_q;    // [B*H*g*nseg][64][d]
  float* part_kv;   // [B*H*g*nseg][2][64][d]
  const int32_t* col_idx;
  const int32_t* csc_idx;
  const int32_t* gblk;
  const int32_t* row_info;   // [heads][nb - g][4] non-global row records
  const int32_t* col_info;   // [heads][nb - g][4] non-global column records, dK/dV order
  int heads, n, nb, g, seg, nseg, split;
  int last_rows;   // tokens in the last block: n - 64 (nb - 1), 1..64
  int items_per_bh, total_items;
  float scale, sl2, inv_scale;   // scale, scale*log2(e), 1/scale
};

// Tile loads for a sequence that may end inside its last block (kRagged): that
// block's missing rows are not read and stage as zeros.  The kernels below are
// instantiated with and without those guards; the whole-block instance has none.
template <bool kRagged, int D>
__device__ __forceinline__ void load_block(TileRegsT<D>& r, const uint16_t* base, int blk,
                                           const BwdArgs& a, int tid) {
  const uint16_t* g = base + (size_t)blk * kBlock * D;
  if (kRagged && blk == a.nb - 1) gload_nat_rows(r, g, tid, a.last_rows);
  else gload_nat(r, g, tid);
}

struct Item {
  int bh, h, blk, start, len, slot, seg;
  int first;   // first listed block
  bool full;   // the list is every block in order (a global row or column)
  // block of list entry t, given the list (read only for a list that is not full)
  __device__ __forceinline__ int at(const int32_t* list, int t) const {
    return full ? first + t : list[t];
  }
};

// Item v of a per-(batch, head) list: non-global blocks first (whole list), then
// each global block's segments of a.seg blocks.  A non-global item comes from its
// record (row or column: block, list start, length, first listed block); a global
// row or column lists every block in order, so its segments need no lookup.
// kv: the dK/dV items, whose non-global key blocks run longest column first
__device__ __forceinline__ Item decode(const BwdArgs& a, int v, bool kv) {
  Item it;
  it.bh = v / a.items_per_bh;
  const int r = v - it.bh * a.items_per_bh;
  it.h = it.bh % a.heads;
  const int ng = a.nb - a.g;
  it.seg = 0;
  it.slot = -1;
  if (r < ng) {
    const int4 rec = *reinterpret_cast<const int4*>((kv ? a.col_info : a.row_info) +
                                                    4 * ((int64_t)it.h * ng + r));
    it.blk = rec.x;
    it.start = rec.y;
    it.len = rec.z;
    it.first = rec.w;
    it.full = false;
  } else {
    const int gi = (r - ng) / a.nseg;
    const int s = (r - ng) - gi * a.nseg;
    it.blk = a.gblk[gi];
    it.seg = s;
    it.full = true;
    it.start = 0;
    if (a.split) {
      it.first = s * a.seg;
      it.len = min(a.seg, a.nb - s * a.seg);
      it.slot = (it.bh * a.g + gi) * a.nseg + s;
    } else {
      it.first = 0;
      it.len = a.nb;
    }
  }
  return it;
}

}  // namespace bwd
}  // namespace bsattn
