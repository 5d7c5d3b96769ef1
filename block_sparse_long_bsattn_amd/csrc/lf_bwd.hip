// Longformer sliding-window + symmetric global attention backward on gfx950.
//
// The page gives the forward only ("Longformer: The Long-Document Transformer",
// §3.1 "Sliding Window", "Dilated Sliding Window" and "Global Attention", eq. (1);
// the autoregressive mode of §4.1); this is its exact gradient, recomputing
// P = exp(scale * Q K^T - lse) from the saved log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// where token p attends to token q iff q is in p's (dilated, possibly causal)
// window, or p is global, or q is global.  Each residue class of a dilated window
// is walked in its own 64-row class tiles.  No atomics: every output tile has one
// owner.
//
// Kernels (per call):
//   lf_bwd_dq    row-owned, two kinds of item:
//                * a 64-row query class tile (not made only of global tokens): its
//                  window's key tiles, then the tiles of global keys outside them
//                  (rows gathered by index), as in the forward; writes dQ and D
//                  for its non-global rows (rowsum(dO * O) corrected by the row
//                  sum of dS: sum P * dP with the recomputed probabilities);
//                * a segment of rseg key tiles (as in the forward) for a tile of
//                  global query rows (full rows): writes D (first segment) and an
//                  fp32 partial dQ.
//   lf_bwd_dkdv  column-owned, two kinds of item:
//                * a 64-key class tile holding no global key: the query tiles of
//                  its class within the window, then the global query rows
//                  outside them (gathered);
//                * a segment of cseg natural query tiles (sized per call) for a key
//                  class tile holding global keys (their columns are full): fp32
//                  partial dK, dV.
//   lf_bwd_fold    (past 16 segments only) folds runs of consecutive partials into one
//                  each, over many work-groups, so that the sums below stay short.
//   lf_bwd_reduce  sums the partials in segment order and writes dQ of the
//                global rows and dK, dV of the key class tiles holding global keys.

#include "attn_tile.hpp"
#include "fold.hpp"
#include "internal.hpp"
#include "lf_tile.hpp"

namespace bsattn {
namespace {

constexpr int kThreads = 128;
template <int D>
constexpr int kTileOf = kBlock * D;   // floats of one fp32 partial tile

struct LfBwdArgs {
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
  // projections of the global rows' attention and their gradients: the same as
  // q, k, v, dq, dk, dv unless separate global projections are given (gproj)
  const uint16_t* qg;
  const uint16_t* kg;
  const uint16_t* vg;
  uint16_t* dqg;
  uint16_t* dkg;
  uint16_t* dvg;
  int gproj;
  float* dbuf;       // D [B*H*n]
  float* part_q;     // [B*H*ngt*nseg][64][d] dQ of the global query rows
  float* part_kv;    // [periods*nct_g*cnseg][2][64][d] dK, dV of key class tiles
  const float* red_q;   // what lf_bwd_reduce sums: part_q, or its folds (rq_n per tile)
  const float* red_kv;  // part_kv, or its folds (rkv_n per tile)
  int rq_n, rkv_n;
                     // holding global keys
  const int32_t* gtok;         // [ng]
  const int32_t* gidx;         // [n]
  const uint64_t* tile_gmask;  // [nt]
  const LfTileRef* ct;         // [nct]: class tiles without global keys, then those with
  int heads, n, nt, ng, ngt;
  int nseg, rseg;   // global query rows: nseg segments of rseg key tiles
  int cnseg, cseg;  // columns holding global keys: cnseg segments of cseg query tiles
  int nct, nct_plain, nct_g, ph;   // class tiles (all / without / with global keys), heads
                                   // per head period
  LfWindow win;                    // key range of each row, in class indices
  int dq_band_items, dq_items;
  int kv_plain_items, kv_items;   // lf_bwd_dkdv_kernel: window items, then global-row items
  int kv_seg_items;               // lf_bwd_dkdv_seg_kernel: global-column segments
  float scale, sl2, inv_scale;   // scale, scale*log2(e), 1/scale
};

// ---------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------

template <int D>
using LdsTileT = uint16_t[kBlock * kStrideOf<D>];

// One dQ item; kBand: a 64-row query class tile (v indexes periods*nct), else a
// segment of a global query tile (v indexes B*H*ngt*nseg).  D: head dimension.
template <int D, bool kBand>
__device__ __forceinline__ void lf_bwd_dq_item(const LfBwdArgs& a, int v, LdsTileT<D>* sK,
                                               LdsTileT<D>* sV) {
  constexpr int kS = kStrideOf<D>, kC = D / 16, kT = D / 32;
  constexpr bool band = kBand;
  int bh, gt = 0, seg = 0;
  int cls = 0, stride = 1, t = 0, nc = a.n;   // class tile of a band item
  uint64_t vm_q = ~0ull, gm_q = 0ull;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (kBand) {
    const int per = v / a.nct;
    const LfTileRef e = a.ct[v - per * a.nct];
    bh = per * a.ph + e.h;
    cls = e.c; stride = e.s; t = e.t; nc = e.nc;
    vm_q = valid_rows(t, nc);
    gm_q = class_gbits(a.gidx, a.tile_gmask, a.ng, cls, stride, t, nc, lane);
    if (gm_q == vm_q) return;   // all rows global: the global items own them
  } else {
    const int per_bh = a.ngt * a.nseg;
    bh = v / per_bh;
    const int rem = v - bh * per_bh;
    gt = rem / a.nseg;
    seg = rem - gt * a.nseg;
  }
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)bh * a.n * D;
  const int xq = 32 * wave + col;
  // this lane's class index (band items) and query token
  const int i = band ? min(t * kBlock + xq, nc - 1) : 0;
  const int p = band ? cls + stride * i : global_token(a.gtok, a.ng, gt, xq);

  // key tiles: band items walk the window's class tiles [lo_u, hi_u], then the
  // global tiles with an eligible key; global items walk the rseg natural tiles of
  // their segment
  int lo_u = 0, hi_u = -1, ntile;
  int klo = 0, khi = -1;   // this row's window, in class indices (band items)
  if constexpr (kBand) {
    band_keys(a.win, t, nc, (nc + kBlock - 1) / kBlock, lo_u, hi_u);
    a.win.keys(i, klo, khi);
    ntile = hi_u - lo_u + 1 + a.ngt;
  } else {
    lo_u = seg * a.rseg;
    hi_u = min(a.nt, lo_u + a.rseg) - 1;
    ntile = hi_u - lo_u + 1;
  }
  const int nband = hi_u - lo_u + 1;
  // The next tile at or after x, skipping global tiles with no eligible key; for a
  // global tile, el receives its eligible keys.
  auto next_tile = [&](int x, uint64_t& el) -> int {
    for (; x < ntile; ++x) {
      if (x < nband) return x;
      el = global_outside(a.gtok, a.ng, x - nband, cls, stride, lo_u, hi_u, lane);
      if (el != 0ull) return x;
    }
    return x;
  };
  // Keys of tile x this lane's row may attend to, in two steps (see lf_band_item of
  // the forward): mask_issue reads the tile's global-row word before the iteration's
  // prefetch, mask_done (every lane) applies it.
  struct TileMask {
    bool need;      // uniform
    bool cut;       // a band tile the window cuts or the class ends in
    uint64_t bits;  // cut band tile: window and class-end bits; global tile: el
    ClassGBits g;
  };
  auto mask_issue = [&](int x, uint64_t el) -> TileMask {
    TileMask m{false, false, el, ClassGBits{0ull, -1}};
    if constexpr (kBand) {
      if (x >= nband) {
        m.need = el != ~0ull;
        return m;
      }
      const int u = lo_u + x;
      const uint64_t vm = valid_rows(u, nc);
      if (!tiles_in_window(a.win, t, u) || vm != ~0ull) {
        const int j0 = u * kBlock;
        m.need = m.cut = true;
        m.bits = bit_range(klo - j0, khi - j0) & vm;
        m.g = class_gbits_issue(a.gidx, a.tile_gmask, a.ng, cls, stride, u, nc, lane);
      }
    } else if (lo_u + x == a.nt - 1) {   // keys past the end of the sequence
      m.bits = valid_rows(a.nt - 1, a.n);
      m.need = m.bits != ~0ull;
    }
    return m;
  };
  auto mask_done = [&](const TileMask& m) -> uint64_t {
    return m.cut ? m.bits | class_gbits_done(m.g, a.ng, stride) : m.bits;
  };
  const uint16_t* kbase = (band ? a.k : a.kg) + bh_off;
  const uint16_t* vbase = (band ? a.v : a.vg) + bh_off;
  auto tile_load = [&](int x, TileRegsT<D>& kr, TileRegsT<D>& vr) {
    if (x < nband) {
      gload_class(kr, kbase, cls, stride, lo_u + x, nc, tid);
      gload_class(vr, vbase, cls, stride, lo_u + x, nc, tid);
    } else {
      gload_gather(kr, a.k + bh_off, a.gtok, a.ng, x - nband, tid);
      gload_gather(vr, a.v + bh_off, a.gtok, a.ng, x - nband, tid);
    }
  };

  uint64_t el = ~0ull;   // eligible keys of tile x when it is a global tile
  int x = next_tile(0, el);
  TileRegsT<D> kr, vr;
  if (x < ntile) tile_load(x, kr, vr);
  bf16x8 qB[kC], doB[kC];
  float dsum = 0.f;
  {
    const size_t off = bh_off + (size_t)p * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const u32x4 qv = ldg16((band ? a.q : a.qg) + off + 16 * c);
      const u32x4 dv = ldg16(a.dout + off + 16 * c);
      const u32x4 ov = ldg16(a.o + off + 16 * c);
      qB[c] = __builtin_bit_cast(bf16x8, qv);
      doB[c] = __builtin_bit_cast(bf16x8, dv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(ov[e]), dsum);
        dsum = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(ov[e]), dsum);
      }
      if (a.o_lo != nullptr) {   // O + its rounding residual: D to ~2^-17 relative
        const u32x4 rv = ldg16(a.o_lo + off + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dsum = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(rv[e]), dsum);
          dsum = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(rv[e]), dsum);
        }
      }
    }
  }
  const float Dq = partner_sum(dsum);   // D = rowsum(dO * O)
  // The first segment of a global query tile writes this D for the dK/dV kernels.  A
  // band item holds every key of its (non-global) rows and writes D after the loop,
  // corrected by the row sum of dS: that sum is sum P dP - D sum P, with the
  // probabilities P the backward itself recomputes, so D + sum dS is sum P dP free
  // of the bf16 rounding of the weights behind O.
  if (!band && seg == 0 && hl == 0) a.dbuf[(size_t)bh * a.n + p] = Dq;
  const float lse2 = a.lse[(size_t)bh * a.n + p] * kLog2e;
  if (x < ntile) {
    lds_store_nat(sK[0], kr, tid);
    lds_store_nat(sV[0], vr, tid);
  }
  wait_all_loads();

  f32x16 g[kT];   // dQ^T: g[t] holds d rows 32t..32t+31
#pragma unroll
  for (int t = 0; t < kT; ++t) g[t] = zero16();
  float ds_sum = 0.f;   // this half-lane's share of the row sum of dS (masked keys: 0)
  int cur = 0;
  while (x < ntile) {
    __syncthreads();
    uint64_t el_next = ~0ull;
    const int xn = next_tile(x + 1, el_next);
    const TileMask mk = mask_issue(x, el);
    if (xn < ntile) tile_load(xn, kr, vr);
    // S^T = K Q^T and dP^T = V dO^T  (rows = keys, columns = this lane's query)
    f32x16 s0 = zero16(), s1 = zero16(), p0 = zero16(), p1 = zero16();
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const bf16x8 k0 = ld16(sK[cur] + col * kS + 16 * c + 8 * hl);
      const bf16x8 k1 = ld16(sK[cur] + (32 + col) * kS + 16 * c + 8 * hl);
      const bf16x8 v0 = ld16(sV[cur] + col * kS + 16 * c + 8 * hl);
      const bf16x8 v1 = ld16(sV[cur] + (32 + col) * kS + 16 * c + 8 * hl);
      s0 = mfma32(k0, qB[c], s0);
      s1 = mfma32(k1, qB[c], s1);
      p0 = mfma32(v0, doB[c], p0);
      p1 = mfma32(v1, doB[c], p1);
    }
    if (mk.need) mask_rows(s0, s1, hl, mask_done(mk));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // P = 2^(S*scale*log2(e) - lse*log2(e)), the scale applied in fp32;
      // dS = P * (dP - D)
      s0[r] = fast_exp2(__builtin_fmaf(s0[r], a.sl2, -lse2)) * (p0[r] - Dq);
      s1[r] = fast_exp2(__builtin_fmaf(s1[r], a.sl2, -lse2)) * (p1[r] - Dq);
    }
    if constexpr (kBand) {
      float r0 = s0[0], r1 = s1[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        r0 += s0[r];
        r1 += s1[r];
      }
      ds_sum += r0 + r1;
    }
    // dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q]; K^T from transpose reads
    const bf16x8 dc[4] = {pack8(s0, 0), pack8(s0, 8), pack8(s1, 0), pack8(s1, 8)};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < kT; ++t) g[t] = mfma32(ld_tr8<D>(sK[cur], t, c, lane), dc[c], g[t]);
    if (xn < ntile) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
    cur ^= 1;
    x = xn;
    el = el_next;
  }

  const float sc = a.scale;
  if constexpr (kBand) {
    const float dfix = Dq + partner_sum(ds_sum);
    if (((vm_q & ~gm_q) >> xq) & 1ull) {   // rows of global tokens: global items
      if (hl == 0) a.dbuf[(size_t)bh * a.n + p] = dfix;
      uint16_t* op = a.dq + bh_off + (size_t)p * D + 4 * hl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          w[t][0] = pack_bf16x2(g[t][4 * j] * sc, g[t][4 * j + 1] * sc);
          w[t][1] = pack_bf16x2(g[t][4 * j + 2] * sc, g[t][4 * j + 3] * sc);
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) *reinterpret_cast<u32x2*>(op + 32 * t + 8 * j) = w[t];
      }
      if (a.gproj) {   // the global projections get nothing from this row
        uint16_t* zp = a.dqg + bh_off + (size_t)p * D + 4 * hl;
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < kT; ++t) *reinterpret_cast<u32x2*>(zp + 32 * t + 8 * j) = z;
      }
    }
  } else {
    const size_t slot = ((size_t)bh * a.ngt + gt) * a.nseg + seg;
    float* pp = a.part_q + slot * kTileOf<D> + xq * D + 4 * hl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 w[kT];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int t = 0; t < kT; ++t) w[t][e] = g[t][4 * j + e] * sc;
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pp + 32 * t + 8 * j) = w[t];
    }
  }
}

// D = 128 takes more than half the registers: one wave per SIMD.
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void lf_bwd_dq_kernel(LfBwdArgs a) {
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sK[2];
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sV[2];
  const int gitems = a.dq_items - a.dq_band_items;   // global-row segments first
  const int v = xcd_remap_two(blockIdx.x, gitems, a.dq_band_items);
  if (v < 0) return;
  if (v < gitems)
    lf_bwd_dq_item<D, false>(a, v, sK, sV);
  else
    lf_bwd_dq_item<D, true>(a, v - gitems, sK, sV);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

// Kinds of dK/dV item.
enum LfKvKind {
  kKvPlain = 0,   // a key class tile without global keys (v indexes periods*nct_plain)
  kKvSeg = 1,     // a segment of a key class tile holding global keys
  kKvGRows = 2,   // with separate global projections: a natural key tile against the
                  // global query rows only, giving dK_g, dV_g (v indexes B*H*nt)
};

template <int D, int kKind>
__device__ __forceinline__ void lf_bwd_dkdv_item(const LfBwdArgs& a, int v, LdsTileT<D>* sQ,
                                                 LdsTileT<D>* sO, float (*sL)[kBlock],
                                                 float (*sD)[kBlock]) {
  constexpr int kS = kStrideOf<D>, kC = D / 16, kT = D / 32;
  constexpr bool kPlain = kKind == kKvPlain;
  constexpr bool kGRows = kKind == kKvGRows;
  int per = 0, gki = 0, seg = 0, bh, cls = 0, stride = 1, u, nc = a.n;
  if constexpr (kGRows) {
    bh = v / a.nt;
    u = v - bh * a.nt;
  } else {
    LfTileRef ref;
    if constexpr (kPlain) {
      per = v / a.nct_plain;
      ref = a.ct[v - per * a.nct_plain];
    } else {
      const int per_p = a.nct_g * a.cnseg;
      per = v / per_p;
      const int rem = v - per * per_p;
      gki = rem / a.cnseg;
      seg = rem - gki * a.cnseg;
      ref = a.ct[a.nct_plain + gki];
    }
    bh = per * a.ph + ref.h;
    cls = ref.c; stride = ref.s; u = ref.t; nc = ref.nc;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)bh * a.n * D;
  const int kx = 32 * wave + col;                 // this lane's key within the tile
  const int jc = min(u * kBlock + kx, nc - 1);    // ... its class index
  const int q_tok = cls + stride * jc;            // ... and its token
  const bool key_valid = u * kBlock + kx < nc;
  int rlo, rhi;   // rows whose window holds this lane's key, in class indices
  a.win.rows(jc, rlo, rhi);
  bool key_global = false;
  if constexpr (kKind == kKvSeg)
    key_global = (class_gbits(a.gidx, a.tile_gmask, a.ng, cls, stride, u, nc, lane) >> kx) & 1ull;

  // query tiles: plain items walk the window's class tiles [lo, hi] of the key's
  // class, then the global tiles with an eligible row (none with separate global
  // projections: those rows are the global-row items'); segment items walk cseg
  // natural tiles (the column of a global key is full); global-row items walk the
  // global tiles only
  int lo, hi, ntile;
  int qc = cls, qs = stride, qnc = nc;   // class of the query tiles walked
  if constexpr (kPlain) {
    band_queries(a.win, u, nc, (nc + kBlock - 1) / kBlock, lo, hi);
    ntile = hi - lo + 1 + (a.gproj ? 0 : a.ngt);
  } else if constexpr (kGRows) {
    lo = 0;
    hi = -1;
    ntile = a.ngt;
  } else {
    qc = 0; qs = 1; qnc = a.n;
    lo = seg * a.cseg;
    hi = min(a.nt, lo + a.cseg) - 1;
    ntile = hi - lo + 1;
  }
  const int nband = hi - lo + 1;
  // The next tile at or after x, skipping global tiles with no eligible row; for a
  // global tile, el receives its eligible rows.
  auto next_tile = [&](int x, uint64_t& el) -> int {
    for (; x < ntile; ++x) {
      if (x < nband) return x;
      el = global_outside(a.gtok, a.ng, x - nband, cls, stride, lo, hi, lane);
      if (el != 0ull) return x;
    }
    return x;
  };
  // The global rows of a plain item's band tile, read before the iteration's
  // prefetch (see lf_band_item of the forward); a zero word when not needed.
  auto plain_gbits_issue = [&](int x) -> ClassGBits {
    ClassGBits g{0ull, -1};
    if constexpr (kPlain) {
      if (x < nband) {
        const int tq = lo + x;
        if (!tiles_in_window(a.win, tq, u) || valid_rows(tq, nc) != ~0ull || a.gproj)
          g = class_gbits_issue(a.gidx, a.tile_gmask, a.ng, cls, stride, tq, nc, lane);
      }
    }
    return g;
  };
  // Segment items test the dilated window in token coordinates: query rows whose
  // distance to the key is a multiple of the stride (bits 0, s, 2s, ... shifted).
  uint64_t stride_bits = 0ull;
  if constexpr (kKind == kKvSeg)
    for (int b = 0; b < kBlock; b += stride) stride_bits |= 1ull << b;
  const uint16_t* qbase = (kGRows ? a.qg : a.q) + bh_off;
  const uint16_t* dobase = a.dout + bh_off;
  const float* lbase = a.lse + (size_t)bh * a.n;
  const float* dbase = a.dbuf + (size_t)bh * a.n;
  // the lse and D of row tid (tid < 64), then the tile loads (issued last, so that a
  // wait for the small loads never has to wait for the tiles)
  auto tile_load = [&](int x, TileRegsT<D>& qr, TileRegsT<D>& dr, float& lv, float& dval) {
    const int tok_row = x < nband ? class_token(qc, qs, lo + x, qnc, tid & 63)
                                  : global_token(a.gtok, a.ng, x - nband, tid & 63);
    if (tid < kBlock) {
      lv = lbase[tok_row];
      dval = dbase[tok_row];
    }
    if (x < nband) {
      gload_class(qr, qbase, qc, qs, lo + x, qnc, tid);
      gload_class(dr, dobase, qc, qs, lo + x, qnc, tid);
    } else {
      gload_gather(qr, qbase, a.gtok, a.ng, x - nband, tid);
      gload_gather(dr, dobase, a.gtok, a.ng, x - nband, tid);
    }
  };

  uint64_t el = ~0ull;   // eligible rows of tile x when it is a global tile
  int x = next_tile(0, el);
  TileRegsT<D> qr, dr;
  float lv = 0.f, dval = 0.f;
  if (x < ntile) tile_load(x, qr, dr, lv, dval);
  bf16x8 kB[kC], vB[kC];
  {
    const size_t off = bh_off + (size_t)q_tok * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      kB[c] = ld16((kGRows ? a.kg : a.k) + off + 16 * c);
      vB[c] = ld16((kGRows ? a.vg : a.v) + off + 16 * c);
    }
  }
  // sL and sD hold -lse/scale and -D to seed S (raw score units; the scale is
  // applied in fp32 before the exponential) and dP
  if (x < ntile) {
    lds_store_nat(sQ[0], qr, tid);
    lds_store_nat(sO[0], dr, tid);
    if (tid < kBlock) { sL[0][tid] = -lv * a.inv_scale; sD[0][tid] = -dval; }
  }
  wait_all_loads();

  f32x16 dv[kT], dk[kT];   // dV^T, dK^T: tile t holds d rows 32t..32t+31
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    dv[t] = zero16();
    dk[t] = zero16();
  }
  int cur = 0;
  while (x < ntile) {
    __syncthreads();
    uint64_t el_next = ~0ull;
    const int xn = next_tile(x + 1, el_next);
    const ClassGBits gw = plain_gbits_issue(x);
    if (xn < ntile) tile_load(xn, qr, dr, lv, dval);
    // S[q][key] = Q K^T, dP[q][key] = dO V^T; rows = queries (2 tiles), column = key.
    // Row q of register r is 32*qt + 8*(r/4) + 4*hl + r%4.
    f32x16 s0, s1, p0, p1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sL[cur][8 * j + 4 * hl]);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sL[cur][32 + 8 * j + 4 * hl]);
      const f32x4 D0 = *reinterpret_cast<const f32x4*>(&sD[cur][8 * j + 4 * hl]);
      const f32x4 D1 = *reinterpret_cast<const f32x4*>(&sD[cur][32 + 8 * j + 4 * hl]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0[4 * j + e] = l0[e];
        s1[4 * j + e] = l1[e];
        p0[4 * j + e] = D0[e];
        p1[4 * j + e] = D1[e];
      }
    }
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const bf16x8 q0 = ld16(sQ[cur] + col * kS + 16 * c + 8 * hl);
      const bf16x8 q1 = ld16(sQ[cur] + (32 + col) * kS + 16 * c + 8 * hl);
      const bf16x8 o0 = ld16(sO[cur] + col * kS + 16 * c + 8 * hl);
      const bf16x8 o1 = ld16(sO[cur] + (32 + col) * kS + 16 * c + 8 * hl);
      s0 = mfma32(q0, kB[c], s0);
      s1 = mfma32(q1, kB[c], s1);
      p0 = mfma32(o0, vB[c], p0);
      p1 = mfma32(o1, vB[c], p1);
    }
    // allowed (query row of this tile, this lane's key): in the window, or the
    // query is global, or the key is global
    if (x < nband) {
      const int tq = lo + x, i0 = tq * kBlock;
      if constexpr (kPlain) {
        // with separate global projections the rows of global tokens are excluded
        const uint64_t vq = valid_rows(tq, nc);
        if (!tiles_in_window(a.win, tq, u) || vq != ~0ull || a.gproj) {
          const uint64_t win = bit_range(rlo - i0, rhi - i0) & vq;
          const uint64_t gq = class_gbits_done(gw, a.ng, stride);
          const uint64_t ok = a.gproj ? win & ~gq : win | gq;
          if (ok != ~0ull) mask_rows(s0, s1, hl, ok);
        }
      } else if constexpr (kKind == kKvSeg) {
        // natural query tile: the rows p = i0 + x whose window holds the key (tokens
        // cls + s*rlo .. cls + s*rhi at a multiple of s from it) or that are global;
        // every row for a global key; only rows before the end of the sequence
        const uint64_t vq = valid_rows(tq, a.n);
        const uint64_t gq = load_uniform_u64(a.tile_gmask, tq);
        if (key_global) {
          const uint64_t ok = a.gproj ? vq & ~gq : vq;
          if (ok != ~0ull) mask_rows(s0, s1, hl, ok);
        } else if (stride > 1 || vq != ~0ull || a.gproj || !tiles_in_window(a.win, tq, u)) {
          int r = (q_tok - i0) % stride;
          if (r < 0) r += stride;
          const uint64_t win = bit_range(cls + stride * rlo - i0, cls + stride * rhi - i0) &
                               (stride_bits << r);
          const uint64_t ok = (a.gproj ? win & ~gq : win | gq) & vq;
          mask_rows(s0, s1, hl, ok);
        }
      }
    } else if (el != ~0ull) {
      mask_rows(s0, s1, hl, el);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = fast_exp2(s0[r] * a.sl2);     // P
      s1[r] = fast_exp2(s1[r] * a.sl2);
      p0[r] *= s0[r];                       // dS = P * (dP - D)
      p1[r] *= s1[r];
    }
    // dV^T[d][key] += sum_q dO^T[d][q] P[q][key];  dK^T[d][key] += sum_q Q^T[d][q] dS[q][key]
    const bf16x8 pc[4] = {pack8(s0, 0), pack8(s0, 8), pack8(s1, 0), pack8(s1, 8)};
    const bf16x8 dc[4] = {pack8(p0, 0), pack8(p0, 8), pack8(p1, 0), pack8(p1, 8)};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int t = 0; t < kT; ++t) dv[t] = mfma32(ld_tr8<D>(sO[cur], t, c, lane), pc[c], dv[t]);
#pragma unroll
      for (int t = 0; t < kT; ++t) dk[t] = mfma32(ld_tr8<D>(sQ[cur], t, c, lane), dc[c], dk[t]);
    }
    if constexpr (kKind == kKvSeg) {
      // A column holding global keys sums over every row of the sequence, and with a
      // short window each row can put a large share of its mass on a global key:
      // then the bf16 rounding of P and dS (2^-9 relative per term) would add up
      // over n terms of dV and dK.  These items also feed the rounding residues,
      // P - bf16(P) and dS - bf16(dS) rounded to bf16, through the same products,
      // which leaves about 2^-17 relative per term.
      residue8(s0, pc[0], 0); residue8(s0, pc[1], 8);
      residue8(s1, pc[2], 0); residue8(s1, pc[3], 8);
      residue8(p0, dc[0], 0); residue8(p0, dc[1], 8);
      residue8(p1, dc[2], 0); residue8(p1, dc[3], 8);
      const bf16x8 pl[4] = {pack8(s0, 0), pack8(s0, 8), pack8(s1, 0), pack8(s1, 8)};
      const bf16x8 dl[4] = {pack8(p0, 0), pack8(p0, 8), pack8(p1, 0), pack8(p1, 8)};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int t = 0; t < kT; ++t) dv[t] = mfma32(ld_tr8<D>(sO[cur], t, c, lane), pl[c], dv[t]);
#pragma unroll
        for (int t = 0; t < kT; ++t) dk[t] = mfma32(ld_tr8<D>(sQ[cur], t, c, lane), dl[c], dk[t]);
      }
    }
    if (xn < ntile) {
      lds_store_nat(sQ[cur ^ 1], qr, tid);
      lds_store_nat(sO[cur ^ 1], dr, tid);
      if (tid < kBlock) { sL[cur ^ 1][tid] = -lv * a.inv_scale; sD[cur ^ 1][tid] = -dval; }
    }
    cur ^= 1;
    x = xn;
    el = el_next;
  }

  const float sc = a.scale;
  if constexpr (kKind != kKvSeg) {
    if (!key_valid) return;
    const size_t off = bh_off + (size_t)q_tok * D + 4 * hl;
    uint16_t* kp = (kGRows ? a.dkg : a.dk) + off;
    uint16_t* vp = (kGRows ? a.dvg : a.dv) + off;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x2 kw[kT], vw[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        kw[t][0] = pack_bf16x2(dk[t][4 * j] * sc, dk[t][4 * j + 1] * sc);
        kw[t][1] = pack_bf16x2(dk[t][4 * j + 2] * sc, dk[t][4 * j + 3] * sc);
      }
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        vw[t][0] = pack_bf16x2(dv[t][4 * j], dv[t][4 * j + 1]);
        vw[t][1] = pack_bf16x2(dv[t][4 * j + 2], dv[t][4 * j + 3]);
      }
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<u32x2*>(kp + 32 * t + 8 * j) = kw[t];
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<u32x2*>(vp + 32 * t + 8 * j) = vw[t];
    }
  } else {
    const size_t slot = ((size_t)per * a.nct_g + gki) * a.cnseg + seg;
    float* pk = a.part_kv + slot * 2 * kTileOf<D> + kx * D + 4 * hl;
    float* pv = pk + kTileOf<D>;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 kw[kT], vw[kT];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int t = 0; t < kT; ++t) kw[t][e] = dk[t][4 * j + e] * sc;
#pragma unroll
        for (int t = 0; t < kT; ++t) vw[t][e] = dv[t][4 * j + e];
      }
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pk + 32 * t + 8 * j) = kw[t];
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pv + 32 * t + 8 * j) = vw[t];
    }
  }
}

// The window and global-row items: built at 256 VGPRs with no spills, so they run
// two waves per SIMD, about 25 % faster than one.  (Asking for two waves
// explicitly makes the compiler spill two registers instead; the resource report
// of the build shows which one it got.)
template <int D>
__global__ __launch_bounds__(kThreads) void lf_bwd_dkdv_kernel(LfBwdArgs a) {
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sQ[2];
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sO[2];   // dO
  __shared__ __attribute__((aligned(16))) float sL[2][kBlock];   // -lse / scale
  __shared__ __attribute__((aligned(16))) float sD[2][kBlock];   // -D
  const int v = xcd_remap_two(blockIdx.x, a.kv_plain_items, a.kv_items - a.kv_plain_items);
  if (v < 0) return;
  if (v < a.kv_plain_items)
    lf_bwd_dkdv_item<D, kKvPlain>(a, v, sQ, sO, sL, sD);
  else
    lf_bwd_dkdv_item<D, kKvGRows>(a, v - a.kv_plain_items, sQ, sO, sL, sD);
}

// The segments of key class tiles holding global keys, a launch of their own: their
// residue products need more registers than the window items may use at two
// waves per SIMD.  Launched before lf_bwd_dkdv_kernel: they are few and as long as
// its items.
template <int D>
__global__ __launch_bounds__(kThreads) void lf_bwd_dkdv_seg_kernel(LfBwdArgs a) {
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sQ[2];
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sO[2];   // dO
  __shared__ __attribute__((aligned(16))) float sL[2][kBlock];   // -lse / scale
  __shared__ __attribute__((aligned(16))) float sD[2][kBlock];   // -D
  const int v = xcd_remap(blockIdx.x, a.kv_seg_items);
  if (v >= a.kv_seg_items) return;
  lf_bwd_dkdv_item<D, kKvSeg>(a, v, sQ, sO, sL, sD);
}

// Segment sums in segment order.  Work-groups [0, B*H*ngt): dQ of global tile gt,
// rows scattered to their tokens; then periods*nct_g*2: dK (kind 0) or dV (kind 1)
// of the key class tiles holding global keys, rows scattered to their tokens.
// Thread t sums 16 consecutive floats of the 64 x D tile at 16 t + 4096 u,
// u = 0 .. D/64 - 1.
template <int D>
__global__ __launch_bounds__(256) void lf_bwd_reduce_kernel(LfBwdArgs a, int nq_groups) {
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const int e0 = threadIdx.x * 16 + 4096 * u;
    const int row = e0 / D;
    const float* src;
    size_t stride;
    uint16_t* dst;
    if ((int)blockIdx.x < nq_groups) {
      const int idx = blockIdx.x;   // bh * ngt + gt
      const int bh = idx / a.ngt, gt = idx - bh * a.ngt;
      const int j = gt * kBlock + row;
      if (j >= a.ng) continue;
      src = a.red_q + (size_t)idx * a.rq_n * kTileOf<D> + e0;
      stride = kTileOf<D>;
      const size_t row_off = ((size_t)bh * a.n + a.gtok[j]) * D + (e0 % D);
      dst = a.dqg + row_off;
      if (a.gproj) {   // the window projections get nothing from a global row
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = 0.f;
        store16_bf16(a.dq + row_off, z, 1.f);
      }
    } else {
      const int w = blockIdx.x - nq_groups;
      const int kind = w & 1, idx = w >> 1;   // idx = period * nct_g + gki
      const int per = idx / a.nct_g, gki = idx - per * a.nct_g;
      const LfTileRef e = a.ct[a.nct_plain + gki];
      const int ci = e.t * kBlock + row;      // class index of this row
      if (ci >= e.nc) continue;
      const int bh = per * a.ph + e.h;
      src = a.red_kv + (size_t)idx * a.rkv_n * 2 * kTileOf<D> + kind * kTileOf<D> + e0;
      stride = 2 * kTileOf<D>;
      dst = (kind == 0 ? a.dk : a.dv) + ((size_t)bh * a.n + e.c + (size_t)e.s * ci) * D +
            (e0 % D);
    }
    float acc[16];
    sum_partials(src, stride, (int)blockIdx.x < nq_groups ? a.rq_n : a.rkv_n, acc);
    store16_bf16(dst, acc, 1.f);
  }
}

struct LfBwdWs {
  size_t dbuf, part_q, part_kv, fold_q, fold_kv, total;
};

LfBwdWs lf_bwd_ws_layout(const lfattn_plan* P, int batch, int heads, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t bh = (size_t)batch * heads;
  const size_t periods = bh / (P->heads > 0 ? P->heads : 1);
  const size_t tile = (size_t)kBlock * d;   // floats of one partial tile
  LfBwdWs w;
  w.dbuf = 0;
  w.part_q = up(bh * P->n * sizeof(float));
  const size_t tiles_q = bh * P->ngt, tiles_kv = periods * (P->nct - P->nct_plain);
  const Fold fq = fold_plan(lf_row_seg(P, batch, heads).nseg);
  const Fold fkv = fold_plan(lf_col_seg(P, batch, heads).nseg);
  const size_t rows = tiles_q * lf_row_seg(P, batch, heads).nseg;
  const size_t cols = tiles_kv * lf_col_seg(P, batch, heads).nseg;
  w.part_kv = up(w.part_q + rows * tile * sizeof(float));
  w.fold_q = up(w.part_kv + cols * 2 * tile * sizeof(float));
  w.fold_kv = up(w.fold_q + (fq.chunk ? tiles_q * fq.nfold * tile * sizeof(float) : 0));
  w.total = up(w.fold_kv + (fkv.chunk ? tiles_kv * fkv.nfold * 2 * tile * sizeof(float) : 0));
  return w;
}

template <int D>
int launch_lf_bwd_d(const LfBwdArgs& a, const lfattn_plan* P, int bhn, int periods,
                    hipStream_t stream) {
  int st;
  {
    ProfScope prof_(D == 128 ? "lf_bwd_dq_d128" : "lf_bwd_dq", stream);
    hipLaunchKernelGGL(lf_bwd_dq_kernel<D>,
                       dim3(8 * ((a.dq_band_items + 7) / 8 + (a.dq_items - a.dq_band_items + 7) / 8)),
                       dim3(kThreads), 0, stream, a);
  }
  if ((st = check_hip(hipGetLastError(), "lf_bwd_dq launch"))) return st;
  if (a.kv_seg_items > 0) {
    {
      ProfScope prof_(D == 128 ? "lf_bwd_dkdv_seg_d128" : "lf_bwd_dkdv_seg", stream);
      hipLaunchKernelGGL(lf_bwd_dkdv_seg_kernel<D>, dim3(8 * ((a.kv_seg_items + 7) / 8)),
                         dim3(kThreads), 0, stream, a);
    }
    if ((st = check_hip(hipGetLastError(), "lf_bwd_dkdv_seg launch"))) return st;
  }
  if (a.kv_items > 0) {
    {
      ProfScope prof_(D == 128 ? "lf_bwd_dkdv_d128" : "lf_bwd_dkdv", stream);
      const int kg = a.kv_items - a.kv_plain_items;
      hipLaunchKernelGGL(lf_bwd_dkdv_kernel<D>, dim3(8 * ((a.kv_plain_items + 7) / 8 + (kg + 7) / 8)),
                         dim3(kThreads), 0, stream, a);
    }
    if ((st = check_hip(hipGetLastError(), "lf_bwd_dkdv launch"))) return st;
  }
  const int nq_groups = bhn * P->ngt;
  const int groups = nq_groups + periods * a.nct_g * 2;
  if (groups == 0) return 0;
  const Fold fq = fold_plan(a.nseg), fkv = fold_plan(a.cnseg);
  const FoldSumJob jq = fold_sum_job(a.part_q, const_cast<float*>(a.red_q), nq_groups, a.nseg,
                                     fq, kTileOf<D>);
  const FoldSumJob jkv = fold_sum_job(a.part_kv, const_cast<float*>(a.red_kv),
                                      periods * a.nct_g, a.cnseg, fkv, 2 * kTileOf<D>);
  if (jq.blocks + jkv.blocks > 0) {
    {
      ProfScope prof_("lf_bwd_fold", stream);
      hipLaunchKernelGGL(fold_sum_kernel, dim3(jq.blocks + jkv.blocks), dim3(256), 0, stream, jq,
                         jkv);
    }
    if ((st = check_hip(hipGetLastError(), "lf_bwd_fold launch"))) return st;
  }
  {
    ProfScope prof_(D == 128 ? "lf_bwd_reduce_d128" : "lf_bwd_reduce", stream);
    hipLaunchKernelGGL(lf_bwd_reduce_kernel<D>, dim3(groups), dim3(256), 0, stream, a, nq_groups);
  }
  return check_hip(hipGetLastError(), "lf_bwd_reduce launch");
}
}  // namespace

size_t lf_bwd_workspace_bytes(const lfattn_plan* P, int batch, int heads, int d) {
  return lf_bwd_ws_layout(P, batch, heads, d).total;
}

int launch_lf_bwd(const lfattn_plan* P, int batch, int heads, int d, float scale, const void* q,
                  const void* k, const void* v, const void* qg, const void* kg,
                  const void* vg, const void* o, const void* o_lo, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, void* dqg, void* dkg,
                  void* dvg, void* ws, hipStream_t stream) {
  const LfBwdWs w = lf_bwd_ws_layout(P, batch, heads, d);
  char* base = (char*)ws;
  LfBwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o; a.o_lo = (const uint16_t*)o_lo; a.lse = lse;
  a.dout = (const uint16_t*)dout;
  a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
  a.gproj = qg != nullptr ? 1 : 0;
  a.qg = (const uint16_t*)(a.gproj ? qg : q);
  a.kg = (const uint16_t*)(a.gproj ? kg : k);
  a.vg = (const uint16_t*)(a.gproj ? vg : v);
  a.dqg = (uint16_t*)(a.gproj ? dqg : dq);
  a.dkg = (uint16_t*)(a.gproj ? dkg : dk);
  a.dvg = (uint16_t*)(a.gproj ? dvg : dv);
  a.dbuf = (float*)(base + w.dbuf);
  a.part_q = (float*)(base + w.part_q);
  a.part_kv = (float*)(base + w.part_kv);
  a.gtok = P->d_gtok; a.gidx = P->d_gidx; a.tile_gmask = P->d_tile_gmask;
  a.ct = P->d_ct;
  a.heads = heads; a.n = P->n; a.nt = P->nt; a.ng = P->ng; a.ngt = P->ngt;
  const LfSeg rs = lf_row_seg(P, batch, heads);
  const LfSeg cs = lf_col_seg(P, batch, heads);
  a.nseg = rs.nseg; a.rseg = rs.seg; a.cnseg = cs.nseg; a.cseg = cs.seg;
  const Fold fq = fold_plan(a.nseg), fkv = fold_plan(a.cnseg);
  a.red_q = fq.chunk ? (const float*)(base + w.fold_q) : a.part_q;
  a.red_kv = fkv.chunk ? (const float*)(base + w.fold_kv) : a.part_kv;
  a.rq_n = fq.nfold; a.rkv_n = fkv.nfold;
  a.nct = P->nct; a.nct_plain = P->nct_plain; a.nct_g = P->nct - P->nct_plain;
  a.ph = P->heads > 0 ? P->heads : 1;
  a.win = lf_window(P);
  a.scale = scale;
  a.sl2 = scale * kLog2e;
  a.inv_scale = 1.f / scale;
  const int bhn = batch * heads;
  const int periods = bhn / a.ph;
  a.dq_band_items = periods * a.nct;
  a.dq_items = a.dq_band_items + bhn * P->ngt * a.nseg;
  a.kv_plain_items = periods * a.nct_plain;
  a.kv_items = a.kv_plain_items + (a.gproj ? bhn * P->nt : 0);
  a.kv_seg_items = periods * a.nct_g * a.cnseg;
  return d == 128 ? launch_lf_bwd_d<128>(a, P, bhn, periods, stream)
                  : launch_lf_bwd_d<kHead>(a, P, bhn, periods, stream);
}

}  // namespace bsattn
