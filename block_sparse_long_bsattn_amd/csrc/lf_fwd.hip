// Longformer sliding-window + symmetric global attention forward on gfx950.
// Head dimension d = 64 (every configuration on the pages) or 128: one template,
// the d-wide loops unrolled per instance.
//
// Pattern ("Longformer: The Long-Document Transformer", §3.1 "Sliding Window",
// "Dilated Sliding Window" and "Global Attention"; the autoregressive mode of
// §4.1): token p attends to token q iff q is in p's window (q = p + k*(d+1) with
// k in [-w1, w1], or in [-w1, 0] when causal; d is the head's dilation), or p is
// global, or q is global.  Scores are scaled as in §3.1 eq. (1).  §3.2 and App. A
// describe the band as a banded matrix product that only computes a fixed number
// of diagonals; here each residue class of the window is walked in 64x64 tiles.
//
// Kernels (per call):
//   lf_attn     one 128-thread work-group per item, two kinds of item:
//               * a 64-row query tile of one residue class: the class's key tiles
//                 that overlap the window, then the tiles of global keys (rows
//                 gathered by index from K and V) that those tiles do not hold.
//                 Only tiles the window cuts need an element mask; keys that are
//                 global are allowed in every tile.  Rows of global tokens and
//                 rows past the class's end are not written.
//               * a segment of key tiles (8 to 64, sized per call from the work
//                 per work-group slot) for a tile of global query rows
//                 (a global token attends to every token), query rows gathered by
//                 index, writing a partial record.  With separate global
//                 projections (§3.1 "Linear Projections for Global Attention") these
//                 rows read Q_g, K_g, V_g instead of Q, K, V.
//   lf_fold     (past 16 segments only) folds runs of consecutive partial records into
//               one each, over many work-groups, so that the merge below stays short.
//   lf_combine  merges those partials in a fixed order and scatters O and lse back
//               to the global tokens' positions.

#include "attn_tile.hpp"
#include "fold.hpp"
#include "internal.hpp"
#include "lf_tile.hpp"

namespace bsattn {
namespace {

constexpr int kThreads = 128;

struct LfArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* qg;   // projections of the global rows' attention (q, k, v unless
  const uint16_t* kg;   // separate global projections are given)
  const uint16_t* vg;
  uint16_t* o;
  uint16_t* o_lo;       // bf16 rounding residual of O, or null
  float* lse;
  float* part;          // [B*H*ngt*nseg] partial records of the global query rows
  const float* mpart;   // [B*H*ngt*mcount] records lf_combine merges: part, or its folds
  int mcount;
  const int32_t* gtok;  // [ng]
  const int32_t* gidx;  // [n]
  const uint64_t* tile_gmask;  // [nt] bit x set iff token 64u+x is global
  const LfTileRef* ct;  // [nct] class tiles of one head period
  int heads, n, nt, ng, ngt, nseg, rseg;   // global rows: nseg segments of rseg tiles
  int nct, ph;          // class tiles and heads per head period
  LfWindow win;         // key range of each row, in class indices
  int band_items, total_items;
  float sl2;
};

template <int D>
using LdsTileT = uint16_t[kBlock * kStrideOf<D>];

template <int D>
__device__ __forceinline__ void lf_band_item(const LfArgs& a, int v, LdsTileT<D>* sK,
                                             LdsTileT<D>* sV) {
  const int per = v / a.nct;
  const LfTileRef e = a.ct[v - per * a.nct];
  const int bh = per * a.ph + e.h;
  const int cls = e.c, stride = e.s, t = e.t, nc = e.nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const uint64_t vm_q = valid_rows(t, nc);
  const uint64_t gm_q = class_gbits(a.gidx, a.tile_gmask, a.ng, cls, stride, t, nc, lane);
  if (gm_q == vm_q) return;   // every row global: the global items own them
  const size_t bh_off = (size_t)bh * a.n * D;
  const int xq = 32 * wave + col;
  const int i = min(t * kBlock + xq, nc - 1);   // this lane's class index
  const int p = cls + stride * i;               // ... and its token

  bf16x8 qB[D / 16];
  {
    const uint16_t* qp = a.q + bh_off + (size_t)p * D + 8 * hl;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) qB[k] = ld16(qp + 16 * k);
  }
  const int ntc = (nc + kBlock - 1) / kBlock;
  int lo_u, hi_u;
  band_keys(a.win, t, nc, ntc, lo_u, hi_u);
  int klo, khi;   // this row's window, in class indices
  a.win.keys(i, klo, khi);
  const int nband = hi_u - lo_u + 1;
  const int ntile = nband + a.ngt;

  // Global tile gt contributes key j iff j < ng and no band tile holds that key.
  auto global_elig = [&](int gt) -> uint64_t {
    return global_outside(a.gtok, a.ng, gt, cls, stride, lo_u, hi_u, lane);
  };

  FwdStateT<D> st;
  fwd_state_init(st);
  auto tile_load = [&](int x, TileRegsT<D>& kr, TileRegsT<D>& vr) {
    if (x < nband) {
      gload_class(kr, a.k + bh_off, cls, stride, lo_u + x, nc, tid);
      gload_class(vr, a.v + bh_off, cls, stride, lo_u + x, nc, tid);
    } else {
      gload_gather(kr, a.k + bh_off, a.gtok, a.ng, x - nband, tid);
      gload_gather(vr, a.v + bh_off, a.gtok, a.ng, x - nband, tid);
    }
  };

  // The next tile at or after x, skipping global tiles with no eligible key; for a
  // global tile, el receives its eligible keys.
  auto next_tile = [&](int x, uint64_t& el) -> int {
    for (; x < ntile; ++x) {
      if (x < nband) return x;
      el = global_elig(x - nband);
      if (el != 0ull) return x;
    }
    return x;
  };
  // Keys of tile x this lane's row may attend to.  A band tile needs a mask where
  // the window cuts it or the class ends inside it (keys that are global are
  // allowed anywhere); a global tile has the eligible keys el of next_tile.
  // mask_issue reads the tile's global-row word, mask_done (every lane) applies it.
  struct TileMask {
    bool need;           // uniform: the tile needs a mask
    bool band;
    uint64_t bits;       // band: window and class-end bits; global tile: el
    ClassGBits g;        // band: the global rows of the tile
  };
  auto mask_issue = [&](int x, uint64_t el) -> TileMask {
    TileMask m{false, x < nband, el, ClassGBits{0ull, -1}};
    if (!m.band) {
      m.need = el != ~0ull;
      return m;
    }
    const int u = lo_u + x;
    const uint64_t vm = valid_rows(u, nc);
    m.need = !tiles_in_window(a.win, t, u) || vm != ~0ull;
    if (m.need) {
      const int j0 = u * kBlock;
      m.bits = bit_range(klo - j0, khi - j0) & vm;
      m.g = class_gbits_issue(a.gidx, a.tile_gmask, a.ng, cls, stride, u, nc, lane);
    }
    return m;
  };
  auto mask_done = [&](const TileMask& m) -> uint64_t {
    return m.band ? m.bits | class_gbits_done(m.g, a.ng, stride) : m.bits;
  };

  uint64_t el = ~0ull;   // eligible keys of tile x when it is a global tile
  int x = next_tile(0, el);
  TileRegsT<D> kr, vr;
  if (x < ntile) {
    tile_load(x, kr, vr);
    lds_store_nat(sK[0], kr, tid);
    lds_store_nat(sV[0], vr, tid);
  }
  // Drain the prologue's loads (Q): a wait for them left inside the loop would, with
  // the in-order load counter, also wait for each iteration's prefetch.  For the
  // same reason an iteration reads its tile's mask word before it issues the
  // prefetch, so that the wait for the word leaves the prefetch in flight.
  wait_all_loads();
  int cur = 0;
  while (x < ntile) {
    __syncthreads();
    uint64_t el_next = ~0ull;
    const int xn = next_tile(x + 1, el_next);
    const TileMask mk = mask_issue(x, el);
    if (xn < ntile) tile_load(xn, kr, vr);
    f32x16 s0, s1;
    qk_tile(sK[cur], qB, col, hl, s0, s1);
    if (mk.need) mask_rows(s0, s1, hl, mask_done(mk));
    bf16x8 pc[4];
    softmax_step(s0, s1, st, pc, a.sl2);
    pv_tile(sV[cur], pc, lane, st);
    if (xn < ntile) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
    cur ^= 1;
    x = xn;
    el = el_next;
  }

  const float l_tot = partner_sum(st.l), lb_tot = partner_sum(st.lb);
  if (((vm_q & ~gm_q) >> xq) & 1ull)
    write_o_bf16(st, l_tot, lb_tot, hl, a.o + bh_off + (size_t)p * D,
                 a.o_lo != nullptr ? a.o_lo + bh_off + (size_t)p * D : nullptr,
                 a.lse != nullptr ? a.lse + (size_t)bh * a.n + p : nullptr);
}

// Item v of the global rows: (bh, global tile gt, segment s of rseg key tiles).
template <int D>
__device__ __forceinline__ void lf_global_item(const LfArgs& a, int v, LdsTileT<D>* sK,
                                               LdsTileT<D>* sV) {
  const int per_bh = a.ngt * a.nseg;
  const int bh = v / per_bh;
  const int rem = v - bh * per_bh;
  const int gt = rem / a.nseg, s = rem - gt * a.nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)bh * a.n * D;
  const int qr = 32 * wave + col;

  bf16x8 qB[D / 16];
  {
    const uint16_t* qp = a.qg + bh_off + (size_t)global_token(a.gtok, a.ng, gt, qr) * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qB[c] = ld16(qp + 16 * c);
  }
  const int u_begin = s * a.rseg;
  const int u_end = min(a.nt, u_begin + a.rseg);
  FwdStateT<D> st;
  fwd_state_init(st);
  TileRegsT<D> kr, vr;
  gload_class(kr, a.kg + bh_off, 0, 1, u_begin, a.n, tid);
  gload_class(vr, a.vg + bh_off, 0, 1, u_begin, a.n, tid);
  lds_store_nat(sK[0], kr, tid);
  lds_store_nat(sV[0], vr, tid);
  wait_all_loads();   // Q: see lf_band_item
  for (int u = u_begin; u < u_end; ++u) {
    const int cur = (u - u_begin) & 1;
    __syncthreads();
    const bool more = u + 1 < u_end;
    if (more) {
      gload_class(kr, a.kg + bh_off, 0, 1, u + 1, a.n, tid);
      gload_class(vr, a.vg + bh_off, 0, 1, u + 1, a.n, tid);
    }
    f32x16 s0, s1;
    qk_tile(sK[cur], qB, col, hl, s0, s1);
    if (u == a.nt - 1) {   // keys past the end of a sequence that ends inside a tile
      const uint64_t vm = valid_rows(u, a.n);
      if (vm != ~0ull) mask_rows(s0, s1, hl, vm);
    }
    bf16x8 pc[4];
    softmax_step(s0, s1, st, pc, a.sl2);
    pv_tile(sV[cur], pc, lane, st);
    if (more) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
  }
  const float l_tot = partner_sum(st.l), lb_tot = partner_sum(st.lb);
  write_partial(st, l_tot, lb_tot, hl, qr, a.part + (size_t)v * kPartFloatsOf<D>);
}

// The global-row segments first (up to the average work of a work-group slot), then
// the band items, each kind spread over all XCDs.  D = 128 takes more than half the
// registers: one wave per SIMD.
template <int D>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void lf_attn_kernel(LfArgs a) {
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sK[2];
  __shared__ __attribute__((aligned(16))) LdsTileT<D> sV[2];
  const int gitems = a.total_items - a.band_items;
  const int v = xcd_remap_two(blockIdx.x, gitems, a.band_items);
  if (v < 0) return;
  if (v < gitems)
    lf_global_item<D>(a, v, sK, sV);
  else
    lf_band_item<D>(a, v - gitems, sK, sV);
}

// Thread t: global row t / 4 of the tile, columns 16 (t % 4) + 64 u .. +15.
template <int D>
__global__ __launch_bounds__(256) void lf_combine_kernel(LfArgs a) {
  const int idx = blockIdx.x;   // bh * ngt + gt
  const int bh = idx / a.ngt, gt = idx - bh * a.ngt;
  const int row = threadIdx.x >> 2, dq = (threadIdx.x & 3) * 16;
  const int j = gt * kBlock + row;
  if (j >= a.ng) return;
  const int tok = a.gtok[j];   // read alongside the partial records
  float M = 0.f, L = 0.f;
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    float acc[16], Lb;
    merge_partials<D>(a.mpart + (size_t)idx * a.mcount * kPartFloatsOf<D>, a.mcount, row,
                      dq + 64 * u, acc, M, L, Lb);
    const size_t off = ((size_t)bh * a.n + tok) * D + dq + 64 * u;
    store16_bf16_lo(a.o + off, a.o_lo != nullptr ? a.o_lo + off : nullptr, acc, 1.f / Lb);
  }
  if (a.lse != nullptr && (threadIdx.x & 3) == 0)
    a.lse[(size_t)bh * a.n + tok] = (M + __log2f(L)) * kLn2;
}

}  // namespace

size_t lf_workspace_bytes(const lfattn_plan* P, int batch, int heads, int d) {
  if (P->ng == 0) return 0;
  const size_t rec = d == 128 ? kPartFloatsOf<128> : kPartFloatsOf<kHead>;
  const int nseg = lf_row_seg(P, batch, heads).nseg;
  const Fold f = fold_plan(nseg);
  return (size_t)batch * heads * P->ngt * (nseg + (f.chunk ? f.nfold : 0)) * rec * sizeof(float);
}

int launch_lf_fwd(const lfattn_plan* P, int batch, int heads, int d, float scale, const void* q,
                  const void* k, const void* v, const void* qg, const void* kg,
                  const void* vg, void* o, float* lse, void* o_lo, void* ws,
                  hipStream_t stream) {
  LfArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.qg = (const uint16_t*)(qg != nullptr ? qg : q);
  a.kg = (const uint16_t*)(kg != nullptr ? kg : k);
  a.vg = (const uint16_t*)(vg != nullptr ? vg : v);
  a.o = (uint16_t*)o; a.o_lo = (uint16_t*)o_lo; a.lse = lse;
  const bool has_g = P->ng > 0;
  a.part = has_g ? (float*)ws : nullptr;
  a.gtok = P->d_gtok; a.gidx = P->d_gidx; a.tile_gmask = P->d_tile_gmask;
  a.ct = P->d_ct;
  a.heads = heads; a.n = P->n; a.nt = P->nt; a.ng = P->ng; a.ngt = P->ngt;
  const LfSeg rs = lf_row_seg(P, batch, heads);
  a.nseg = rs.nseg; a.rseg = rs.seg;
  a.nct = P->nct;
  a.ph = P->heads > 0 ? P->heads : 1;
  a.win = lf_window(P);
  a.sl2 = scale * kLog2e;
  const int bhn = batch * heads;
  const Fold fold = fold_plan(a.nseg);
  const size_t rec = d == 128 ? kPartFloatsOf<128> : kPartFloatsOf<kHead>;
  a.mpart = fold.chunk && has_g ? a.part + (size_t)bhn * P->ngt * a.nseg * rec : a.part;
  a.mcount = fold.nfold;
  a.band_items = bhn / a.ph * P->nct;
  a.total_items = a.band_items + (has_g ? bhn * P->ngt * a.nseg : 0);
  int st;
  {
    ProfScope prof_(d == 128 ? "lf_attn_d128" : "lf_attn", stream);
    const dim3 grid(8 * ((a.band_items + 7) / 8 + (a.total_items - a.band_items + 7) / 8));
    if (d == 128)
      hipLaunchKernelGGL(lf_attn_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(lf_attn_kernel<kHead>, grid, dim3(kThreads), 0, stream, a);
  }
  if ((st = check_hip(hipGetLastError(), "lf_attn launch"))) return st;
  if (!has_g) return 0;
  if (fold.chunk) {
    ProfScope prof_("lf_fold", stream);
    float* dst = const_cast<float*>(a.mpart);
    const int groups = bhn * P->ngt * fold.nfold;
    if (d == 128)
      hipLaunchKernelGGL(fold_softmax_kernel<128>, dim3(groups * 8), dim3(256), 0, stream, a.part,
                         dst, a.nseg, fold.chunk, fold.nfold);
    else
      hipLaunchKernelGGL(fold_softmax_kernel<kHead>, dim3(groups * 4), dim3(256), 0, stream,
                         a.part, dst, a.nseg, fold.chunk, fold.nfold);
    if ((st = check_hip(hipGetLastError(), "lf_fold launch"))) return st;
  }
  {
    ProfScope prof_("lf_combine", stream);
    if (d == 128)
      hipLaunchKernelGGL(lf_combine_kernel<128>, dim3(bhn * P->ngt), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(lf_combine_kernel<kHead>, dim3(bhn * P->ngt), dim3(256), 0, stream, a);
  }
  return check_hip(hipGetLastError(), "lf_combine launch");
}

}  // namespace bsattn
