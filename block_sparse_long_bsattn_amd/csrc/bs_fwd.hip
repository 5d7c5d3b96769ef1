// BigBird-ITC block-sparse attention forward on gfx950.
//
// Computes, per (batch, head) and query block i, softmax over the keys of the
// blocks in N(i) of scale * Q K^T, times V ("Big Bird: Transformers for Longer
// Sequences", §2 eq. (AT) and App. D eq. (13), Fig. 6; scaled scores as in
// "Longformer: The Long-Document Transformer", §3.1 eq. (1)).
//
// Head dimension d = 64 (every configuration on the pages) or 128 (bf16 only):
// one kernel template, the d-wide loops unrolled per instance.
//
// Work decomposition (one 128-thread work-group = 2 waves = one 64-row query
// block; wave w owns query rows 32w .. 32w+31):
//   * a non-global query block is one item walking its whole key-block list;
//   * a global query block (a full row, App. D Fig. 6 "direct multiplication")
//     is split into segments of key blocks (their length set per call from the
//     total work) that write partial (unnormalised O, running max, running sum);
//     bs_fwd_combine merges them in a fixed order.  Each XCD starts the segments
//     of its share of the items before the other items.
// Per key block: K and V are staged through double-buffered LDS in natural
// layout; S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA (V^T read with
// LDS transpose reads); the online softmax runs in fp32 registers, one query per
// lane (column of the accumulator), 32 keys per lane and the other 32 in the
// partner lane l ^ 32.

#include <algorithm>

#include "attn_tile.hpp"
#include "fold.hpp"
#include "internal.hpp"

namespace bsattn {
namespace {

constexpr int kFwdThreads = 128;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  uint16_t* o_lo;   // bf16 rounding residual of O, or null
  float* lse;
  float* part;
  const int32_t* col_idx;
  const int32_t* row_info;   // [heads][nb - g][4] non-global row records
  const int32_t* gblk;
  int heads, n, nb, g, seg, nseg, split;
  int last_rows;   // tokens in the last block: n - 64 (nb - 1), 1..64
  int items_per_bh, total_items;
  float sl2;  // scale * log2(e)
};

struct Item {
  int bh, h, i, start, len, slot;
  int first;   // first key block of the item
  bool full;   // the row lists every key block in order (a global row)
  // key block of list entry t (the list is read only for a row that is not full)
  __device__ __forceinline__ int at(const int32_t* list, int t) const {
    return full ? first + t : list[t];
  }
};

// Item v of a per-(batch, head) list: non-global rows first (whole row, from the
// row's record: block, list start, length, first key block), then each global
// row's segments of a.seg key blocks; a global row lists every key block in
// order, so its segments need no lookup.
__device__ __forceinline__ Item decode_row_item(const FwdArgs& a, int v) {
  Item it;
  it.bh = v / a.items_per_bh;
  const int r = v - it.bh * a.items_per_bh;
  it.h = it.bh % a.heads;
  const int ng = a.nb - a.g;
  it.slot = -1;
  if (r < ng) {
    const int4 rec = *reinterpret_cast<const int4*>(a.row_info + 4 * ((int64_t)it.h * ng + r));
    it.i = rec.x;
    it.start = rec.y;
    it.len = rec.z;
    it.first = rec.w;
    it.full = false;
  } else {
    const int gi = (r - ng) / a.nseg;
    const int s = (r - ng) - gi * a.nseg;
    it.i = a.gblk[gi];
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

// kRagged: the sequence ends inside its last block (n % 64 != 0); the instance for
// whole blocks carries none of that block's masking and guards.  D: head dimension.
// gload_nat for a tile whose rows at or past `rows` are not tokens: those rows read
// row rows - 1 instead.  The values are finite and the caller masks those keys out
// (P = 0) or drops those query rows, so no per-row predicate or branch is needed.
template <int D>
__device__ __forceinline__ void gload_nat_clamp(TileRegsT<D>& r, const uint16_t* g, int tid,
                                                int rows) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  const int c = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) r.v[u] = ldg16(g + min(row + kRpp * u, rows - 1) * D + 8 * c);
}

template <int D, bool kRagged>
__global__ __launch_bounds__(kFwdThreads) void bs_fwd_bf16_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBlock * kStrideOf<D>];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBlock * kStrideOf<D>];

  const int v = xcd_item_long_first(blockIdx.x, a.total_items, a.items_per_bh, a.nb - a.g);
  if (v < 0) return;
  const Item it = decode_row_item(a, v);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)it.bh * a.n * D;
  const int qrow = it.i * kBlock + 32 * wave + col;   // token index of this lane's query
  const int32_t* keys = a.col_idx + it.start;
  const uint16_t* kbase = a.k + bh_off;
  const uint16_t* vbase = a.v + bh_off;
  const int len = it.len;
  auto kaddr = [&](int kb) { return kbase + (size_t)kb * kBlock * D; };
  auto vaddr = [&](int kb) { return vbase + (size_t)kb * kBlock * D; };
  // a sequence that ends inside its last block: that block's missing rows are not
  // read (their positions repeat the last token's row, one code path for every
  // tile), they are masked out as keys, and no output is written for them
  auto tile_load = [&](int kb, TileRegsT<D>& kr, TileRegsT<D>& vr) {
    if (kRagged) {
      const int rows = kb == a.nb - 1 ? a.last_rows : kBlock;
      gload_nat_clamp(kr, kaddr(kb), tid, rows);
      gload_nat_clamp(vr, vaddr(kb), tid, rows);
    } else {
      gload_nat(kr, kaddr(kb), tid);
      gload_nat(vr, vaddr(kb), tid);
    }
  };

  TileRegsT<D> kr, vr;
  int kb_cur = 0;
  if (len > 0) {
    kb_cur = it.first;
    tile_load(kb_cur, kr, vr);
  }
  int kb_next = len > 1 ? it.at(keys, 1) : 0;
  bf16x8 qB[D / 16];
  {
    // query rows past the end read the last token's row; their outputs are dropped
    const uint16_t* qp = a.q + bh_off + (size_t)(kRagged ? min(qrow, a.n - 1) : qrow) * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qB[c] = ld16(qp + 16 * c);
  }
  lds_store_nat(sK[0], kr, tid);
  lds_store_nat(sV[0], vr, tid);
  FwdStateT<D> st;
  fwd_state_init(st);
  for (int t = 0; t < len; ++t) {
    const int cur = t & 1;
    __syncthreads();
    const bool more = t + 1 < len;
    f32x16 s0, s1;
    qk_tile(sK[cur], qB, col, hl, s0, s1);
    if (kRagged && kb_cur == a.nb - 1) mask_keys_from(s0, s1, hl, a.last_rows);
    const int kb_after = kb_next;   // block of tile t + 1
    if (more) {
      tile_load(kb_next, kr, vr);
      kb_next = t + 2 < len ? it.at(keys, t + 2) : 0;
    }
    // V^T operands read now; the softmax covers their LDS latency
    bf16x8 vA[D / 8];
    pv_load(sV[cur], lane, vA);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pc[4];
    softmax_step(s0, s1, st, pc, a.sl2);
    pv_mma(vA, pc, st);
    if (more) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
    kb_cur = kb_after;
  }

  const float l_tot = partner_sum(st.l), lb_tot = partner_sum(st.lb);
  if (it.slot < 0) {
    if (!kRagged || qrow < a.n)
      write_o_bf16(st, l_tot, lb_tot, hl, a.o + bh_off + (size_t)qrow * D,
                   a.o_lo != nullptr ? a.o_lo + bh_off + (size_t)qrow * D : nullptr,
                   a.lse != nullptr ? a.lse + (size_t)it.bh * a.n + qrow : nullptr);
  } else {
    write_partial(st, l_tot, lb_tot, hl, 32 * wave + col,
                  a.part + (size_t)it.slot * kPartFloatsOf<D>);
  }
}

// Merge the segment partials of every split global query block, in segment
// order: M = max_s m_s, L = sum_s l_s 2^(m_s - M) (and Lb from the lb_s),
// O = sum_s O_s 2^(m_s - M) / Lb, lse = M + log2 L.  Thread t: query row t / 4,
// columns 16 (t % 4) + 64 u .. +15, u = 0 .. D/64 - 1.
template <int D>
__global__ __launch_bounds__(256) void bs_fwd_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ gblk, int heads, int n,
    int g, int nseg, uint16_t* __restrict__ o, uint16_t* __restrict__ o_lo,
    float* __restrict__ lse) {
  const int idx = blockIdx.x;           // (bh, gi)
  const int bh = idx / g, gi = idx - bh * g;
  const int row = threadIdx.x >> 2, dq = (threadIdx.x & 3) * 16;
  const int tok = gblk[gi] * kBlock + row;
  float M = 0.f, L = 0.f;
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    float acc[16], Lb;
    merge_partials<D>(part + (size_t)idx * nseg * kPartFloatsOf<D>, nseg, row, dq + 64 * u, acc,
                      M, L, Lb);
    if (tok >= n) return;   // past the end of a sequence that ends inside this block
    const size_t off = ((size_t)bh * n + tok) * D + dq + 64 * u;
    store16_bf16_lo(o + off, o_lo != nullptr ? o_lo + off : nullptr, acc, 1.f / Lb);
  }
  if (lse != nullptr && (threadIdx.x & 3) == 0)
    lse[(size_t)bh * n + tok] = (M + __log2f(L)) * kLn2;
  (void)heads;
}

// fp32 path: register-tiled FMA, one 256-thread work-group per query block walking
// its whole row or, when the whole problem has fewer rows than the device has
// work-group slots, per segment of `fseg` key blocks of a row, writing a partial
// record (unnormalised O, running max, running sum) that bs_fwd_f32_combine merges
// in segment order.  Thread t owns queries 4*(t/16)..+3 and, for the scores, keys
// 4*(t%16)..+3 of the current key block; for the output, head-dim columns
// 4*(t%16)..+3.  Each step reads float4 operands from LDS (64 FMAs per 8 reads);
// tile rows are padded to 68 floats, which keeps the float4 reads of 16 different
// rows on distinct banks.  The 16 threads of a query group are 16 consecutive
// lanes, so row reductions are xor-shuffles over 1, 2, 4, 8.
struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* row_info;   // [heads][nb - g][4] non-global row records
  const int32_t* gblk;
  float* part;       // partial records [rows][nseg][kPartFloats] of the split rows
  int heads, n, nb, g, total_items;
  int last_rows;   // tokens in the last block: n - 64 (nb - 1), 1..64
  int fseg, nseg;  // split rows: segments of fseg key blocks, at most nseg per row
  int gsplit;      // only the global rows are split: items_per_bh items per (batch,
  int items_per_bh;   // head), the non-global rows whole, then the global segments
  float scale;
};

constexpr int kF32Stride = kHead + 4;

// one 64x64 fp32 tile: 4 float4 per thread, row-major global -> padded LDS rows
struct TileF32 { f32x4 v[4]; };

// rows at or past `rows` (the end of a sequence inside the last block) are not
// read and stage as zeros
template <bool kRagged>
__device__ __forceinline__ void load_f32_tile(TileF32& t, const float* g, int tid, int rows) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (!kRagged || (4 * tid + 1024 * u) / kHead < rows)
      x = *reinterpret_cast<const f32x4*>(g + 4 * tid + 1024 * u);
    t.v[u] = x;
  }
}

__device__ __forceinline__ void store_f32_tile(float* s, const TileF32& t, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int x = 4 * tid + 1024 * u, row = x / kHead, col = x % kHead;
    *reinterpret_cast<f32x4*>(s + row * kF32Stride + col) = t.v[u];
  }
}

__device__ __forceinline__ float group16_max(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float group16_sum(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// kRagged as for the bf16 kernel: the sequence ends inside its last block.
template <bool kRagged>
__global__ __launch_bounds__(256) void bs_fwd_f32_kernel(FwdF32Args a) {
  __shared__ __attribute__((aligned(16))) float sQ[kBlock * kF32Stride];
  __shared__ __attribute__((aligned(16))) float sK[kBlock * kF32Stride];   // K, then P
  __shared__ __attribute__((aligned(16))) float sV[kBlock * kF32Stride];
  // this item's query block i, its key list [rp0, rp1) and, for a segment of a split
  // row, the index of its partial record (-1: the item holds its whole row)
  int bh, i, rp0, rp1, slot = -1;
  if (a.gsplit) {   // non-global rows whole, global rows in segments, long items first
    const int v = xcd_item_long_first(blockIdx.x, a.total_items, a.items_per_bh, a.nb - a.g);
    if (v < 0) return;
    bh = v / a.items_per_bh;
    const int r = v - bh * a.items_per_bh, h = bh % a.heads, ng = a.nb - a.g;
    if (r < ng) {
      const int32_t* rec = a.row_info + 4 * ((int64_t)h * ng + r);
      i = rec[0];
      rp0 = rec[1];
      rp1 = rp0 + rec[2];
    } else {
      const int gi = (r - ng) / a.nseg, s = (r - ng) - gi * a.nseg;
      i = a.gblk[gi];
      const int base = a.row_ptr[(int64_t)h * a.nb + i];   // a global row lists 0 .. nb-1
      rp0 = base + s * a.fseg;
      rp1 = base + min(a.nb, (s + 1) * a.fseg);
      slot = (bh * a.g + gi) * a.nseg + s;
    }
  } else {   // every row split into nseg segments (or whole when nseg = 1)
    const int v = xcd_remap(blockIdx.x, a.total_items);
    if (v >= a.total_items) return;
    const int row = v / a.nseg, seg = v - row * a.nseg;
    bh = row / a.nb;
    i = row - bh * a.nb;
    const int h = bh % a.heads;
    rp0 = a.row_ptr[(int64_t)h * a.nb + i];
    rp1 = a.row_ptr[(int64_t)h * a.nb + i + 1];
    if (a.nseg > 1) {   // this item's segment of the row
      rp0 += seg * a.fseg;
      if (rp0 >= rp1) return;
      rp1 = min(rp1, rp0 + a.fseg);
      slot = v;
    }
  }
  const int tid = threadIdx.x, tq = tid >> 4, tk = tid & 15;
  const size_t bh_off = (size_t)bh * a.n * kHead;
  auto rows_of = [&](int blk) { return blk == a.nb - 1 ? a.last_rows : kBlock; };
  {
    TileF32 qt;
    load_f32_tile<kRagged>(qt, a.q + bh_off + (size_t)i * kBlock * kHead, tid, rows_of(i));
    store_f32_tile(sQ, qt, tid);
  }

  float m[4], l[4], acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  }
  // K and V of the next key block are loaded into registers one block ahead
  TileF32 kt, vt;
  if (rp0 < rp1) {
    const int kb = a.col_idx[rp0];
    load_f32_tile<kRagged>(kt, a.k + bh_off + (size_t)kb * kBlock * kHead, tid, rows_of(kb));
    load_f32_tile<kRagged>(vt, a.v + bh_off + (size_t)kb * kBlock * kHead, tid, rows_of(kb));
  }
  int krows_next = rp0 < rp1 && kRagged ? rows_of(a.col_idx[rp0]) : kBlock;
  for (int e = rp0; e < rp1; ++e) {
    const int krows = krows_next;   // keys of this block that are tokens
    __syncthreads();   // the previous block's P (in sK) and V are no longer read
    store_f32_tile(sK, kt, tid);
    store_f32_tile(sV, vt, tid);
    if (e + 1 < rp1) {
      const int kb = a.col_idx[e + 1];
      load_f32_tile<kRagged>(kt, a.k + bh_off + (size_t)kb * kBlock * kHead, tid, rows_of(kb));
      load_f32_tile<kRagged>(vt, a.v + bh_off + (size_t)kb * kBlock * kHead, tid, rows_of(kb));
      if (kRagged) krows_next = rows_of(kb);
    }
    __syncthreads();
    // S = Q K^T for queries 4tq+r, keys 4tk+j
    float s[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[r][j] = 0.f;
    // fully unrolled, the loads run far enough ahead that the instance with
    // sequence-end guards no longer fits its registers (it spilled): that one is
    // unrolled four steps at a time
    constexpr int kUnroll = kRagged ? 4 : 16;
#pragma unroll kUnroll
    for (int c = 0; c < kHead; c += 4) {
      f32x4 qv[4], kv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[r] = *reinterpret_cast<const f32x4*>(sQ + (4 * tq + r) * kF32Stride + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[j] = *reinterpret_cast<const f32x4*>(sK + (4 * tk + j) * kF32Stride + c);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int x = 0; x < 4; ++x) s[r][j] = __builtin_fmaf(qv[r][x], kv[j][x], s[r][j]);
    }
    // online softmax per query row (its 64 keys live in the 16 threads of the group)
    float p[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[r][j] = !kRagged || 4 * tk + j < krows ? s[r][j] * a.scale : -INFINITY;
        mx = fmaxf(mx, s[r][j]);
      }
      const float m_new = fmaxf(m[r], group16_max(mx));
      const float alpha = expf(m[r] - m_new);
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[r][j] = expf(s[r][j] - m_new);
        rs += p[r][j];
      }
      l[r] = l[r] * alpha + group16_sum(rs);
      m[r] = m_new;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] *= alpha;
    }
    __syncthreads();   // every thread is done reading K
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 w = {p[r][0], p[r][1], p[r][2], p[r][3]};
      *reinterpret_cast<f32x4*>(sK + (4 * tq + r) * kF32Stride + 4 * tk) = w;
    }
    __syncthreads();
    // O += P V for queries 4tq+r, head-dim columns 4tk..4tk+3
#pragma unroll kUnroll
    for (int k0 = 0; k0 < kBlock; k0 += 4) {
      f32x4 pv[4], vv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = *reinterpret_cast<const f32x4*>(sK + (4 * tq + r) * kF32Stride + k0);
#pragma unroll
      for (int x = 0; x < 4; ++x) vv[x] = *reinterpret_cast<const f32x4*>(sV + (k0 + x) * kF32Stride + 4 * tk);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(pv[r][x], vv[x][c], acc[r][c]);
    }
  }
  if (slot >= 0) {   // partial record: O unnormalised, then m, then l (natural log units)
    float* rec = a.part + (size_t)slot * kPartFloats;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 w = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
      *reinterpret_cast<f32x4*>(rec + (4 * tq + r) * kHead + 4 * tk) = w;
      if (tk == 0) {
        rec[kBlock * kHead + 4 * tq + r] = m[r];
        rec[kBlock * kHead + kBlock + 4 * tq + r] = l[r];
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = i * kBlock + 4 * tq + r;
    if (kRagged && tok >= a.n) break;
    const float inv = 1.f / l[r];
    const f32x4 w = {acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv};
    *reinterpret_cast<f32x4*>(a.o + bh_off + (size_t)tok * kHead + 4 * tk) = w;
    if (a.lse != nullptr && tk == 0) a.lse[(size_t)bh * a.n + tok] = m[r] + logf(l[r]);
  }
}

// Merge the segment records of every split fp32 row, in segment order:
// M = max_s m_s, L = sum_s l_s e^(m_s - M), O = sum_s O_s e^(m_s - M) / L, lse = M + ln L.
// One work-group per split row: work-group (bh, i) when every row is split, (bh, gi)
// for global block gblk[gi] when only the global rows are (gblk not null); thread t:
// query row t / 4, 16 columns.
__global__ __launch_bounds__(256) void bs_fwd_f32_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ gblk, int heads, int n, int nb, int g, int fseg, int nseg,
    float* __restrict__ o, float* __restrict__ lse) {
  const int row = blockIdx.x;   // (bh, i) or (bh, gi)
  const int per = gblk != nullptr ? g : nb;
  const int bh = row / per, h = bh % heads;
  const int i = gblk != nullptr ? gblk[row - bh * per] : row - bh * per;
  const int qr = threadIdx.x >> 2, dq = (threadIdx.x & 3) * 16;
  const int tok = i * kBlock + qr;
  if (tok >= n) return;   // past the end of a sequence that ends inside this block
  const int len = row_ptr[(int64_t)h * nb + i + 1] - row_ptr[(int64_t)h * nb + i];
  const int ns = (len + fseg - 1) / fseg;
  const float* base = part + (size_t)row * nseg * kPartFloats;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, base[(size_t)s * kPartFloats + kBlock * kHead + qr]);
  float L = 0.f, acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* ps = base + (size_t)s * kPartFloats;
    const float f = expf(ps[kBlock * kHead + qr] - M);
    L += ps[kBlock * kHead + kBlock + qr] * f;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ps + qr * kHead + dq + e);
      acc[e] += x[0] * f;
      acc[e + 1] += x[1] * f;
      acc[e + 2] += x[2] * f;
      acc[e + 3] += x[3] * f;
    }
  }
  const float inv = 1.f / L;
  float* op = o + ((size_t)bh * n + tok) * kHead + dq;
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const f32x4 w = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
    *reinterpret_cast<f32x4*>(op + e) = w;
  }
  if (lse != nullptr && (threadIdx.x & 3) == 0) lse[(size_t)bh * n + tok] = M + logf(L);
}

// fp32 row split.  When the rows alone would leave most work-group slots (four per
// compute unit) idle, every row is cut into segments of fseg key blocks (at most
// kF32MaxItems items).  Otherwise the global rows, which list every block, are cut
// into the segments of the bf16 path (seg_plan) and the other rows run whole.
struct F32Plan { int fseg, nseg, gsplit; };
constexpr int kF32MaxItems = 2048;

F32Plan f32_plan(const bsattn_layout* L, int batch) {
  const int64_t rows = (int64_t)batch * L->heads * L->nb;
  const int64_t slots = 4 * (int64_t)(L->cus > 0 ? L->cus : 1);
  F32Plan p{L->nb, 1, 0};
  if (2 * rows >= slots) {
    const SegPlan sp = seg_plan(L, batch);
    if (L->g > 0 && sp.split) p = F32Plan{sp.seg, sp.nseg, 1};
    return p;
  }
  const int64_t pairs = (int64_t)batch * L->heads * L->nnz_per_head;
  int fseg = (int)std::max<int64_t>(1, (pairs + slots - 1) / slots);
  int nseg = (L->nb + fseg - 1) / fseg;
  while (rows * nseg > kF32MaxItems) {
    fseg *= 2;
    nseg = (L->nb + fseg - 1) / fseg;
  }
  if (nseg > 1) p = F32Plan{fseg, nseg, 0};
  return p;
}

}  // namespace

// Workspace of one dtype's forward: bf16 global-row segments or fp32 row segments.
size_t fwd_workspace_bytes_dt(const bsattn_layout* L, int batch, bsattn_dtype dt, int d) {
  if (dt == BSATTN_F32) {
    const F32Plan fp = f32_plan(L, batch);
    const size_t rows = (size_t)batch * L->heads * (fp.gsplit ? L->g : L->nb);
    return fp.nseg > 1 ? rows * fp.nseg * kPartFloats * sizeof(float) : 0;
  }
  const SegPlan sp = seg_plan(L, batch);
  const size_t part = d == 128 ? kPartFloatsOf<128> : kPartFloats;
  const Fold f = fold_plan(sp.nseg);
  return sp.split ? (size_t)batch * L->heads * L->g * (sp.nseg + (f.chunk ? f.nfold : 0)) * part *
                        sizeof(float)
                  : 0;
}

// The size the public query reports: enough for either dtype that the head
// dimension is built for (fp32 has d = 64 only).
size_t fwd_workspace_bytes(const bsattn_layout* L, int batch, int d) {
  const size_t bf = fwd_workspace_bytes_dt(L, batch, BSATTN_BF16, d);
  return d == kHead ? std::max(bf, fwd_workspace_bytes_dt(L, batch, BSATTN_F32, d)) : bf;
}

template <int D>
int launch_fwd_bf16(const bsattn_layout* L, int batch, float scale, const void* q,
                    const void* k, const void* v, void* o, float* lse, void* o_lo, void* ws,
                    hipStream_t stream);

int launch_fwd(const bsattn_layout* L, int batch, bsattn_dtype dt, int d, float scale,
               const void* q, const void* k, const void* v, void* o, float* lse, void* o_lo,
               void* ws, hipStream_t stream) {
  const int bhn = batch * L->heads;
  if (dt == BSATTN_F32) {
    FwdF32Args a;
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
    a.o = (float*)o; a.lse = lse;
    a.row_ptr = L->d_row_ptr; a.col_idx = L->d_col_idx;
    a.row_info = L->d_row_info; a.gblk = L->d_gblk;
    a.heads = L->heads; a.n = L->n; a.nb = L->nb; a.g = L->g;
    const F32Plan fp = f32_plan(L, batch);
    a.fseg = fp.fseg; a.nseg = fp.nseg; a.gsplit = fp.gsplit;
    a.part = (float*)ws;
    a.items_per_bh = fp.gsplit ? (L->nb - L->g) + L->g * fp.nseg : L->nb * fp.nseg;
    a.total_items = bhn * a.items_per_bh;
    a.last_rows = L->n - kBlock * (L->nb - 1);
    a.scale = scale;
    const int grid = 8 * ((a.total_items + 7) / 8);
    {
      ProfScope prof_("bs_fwd_f32", stream);
      if (a.last_rows < kBlock)
        hipLaunchKernelGGL(bs_fwd_f32_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(bs_fwd_f32_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
    }
    int st = check_hip(hipGetLastError(), "bs_fwd_f32 launch");
    if (st || fp.nseg == 1) return st;
    {
      ProfScope prof_("bs_fwd_f32_combine", stream);
      hipLaunchKernelGGL(bs_fwd_f32_combine_kernel, dim3(bhn * (fp.gsplit ? L->g : L->nb)),
                         dim3(256), 0, stream, (const float*)ws, L->d_row_ptr,
                         fp.gsplit ? (const int32_t*)L->d_gblk : nullptr, L->heads, L->n, L->nb,
                         L->g, fp.fseg, fp.nseg, (float*)o, lse);
    }
    return check_hip(hipGetLastError(), "bs_fwd_f32_combine launch");
  }
  if (d == 128) return launch_fwd_bf16<128>(L, batch, scale, q, k, v, o, lse, o_lo, ws, stream);
  return launch_fwd_bf16<kHead>(L, batch, scale, q, k, v, o, lse, o_lo, ws, stream);
}

template <int D>
int launch_fwd_bf16(const bsattn_layout* L, int batch, float scale, const void* q,
                    const void* k, const void* v, void* o, float* lse, void* o_lo, void* ws,
                    hipStream_t stream) {
  const int bhn = batch * L->heads;
  FwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o; a.o_lo = (uint16_t*)o_lo; a.lse = lse; a.part = (float*)ws;
  a.col_idx = L->d_col_idx; a.row_info = L->d_row_info;
  a.gblk = L->d_gblk;
  a.heads = L->heads; a.n = L->n; a.nb = L->nb; a.g = L->g;
  a.last_rows = L->n - kBlock * (L->nb - 1);
  const SegPlan sp = seg_plan(L, batch);
  a.seg = sp.seg; a.nseg = sp.nseg; a.split = sp.split;
  a.items_per_bh = (L->nb - L->g) + L->g * sp.nseg;
  a.total_items = bhn * a.items_per_bh;
  a.sl2 = scale * kLog2e;
  const int grid = 8 * ((a.total_items + 7) / 8);
  {
    ProfScope prof_(D == kHead ? "bs_fwd_bf16" : "bs_fwd_bf16_d128", stream);
    if (a.last_rows < kBlock)
      hipLaunchKernelGGL((bs_fwd_bf16_kernel<D, true>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((bs_fwd_bf16_kernel<D, false>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
  }
  int st = check_hip(hipGetLastError(), "bs_fwd_bf16 launch");
  if (st || !sp.split || L->g == 0) return st;
  const Fold f = fold_plan(sp.nseg);
  const float* merged = (const float*)ws;   // what the combine merges: the partials or folds
  if (f.chunk) {
    float* dst = (float*)ws + (size_t)bhn * L->g * sp.nseg * kPartFloatsOf<D>;
    {
      ProfScope prof_("bs_fwd_fold", stream);
      hipLaunchKernelGGL(fold_softmax_kernel<D>, dim3(bhn * L->g * f.nfold * (D / 16)), dim3(256),
                         0, stream, (const float*)ws, dst, sp.nseg, f.chunk, f.nfold);
    }
    if ((st = check_hip(hipGetLastError(), "bs_fwd_fold launch"))) return st;
    merged = dst;
  }
  {
    ProfScope prof_("bs_fwd_combine", stream);
    hipLaunchKernelGGL(bs_fwd_combine_kernel<D>, dim3(bhn * L->g), dim3(256), 0, stream, merged,
                       L->d_gblk, L->heads, L->n, L->g, f.nfold, (uint16_t*)o, (uint16_t*)o_lo,
                       lse);
  }
  return check_hip(hipGetLastError(), "bs_fwd_combine launch");
}

}  // namespace bsattn
