// BigBird-ITC block-sparse attention backward on gfx950.
//
// The pages give no backward pass; this is the exact gradient of the forward in
// bs_fwd.hip ("Big Bird: Transformers for Longer Sequences", §2 eq. (AT); App. D
// Fig. 6), recomputing P = exp(scale * Q K^T - lse) from the saved log-sum-exp:
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Head dimension d = 64 or 128: one template per kernel, instantiated for both.
//
// No atomics: every output tile has one owner.
//   bs_bwd_dq    one work-group per query block (row of the layout): dQ, and D
//                for the next kernel (rowsum(dO * O), corrected by the row sum of
//                dS where the item holds the whole row: then it is sum P * dP
//                with the probabilities this backward recomputes).
//   bs_bwd_dkdv  one work-group per key block (column of the transposed layout):
//                dK and dV, walking the query blocks that see that key block.
//   bs_bwd_reduce  global rows / columns are full-length; they are split into
//                segments (length set per call from the total work) writing fp32
//                partials, summed here in segment order, so results are bitwise
//                reproducible.  Each XCD starts its segments before other items.

#include <mutex>
#include <string>

#include "bs_bwd.hpp"
#include "fold.hpp"

namespace bsattn {

// Device scratch of bsattn_bwd_noalloc (D and the fp32 partials of split global
// rows and columns), for callers that cannot allocate.  Each device holds its own
// copy for the life of the process.  In host code this name is only a stand-in for
// the device symbol: its device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = BSATTN_BWD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

using namespace bwd;

constexpr int kThreads = 128;

template <int D, bool kRagged>
__global__ __launch_bounds__(kThreads) void bs_bwd_dq_kernel(BwdArgs a) {
  constexpr int kS = kStrideOf<D>, kC = D / 16, kT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBlock * kS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBlock * kS];

  const int v = xcd_item_long_first(blockIdx.x, a.total_items, a.items_per_bh, a.nb - a.g);
  if (v < 0) return;
  const Item it = decode(a, v, false);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)it.bh * a.n * D;
  const int qrow = it.blk * kBlock + 32 * wave + col;

  const int32_t* keys = a.col_idx + it.start;
  const uint16_t* kbase = a.k + bh_off;
  const uint16_t* vbase = a.v + bh_off;
  // Keys past the end of a sequence that ends inside its last block stage as zero
  // rows of K and V, which give them dP = 0 and no dQ contribution; query rows past
  // the end read nothing and write nothing.
  TileRegsT<D> kr, vr;
  if (it.len > 0) {
    load_block<kRagged>(kr, kbase, it.first, a, tid);
    load_block<kRagged>(vr, vbase, it.first, a, tid);
  }
  // block index of the next tile, read one iteration ahead of its use
  int kb_next = it.len > 1 ? it.at(keys, 1) : 0;
  const bool qvalid = !kRagged || qrow < a.n;
  bf16x8 qB[kC], doB[kC];
  float dsum = 0.f;
  {
    const size_t off = bh_off + (size_t)qrow * D + 8 * hl;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const u32x4 qv = qvalid ? ldg16(a.q + off + 16 * c) : z;
      const u32x4 dv = qvalid ? ldg16(a.dout + off + 16 * c) : z;
      const u32x4 ov = qvalid ? ldg16(a.o + off + 16 * c) : z;
      qB[c] = __builtin_bit_cast(bf16x8, qv);
      doB[c] = __builtin_bit_cast(bf16x8, dv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(ov[e]), dsum);
        dsum = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(ov[e]), dsum);
      }
      if (a.o_lo != nullptr) {   // O + its rounding residual: D to ~2^-17 relative
        const u32x4 rv = qvalid ? ldg16(a.o_lo + off + 16 * c) : z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dsum = __builtin_fmaf(bf16_lo(dv[e]), bf16_lo(rv[e]), dsum);
          dsum = __builtin_fmaf(bf16_hi(dv[e]), bf16_hi(rv[e]), dsum);
        }
      }
    }
  }
  const float Dq = partner_sum(dsum);   // D = rowsum(dO * O)
  // A segment of a split row writes this D for the dK/dV kernel.  An item holding a
  // whole row writes it after the loop, corrected by the row sum of dS: that sum is
  // sum P dP - D sum P, with the probabilities P the backward itself recomputes, so
  // D + sum dS is sum P dP free of the bf16 rounding of the weights behind O.
  if (it.slot >= 0 && it.seg == 0 && hl == 0 && qvalid) a.dbuf[(size_t)it.bh * a.n + qrow] = Dq;
  // accumulators seeded so that the MFMAs return S - lse/scale (raw score units,
  // the scale applied in fp32 below: P = 2^((S - lse/scale) * scale*log2(e))) and
  // dP - D
  const float lraw = qvalid ? a.lse[(size_t)it.bh * a.n + qrow] * a.inv_scale : 0.f;
  f32x16 seed_s, seed_d;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    seed_s[r] = -lraw;
    seed_d[r] = -Dq;
  }
  lds_store_nat(sK[0], kr, tid);
  lds_store_nat(sV[0], vr, tid);

  f32x16 g[kT];   // dQ^T: g[t] holds d rows 32t..32t+31
#pragma unroll
  for (int t = 0; t < kT; ++t) g[t] = zero16();
  float ds_sum = 0.f;   // this half-lane's share of the row sum of dS
  int kb_cur = it.len > 0 ? it.first : 0;
  for (int t = 0; t < it.len; ++t) {
    const int cur = t & 1;
    __syncthreads();
    const bool more = t + 1 < it.len;
    if (more) {
      load_block<kRagged>(kr, kbase, kb_next, a, tid);
      load_block<kRagged>(vr, vbase, kb_next, a, tid);
    }
    const int kb_after = kb_next;   // block of tile t + 1
    if (more) kb_next = t + 2 < it.len ? it.at(keys, t + 2) : 0;
    // S^T = K Q^T and dP^T = V dO^T  (rows = keys, columns = this lane's query)
    f32x16 s0 = seed_s, s1 = seed_s, p0 = seed_d, p1 = seed_d;
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
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = fast_exp2(s0[r] * a.sl2) * p0[r];      // dS = P * (dP - D)
      s1[r] = fast_exp2(s1[r] * a.sl2) * p1[r];
    }
    // keys past the end of a sequence that ends inside this block are zero rows of
    // K and V: their dS multiplies a zero K row in dQ, but is not part of the row sum
    if (kRagged && kb_cur == a.nb - 1) zero_keys_from(s0, s1, hl, a.last_rows);
    {
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
    if (more) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
    kb_cur = kb_after;
  }

  const float sc = a.scale;
  if (it.slot < 0) {
    const float dfix = Dq + partner_sum(ds_sum);
    if (!qvalid) return;
    if (hl == 0) a.dbuf[(size_t)it.bh * a.n + qrow] = dfix;
    uint16_t* op = a.dq + bh_off + (size_t)qrow * D + 4 * hl;
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
  } else {
    float* pp = a.part_q + (size_t)it.slot * kTileOf<D> + (32 * wave + col) * D + 4 * hl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 w[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) w[t][e] = g[t][4 * j + e] * sc;
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pp + 32 * t + 8 * j) = w[t];
    }
  }
}

template <int D, bool kRagged>
__global__ __launch_bounds__(kThreads) void bs_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kS = kStrideOf<D>, kC = D / 16, kT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][kBlock * kS];
  __shared__ __attribute__((aligned(16))) uint16_t sO[2][kBlock * kS];   // dO
  __shared__ __attribute__((aligned(16))) float sL[2][kBlock];   // -lse / scale
  __shared__ __attribute__((aligned(16))) float sD[2][kBlock];   // -D

  const int v = xcd_item_long_first(blockIdx.x, a.total_items, a.items_per_bh, a.nb - a.g);
  if (v < 0) return;
  const Item it = decode(a, v, true);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)it.bh * a.n * D;
  const int krow = it.blk * kBlock + 32 * wave + col;   // this lane's key token

  const int32_t* qblks = a.csc_idx + it.start;
  const uint16_t* qbase = a.q + bh_off;
  const uint16_t* dobase = a.dout + bh_off;
  const float* lbase = a.lse + (size_t)it.bh * a.n;
  const float* dbase = a.dbuf + (size_t)it.bh * a.n;
  // Query rows past the end of a sequence that ends inside its last block stage as
  // zero rows of Q and dO with lse = +inf and D = 0, so that P = 0 and dS = 0 there;
  // key rows past the end read nothing and write nothing.
  TileRegsT<D> qr, dr;
  float lv = 0.f, dval = 0.f;
  auto load_rowvals = [&](int qb) {
    if (tid < kBlock) {
      const bool ok = !kRagged || qb * kBlock + tid < a.n;
      lv = ok ? lbase[qb * kBlock + tid] : INFINITY;
      dval = ok ? dbase[qb * kBlock + tid] : 0.f;
    }
  };
  if (it.len > 0) {
    load_block<kRagged>(qr, qbase, it.first, a, tid);
    load_block<kRagged>(dr, dobase, it.first, a, tid);
    load_rowvals(it.first);
  }
  // block index of the next tile, read one iteration ahead of its use
  int qb_next = it.len > 1 ? it.at(qblks, 1) : 0;
  const bool kvalid = !kRagged || krow < a.n;
  bf16x8 kB[kC], vB[kC];
  {
    const size_t off = bh_off + (size_t)krow * D + 8 * hl;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      kB[c] = kvalid ? ld16(a.k + off + 16 * c) : bf16x8{};
      vB[c] = kvalid ? ld16(a.v + off + 16 * c) : bf16x8{};
    }
  }
  // sL and sD hold -lse/scale and -D to seed S (raw score units; the scale is
  // applied in fp32 before the exponential) and dP
  lds_store_nat(sQ[0], qr, tid);
  lds_store_nat(sO[0], dr, tid);
  if (tid < kBlock) { sL[0][tid] = -lv * a.inv_scale; sD[0][tid] = -dval; }
  // vB is first read inside the loop: drain the prologue's loads here, or the
  // loop's first use of vB waits on every iteration's tile prefetch as well
  wait_all_loads();

  f32x16 dv[kT], dk[kT];   // dV^T, dK^T: tile t holds d rows 32t..32t+31
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    dv[t] = zero16();
    dk[t] = zero16();
  }
  for (int t = 0; t < it.len; ++t) {
    const int cur = t & 1;
    __syncthreads();
    const bool more = t + 1 < it.len;
    if (more) {
      load_block<kRagged>(qr, qbase, qb_next, a, tid);
      load_block<kRagged>(dr, dobase, qb_next, a, tid);
      load_rowvals(qb_next);
      qb_next = t + 2 < it.len ? it.at(qblks, t + 2) : 0;
    }
    // S[q][key] = Q K^T, dP[q][key] = dO V^T; rows = queries (2 tiles), column = key.
    // Row q of register r is 32*qt + 8*(r/4) + 4*hl + r%4: the seeds are the
    // matching -lse*log2(e) and -D values.
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
    if (more) {
      lds_store_nat(sQ[cur ^ 1], qr, tid);
      lds_store_nat(sO[cur ^ 1], dr, tid);
      if (tid < kBlock) { sL[cur ^ 1][tid] = -lv * a.inv_scale; sD[cur ^ 1][tid] = -dval; }
    }
  }

  const float sc = a.scale;
  if (it.slot < 0) {
    if (!kvalid) return;
    const size_t off = bh_off + (size_t)krow * D + 4 * hl;
    uint16_t* kp = a.dk + off;
    uint16_t* vp = a.dv + off;
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
    float* pk = a.part_kv + (size_t)it.slot * 2 * kTileOf<D> + (32 * wave + col) * D + 4 * hl;
    float* pv = pk + kTileOf<D>;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 kw[kT], vw[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kw[t][e] = dk[t][4 * j + e] * sc;
          vw[t][e] = dv[t][4 * j + e];
        }
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pk + 32 * t + 8 * j) = kw[t];
#pragma unroll
      for (int t = 0; t < kT; ++t) *reinterpret_cast<f32x4*>(pv + 32 * t + 8 * j) = vw[t];
    }
  }
}

// Sum the fp32 partial tiles of split global rows (dQ) and columns (dK, dV) in
// segment order.  Work-group (bh*g + gi)*3 + kind, kind 0 = dQ, 1 = dK, 2 = dV;
// thread t sums floats 16 (t + 256 u) .. +15 of the 64 x D tile, u < D/64.
template <int D>
__global__ __launch_bounds__(256) void bs_bwd_reduce_kernel(
    const float* __restrict__ part_q, const float* __restrict__ part_kv,
    const int32_t* __restrict__ gblk, int n, int g, int nseg, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  const int kind = blockIdx.x % 3;
  const int idx = blockIdx.x / 3;   // bh*g + gi
  const int bh = idx / g, gi = idx - bh * g;
  constexpr int kTile = kTileOf<D>;
  const size_t slot0 = (size_t)idx * nseg;
#pragma unroll
  for (int u = 0; u < D / 64; ++u) {
    const int e0 = (threadIdx.x + 256 * u) * 16;  // 16 consecutive floats of the tile
    float acc[16];
    if (kind == 0) sum_partials(part_q + slot0 * kTile + e0, kTile, nseg, acc);
    else sum_partials(part_kv + slot0 * 2 * kTile + (kind - 1) * kTile + e0, 2 * kTile, nseg, acc);
    // rows past the end of a sequence that ends inside this block are not written
    if (gblk[gi] * kBlock + e0 / D >= n) return;
    uint16_t* dst = kind == 0 ? dq : (kind == 1 ? dk : dv);
    dst += ((size_t)bh * n + (size_t)gblk[gi] * kBlock) * D + e0;
#pragma unroll
    for (int e = 0; e < 16; e += 8) {
      u32x4 w;
      w[0] = pack_bf16x2(acc[e], acc[e + 1]);
      w[1] = pack_bf16x2(acc[e + 2], acc[e + 3]);
      w[2] = pack_bf16x2(acc[e + 4], acc[e + 5]);
      w[3] = pack_bf16x2(acc[e + 6], acc[e + 7]);
      *reinterpret_cast<u32x4*>(dst + e) = w;
    }
  }
}

}  // namespace

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
int noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(BSATTN_EUNSUPPORTED, "bwd_noalloc: device index above 63");
  std::lock_guard<std::mutex> lk(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return check_hip(e, "hipGetSymbolAddress(scratch)");
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return BSATTN_OK;
}

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

size_t bwd_workspace_bytes(const bsattn_layout* L, int batch, int d) {
  size_t bytes = (size_t)batch * L->heads * L->n * sizeof(float);   // D
  bytes = (bytes + 255) & ~(size_t)255;
  const SegPlan sp = seg_plan(L, batch);
  const Fold f = fold_plan(sp.nseg);
  if (sp.split)   // dQ, dK, dV partials, then their folds
    bytes += (size_t)batch * L->heads * L->g * (sp.nseg + (f.chunk ? f.nfold : 0)) * 3 *
             (kBlock * d) * sizeof(float);
  return bytes;
}

namespace {

template <int D>
int launch_bwd_d(const bsattn_layout* L, int batch, float scale, const void* q, const void* k,
                 const void* v, const void* o, const void* o_lo, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* ws, hipStream_t stream) {
  constexpr int kTile = kTileOf<D>;
  BwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o; a.o_lo = (const uint16_t*)o_lo; a.lse = lse;
  a.dout = (const uint16_t*)dout;
  a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
  char* w = (char*)ws;
  a.dbuf = (float*)w;
  size_t off = ((size_t)batch * L->heads * L->n * sizeof(float) + 255) & ~(size_t)255;
  const SegPlan sp = seg_plan(L, batch);
  const size_t nslots = (size_t)batch * L->heads * L->g * sp.nseg;
  a.part_q = sp.split ? (float*)(w + off) : nullptr;
  a.part_kv = sp.split ? (float*)(w + off + nslots * kTile * sizeof(float)) : nullptr;
  a.col_idx = L->d_col_idx; a.csc_idx = L->d_csc_idx;
  a.gblk = L->d_gblk;
  a.row_info = L->d_row_info; a.col_info = L->d_col_info;
  a.heads = L->heads; a.n = L->n; a.nb = L->nb; a.g = L->g;
  a.last_rows = L->n - kBlock * (L->nb - 1);
  a.seg = sp.seg; a.nseg = sp.nseg; a.split = sp.split;
  a.items_per_bh = (L->nb - L->g) + L->g * sp.nseg;
  a.total_items = batch * L->heads * a.items_per_bh;
  a.scale = scale;
  a.sl2 = scale * kLog2e;
  a.inv_scale = 1.f / scale;
  const int grid = 8 * ((a.total_items + 7) / 8);
  {
    ProfScope prof_(D == kHead ? "bs_bwd_dq" : "bs_bwd_dq_d128", stream);
    if (a.last_rows < kBlock)
      hipLaunchKernelGGL((bs_bwd_dq_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((bs_bwd_dq_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  int st = check_hip(hipGetLastError(), "bs_bwd_dq launch");
  if (st) return st;
  {
    ProfScope prof_(D == kHead ? "bs_bwd_dkdv" : "bs_bwd_dkdv_d128", stream);
    if (a.last_rows < kBlock)
      hipLaunchKernelGGL((bs_bwd_dkdv_kernel<D, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((bs_bwd_dkdv_kernel<D, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  }
  st = check_hip(hipGetLastError(), "bs_bwd_dkdv launch");
  if (st || !sp.split || L->g == 0) return st;
  const Fold f = fold_plan(sp.nseg);
  const float* red_q = a.part_q;    // what the reduce sums: the partials or their folds
  const float* red_kv = a.part_kv;
  if (f.chunk) {
    const int groups = batch * L->heads * L->g;
    float* fq = a.part_kv + nslots * 2 * kTile;
    float* fkv = fq + (size_t)groups * f.nfold * kTile;
    const FoldSumJob jq = fold_sum_job(a.part_q, fq, groups, sp.nseg, f, kTile);
    const FoldSumJob jkv = fold_sum_job(a.part_kv, fkv, groups, sp.nseg, f, 2 * kTile);
    {
      ProfScope prof_("bs_bwd_fold", stream);
      hipLaunchKernelGGL(fold_sum_kernel, dim3(jq.blocks + jkv.blocks), dim3(256), 0, stream, jq,
                         jkv);
    }
    if ((st = check_hip(hipGetLastError(), "bs_bwd_fold launch"))) return st;
    red_q = fq;
    red_kv = fkv;
  }
  {
    ProfScope prof_("bs_bwd_reduce", stream);
    hipLaunchKernelGGL(bs_bwd_reduce_kernel<D>, dim3(batch * L->heads * L->g * 3), dim3(256), 0,
                       stream, red_q, red_kv, L->d_gblk, L->n, L->g, f.nfold, a.dq, a.dk, a.dv);
  }
  return check_hip(hipGetLastError(), "bs_bwd_reduce launch");
}

}  // namespace

int launch_bwd(const bsattn_layout* L, int batch, int d, float scale, const void* q,
               const void* k, const void* v, const void* o, const void* o_lo, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, void* ws, hipStream_t stream) {
  if (d == 128)
    return launch_bwd_d<128>(L, batch, scale, q, k, v, o, o_lo, lse, dout, dq, dk, dv, ws, stream);
  return launch_bwd_d<kHead>(L, batch, scale, q, k, v, o, o_lo, lse, dout, dq, dk, dv, ws, stream);
}

}  // namespace bsattn
