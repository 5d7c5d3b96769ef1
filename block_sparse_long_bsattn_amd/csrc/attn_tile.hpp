// One step of the streaming attention forward for a 64-row query tile held by two
// waves (wave w owns query rows 32w..32w+31, one query per lane column):
//   S^T = K Q^T over a 64-key tile, online softmax in fp32, O^T += V^T P^T.
// Shared by the block-sparse and the banded forward kernels.  The head dimension D
// (64, or 128 for the block-sparse instances that take it) sets the number of
// 16-wide contraction chunks of S^T and of 32-row O^T tiles.
#pragma once

#include "common.hpp"

namespace bsattn {

template <int D>
struct FwdStateT {
  f32x16 o[D / 32];   // O^T accumulators: o[t] holds d rows 32t..32t+31, column = query
  float m;         // reference max (log2 units), -inf until the row saw a finite score
  float l;         // this half-lane's share of the row sum (fp32 probabilities)
  float lb;        // ... of the bf16-rounded probabilities that the PV product uses
};
using FwdState = FwdStateT<kHead>;

template <int D>
__device__ __forceinline__ void fwd_state_init(FwdStateT<D>& st) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t) st.o[t] = zero16();
  st.m = -INFINITY;
  st.l = 0.f;
  st.lb = 0.f;
}

// S^T for the 64 keys of the LDS tile sK (natural layout) against this lane's query:
// the plain products of the bf16 operands, accumulated in fp32 (the scale is applied
// afterwards, in fp32).  s0 holds keys 0..31, s1 keys 32..63; register r <-> key
// 8*(r/4) + 4*hl + r%4.  qB holds this lane's query as NQ = D/16 operands.
template <int NQ>
__device__ __forceinline__ void qk_tile(const uint16_t* sK, const bf16x8 (&qB)[NQ], int col,
                                        int hl, f32x16& s0, f32x16& s1) {
  constexpr int kS = kStrideOf<16 * NQ>;
  bf16x8 a[2 * NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    a[2 * c] = ld16(sK + col * kS + 16 * c + 8 * hl);
    a[2 * c + 1] = ld16(sK + (32 + col) * kS + 16 * c + 8 * hl);
  }
  const f32x16 z = zero16();
  s0 = mfma32(a[0], qB[0], z);
  s1 = mfma32(a[1], qB[0], z);
#pragma unroll
  for (int c = 1; c < NQ; ++c) {
    s0 = mfma32(a[2 * c], qB[c], s0);
    s1 = mfma32(a[2 * c + 1], qB[c], s1);
  }
}

// Keys kmin.. of an S^T tile (s0: keys 0..31, s1: keys 32..63, register r <-> key
// 8*(r/4) + 4*hl + r%4) set to -inf: the positions past the end of a sequence
// that ends inside the tile's block.
__device__ __forceinline__ void mask_keys_from(f32x16& s0, f32x16& s1, int hl, int kmin) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int x = 8 * (r >> 2) + 4 * hl + (r & 3);
    if (x >= kmin) s0[r] = -INFINITY;
    if (32 + x >= kmin) s1[r] = -INFINITY;
  }
}

// The same keys set to zero instead (dS of keys that are not tokens).
__device__ __forceinline__ void zero_keys_from(f32x16& s0, f32x16& s1, int hl, int kmin) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int x = 8 * (r >> 2) + 4 * hl + (r & 3);
    if (x >= kmin) s0[r] = 0.f;
    if (32 + x >= kmin) s1[r] = 0.f;
  }
}

// Online softmax over one key tile of raw scores S = Q.K (fp32; -inf marks an
// excluded key).  Probabilities are 2^(S*sl2 - m) with sl2 = scale*log2(e) applied
// in fp32 and m a reference maximum in log2 units.  The reference only moves when
// a block's maximum exceeds it by more than kRescaleSlack, so the unnormalised
// probabilities stay below 2^kRescaleSlack and most blocks need no rescale of O
// and l; the result is exact either way since numerator and denominator share the
// reference.  On return pc[c] holds the bf16 probabilities of key chunk c as MFMA
// operands; st.l has grown by their fp32 sum and st.lb by the sum of the bf16
// values themselves.  O is normalised by lb, which makes it an exact weighted
// average of V (weights summing to 1) whatever the rounding of each P -- this
// matters when one key dominates a row, since that key's P (up to
// 2^kRescaleSlack, not 1) is rounded by up to 2^-8 relative, and the backward's
// D = rowsum(dO * O) inherits any inconsistency of O.  lse comes from l: the
// backward recomputes every P from it, and a sum over many rows of P (the
// gradient of a key that every row sees) would accumulate its rounding.
constexpr float kRescaleSlack = 8.f;

template <int D>
__device__ __forceinline__ void softmax_step(f32x16& s0, f32x16& s1, FwdStateT<D>& st,
                                             bf16x8 (&pc)[4], float sl2) {
  float mx = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[r]), s1[r]);
  mx = partner_max(mx) * sl2;   // block maximum, log2 units (-inf stays -inf)
  // a row starts at its first finite score; afterwards it rescales only when the
  // block exceeds the reference by more than the slack
  const bool started = st.m != -INFINITY;
  const bool need = started ? mx - st.m > kRescaleSlack : mx != -INFINITY;
  if (__any(need)) {
    if (need) {
      const float alpha = started ? fast_exp2(st.m - mx) : 0.f;
      st.l *= alpha;
      st.lb *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) st.o[t][r] *= alpha;
      st.m = mx;
    }
  }
  const float nref = st.m != -INFINITY ? -st.m : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = fast_exp2(__builtin_fmaf(s0[r], sl2, nref));
    s1[r] = fast_exp2(__builtin_fmaf(s1[r], sl2, nref));
  }
  float rs0 = s0[0], rs1 = s1[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    rs0 += s0[r];
    rs1 += s1[r];
  }
  st.l += rs0 + rs1;
  pc[0] = pack8(s0, 0);
  pc[1] = pack8(s0, 8);
  pc[2] = pack8(s1, 0);
  pc[3] = pack8(s1, 8);
  // row sum of the rounded probabilities: one dot product with (1, 1) per pair
  float rb0 = 0.f, rb1 = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 u0 = __builtin_bit_cast(u32x4, pc[c]);
    const u32x4 u1 = __builtin_bit_cast(u32x4, pc[c + 2]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rb0 = sum_bf16x2(u0[e], rb0);
      rb1 = sum_bf16x2(u1[e], rb1);
    }
  }
  st.lb += rb0 + rb1;
}

// O^T += V^T P^T; V is the natural LDS tile sV, its transposed operand comes from
// ds_read_b64_tr_b16 reads: v[(D/32) c + t] is key chunk c of O^T tile t.  pv_load
// issues the reads (early, so that their latency hides behind the softmax), pv_mma
// the MFMAs.
template <int NV>
__device__ __forceinline__ void pv_load(const uint16_t* sV, int lane, bf16x8 (&v)[NV]) {
  constexpr int D = 8 * NV, kT = D / 32;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < kT; ++t) v[kT * c + t] = ld_tr8<D>(sV, t, c, lane);
}

template <int NV, int D>
__device__ __forceinline__ void pv_mma(const bf16x8 (&v)[NV], const bf16x8 (&pc)[4],
                                       FwdStateT<D>& st) {
  static_assert(NV == D / 8, "one operand per key chunk and O^T tile");
  constexpr int kT = D / 32;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int t = 0; t < kT; ++t) st.o[t] = mfma32(v[kT * c + t], pc[c], st.o[t]);
}

template <int D>
__device__ __forceinline__ void pv_tile(const uint16_t* sV, const bf16x8 (&pc)[4], int lane,
                                        FwdStateT<D>& st) {
  bf16x8 v[D / 8];
  pv_load(sV, lane, v);
  pv_mma(v, pc, st);
}

// Final write of a finished row: O (bf16, normalised by lb_tot), optionally its
// rounding residual O - bf16(O) rounded to bf16 (olo_row, may be null), and lse
// (natural log, from l_tot).  orow / olo_row point at this lane's query row;
// lse_out may be null.  l_tot and lb_tot are the row's full sums (both
// half-lanes, partner_sum) of st.l and st.lb.
template <int D>
__device__ __forceinline__ void write_o_bf16(const FwdStateT<D>& st, float l_tot, float lb_tot,
                                             int hl, uint16_t* orow, uint16_t* olo_row,
                                             float* lse_out) {
  const float inv = 1.f / lb_tot;
  uint16_t* op = orow + 4 * hl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    constexpr int kT = D / 32;
    float x[kT][4];
    u32x2 w[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[t][e] = st.o[t][4 * j + e] * inv;
      w[t][0] = pack_bf16x2(x[t][0], x[t][1]);
      w[t][1] = pack_bf16x2(x[t][2], x[t][3]);
    }
#pragma unroll
    for (int t = 0; t < kT; ++t) *reinterpret_cast<u32x2*>(op + 32 * t + 8 * j) = w[t];
    if (olo_row != nullptr) {
      uint16_t* lp = olo_row + 4 * hl;
#pragma unroll
      for (int t = 0; t < kT; ++t) {
        u32x2 r;
        r[0] = pack_bf16x2(x[t][0] - bf16_lo(w[t][0]), x[t][1] - bf16_hi(w[t][0]));
        r[1] = pack_bf16x2(x[t][2] - bf16_lo(w[t][1]), x[t][3] - bf16_hi(w[t][1]));
        *reinterpret_cast<u32x2*>(lp + 32 * t + 8 * j) = r;
      }
    }
  }
  if (lse_out != nullptr && hl == 0) *lse_out = (st.m + __log2f(l_tot)) * kLn2;
}

// Partial record of a split full row: O unnormalised [64][D] fp32, then m[64]
// (log2 units), l[64] and lb[64] (the two row sums), row qr of the query tile.
template <int D>
constexpr int kPartFloatsOf = kBlock * D + 3 * kBlock;
constexpr int kPartFloats = kPartFloatsOf<kHead>;

template <int D>
__device__ __forceinline__ void write_partial(const FwdStateT<D>& st, float l_tot, float lb_tot,
                                              int hl, int qr, float* rec) {
  float* orow = rec + qr * D + 4 * hl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = st.o[t][4 * j + e];
      *reinterpret_cast<f32x4*>(orow + 32 * t + 8 * j) = w;
    }
  }
  if (hl == 0) {
    rec[kBlock * D + qr] = st.m;
    rec[kBlock * D + kBlock + qr] = l_tot;
    rec[kBlock * D + 2 * kBlock + qr] = lb_tot;
  }
}

// Merge nseg partial records (stride kPartFloatsOf<D>) for row `row`, columns dq..dq+15,
// in segment order: M = max m_s, f_s = 2^(m_s - M), L = sum l_s f_s,
// Lb = sum lb_s f_s, acc = sum O_s f_s (O is then acc / Lb, lse M + log2 L).
// Up to kMergeBatch records are read with all their loads in flight together (one
// memory round trip: these merges run on few work-groups and are latency-bound);
// the arithmetic is the same, in the same order, either way.
constexpr int kMergeBatch = 8;

template <int D = kHead>
__device__ __forceinline__ void merge_partials(const float* base, int nseg, int row, int dq,
                                               float (&acc)[16], float& M, float& L,
                                               float& Lb) {
  constexpr int kPart = kPartFloatsOf<D>;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  L = 0.f;
  Lb = 0.f;
  constexpr int kM = kBlock * D, kL = kM + kBlock, kLb = kM + 2 * kBlock;
  if (nseg <= kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], lbv[kMergeBatch];
    f32x4 x[kMergeBatch][4];
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s) {
      if (s < nseg) {
        const float* ps = base + (size_t)s * kPart;
        mv[s] = ps[kM + row];
        lv[s] = ps[kL + row];
        lbv[s] = ps[kLb + row];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[s][q] = *reinterpret_cast<const f32x4*>(ps + row * D + dq + 4 * q);
      }
    }
    M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s)
      if (s < nseg) M = fmaxf(M, mv[s]);
    const float Mref = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s) {
      if (s < nseg) {
        const float f = fast_exp2(mv[s] - Mref);
        L += lv[s] * f;
        Lb += lbv[s] * f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[4 * q] += x[s][q][0] * f;
          acc[4 * q + 1] += x[s][q][1] * f;
          acc[4 * q + 2] += x[s][q][2] * f;
          acc[4 * q + 3] += x[s][q][3] * f;
        }
      }
    }
    return;
  }
  M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < nseg; ++s) M = fmaxf(M, base[(size_t)s * kPart + kM + row]);
  const float Mref = M == -INFINITY ? 0.f : M;
#pragma unroll 4
  for (int s = 0; s < nseg; ++s) {
    const float* ps = base + (size_t)s * kPart;
    const float f = fast_exp2(ps[kM + row] - Mref);
    L += ps[kL + row] * f;
    Lb += ps[kLb + row] * f;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ps + row * D + dq + e);
      acc[e] += x[0] * f;
      acc[e + 1] += x[1] * f;
      acc[e + 2] += x[2] * f;
      acc[e + 3] += x[3] * f;
    }
  }
}

// Sum of nseg fp32 partial tiles (16 consecutive floats at src + s*stride), in
// segment order; up to kMergeBatch tiles with all loads in flight together.
__device__ __forceinline__ void sum_partials(const float* src, size_t stride, int nseg,
                                             float (&acc)[16]) {
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  if (nseg <= kMergeBatch) {
    f32x4 x[kMergeBatch][4];
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s)
      if (s < nseg)
#pragma unroll
        for (int q = 0; q < 4; ++q) x[s][q] = *reinterpret_cast<const f32x4*>(src + s * stride + 4 * q);
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s)
      if (s < nseg)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[4 * q] += x[s][q][0];
          acc[4 * q + 1] += x[s][q][1];
          acc[4 * q + 2] += x[s][q][2];
          acc[4 * q + 3] += x[s][q][3];
        }
    return;
  }
#pragma unroll 4
  for (int s = 0; s < nseg; ++s) {
    const float* ps = src + (size_t)s * stride;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ps + e);
      acc[e] += x[0]; acc[e + 1] += x[1]; acc[e + 2] += x[2]; acc[e + 3] += x[3];
    }
  }
}

// The same, plus the bf16 rounding residual of each value at dst_lo (may be null).
__device__ __forceinline__ void store16_bf16_lo(uint16_t* dst, uint16_t* dst_lo,
                                                const float (&acc)[16], float mul) {
#pragma unroll
  for (int e = 0; e < 16; e += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = acc[e + i] * mul;
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(dst + e) = w;
    if (dst_lo != nullptr) {
      u32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16x2(x[2 * i] - bf16_lo(w[i]), x[2 * i + 1] - bf16_hi(w[i]));
      *reinterpret_cast<u32x4*>(dst_lo + e) = r;
    }
  }
}

__device__ __forceinline__ void store16_bf16(uint16_t* dst, const float (&acc)[16], float mul) {
#pragma unroll
  for (int e = 0; e < 16; e += 8) {
    u32x4 w;
    w[0] = pack_bf16x2(acc[e] * mul, acc[e + 1] * mul);
    w[1] = pack_bf16x2(acc[e + 2] * mul, acc[e + 3] * mul);
    w[2] = pack_bf16x2(acc[e + 4] * mul, acc[e + 5] * mul);
    w[3] = pack_bf16x2(acc[e + 6] * mul, acc[e + 7] * mul);
    *reinterpret_cast<u32x4*>(dst + e) = w;
  }
}

}  // namespace bsattn
