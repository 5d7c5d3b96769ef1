// One step of the streaming attention forward for a 64-row query tile held by two
// waves (wave w owns query rows 32w..32w+31, one query per lane column):
//   S^T = K Q^T over a 64-key tile, online softmax in fp32, O^T += V^T P^T.
// Shared by the block-sparse and the banded forward kernels.
#pragma once

#include "common.hpp"

namespace bsattn {

struct FwdState {
  f32x16 o0, o1;   // O^T accumulators: d rows 0..31 and 32..63, column = query
  f32x16 cinit;    // every register = -(reference max), the QK^T accumulator seed
  float m;         // reference max (log2 units), -inf until the row saw a finite score
  float l;         // this half-lane's share of the row sum
};

__device__ __forceinline__ void fwd_state_init(FwdState& st) {
  st.o0 = zero16();
  st.o1 = zero16();
  st.cinit = zero16();
  st.m = -INFINITY;
  st.l = 0.f;
}

// reference currently baked into st.cinit
__device__ __forceinline__ float seed_ref(const FwdState& st) {
  return st.m != -INFINITY ? st.m : 0.f;
}

// Q operand pre-scaled by sl2 = scale*log2(e) (rounded to bf16), so that the QK^T
// products come out in log2 units.
__device__ __forceinline__ void scale_operands(bf16x8 (&qB)[4], float sl2) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 u = __builtin_bit_cast(u32x4, qB[c]);
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(bf16_lo(u[e]) * sl2, bf16_hi(u[e]) * sl2);
    qB[c] = __builtin_bit_cast(bf16x8, w);
  }
}

// The same rounding applied to a staged tile (32 values per thread), so that a
// kernel holding Q in LDS tiles scores with exactly the forward's operands.
__device__ __forceinline__ void scale_tile(TileRegs& t, float sl2) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(bf16_lo(t.v[u][e]) * sl2, bf16_hi(t.v[u][e]) * sl2);
    t.v[u] = w;
  }
}

// S^T for the 64 keys of the LDS tile sK (natural layout) against this lane's query,
// accumulated on top of `seed`.  s0 holds keys 0..31, s1 keys 32..63; register r <->
// key 8*(r/4) + 4*hl + r%4.
__device__ __forceinline__ void qk_tile(const uint16_t* sK, const bf16x8 (&qB)[4], int col,
                                        int hl, const f32x16& seed, f32x16& s0, f32x16& s1) {
  bf16x8 a[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a[2 * c] = ld16(sK + col * kLdsStride + 16 * c + 8 * hl);
    a[2 * c + 1] = ld16(sK + (32 + col) * kLdsStride + 16 * c + 8 * hl);
  }
  s0 = mfma32(a[0], qB[0], seed);
  s1 = mfma32(a[1], qB[0], seed);
#pragma unroll
  for (int c = 1; c < 4; ++c) {
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

// Online softmax over one key tile whose scores s = S' - m_c arrive relative to the
// seeded reference m_c (log2 units; -inf marks an excluded key).  The reference
// only moves when a block's maximum exceeds it by more than kRescaleSlack, so the
// unnormalised probabilities 2^s stay below 2^kRescaleSlack and most blocks need
// no rescale of O and l; the result is exact either way since numerator and
// denominator share the reference.  On return pc[c] holds the bf16 probabilities
// of key chunk c as MFMA operands and st.l has grown by their fp32 sum.
constexpr float kRescaleSlack = 8.f;

// ref_used is the reference the scores were seeded with (the reference can have
// moved since, when the next block's scores are computed ahead of this softmax).
__device__ __forceinline__ void softmax_step(f32x16& s0, f32x16& s1, FwdState& st,
                                             bf16x8 (&pc)[4], float ref_used) {
  float mx = __builtin_fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s0[r]), s1[r]);
  mx = partner_max(mx);
  {
    const float now = st.m != -INFINITY ? st.m : 0.f;
    const float shift = now - ref_used;
    if (__any(shift != 0.f)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] -= shift;
        s1[r] -= shift;
      }
      mx -= shift;
    }
  }
  // a row starts at its first finite score; afterwards it rescales only when the
  // block exceeds the reference by more than the slack
  const bool started = st.m != -INFINITY;
  const bool need = started ? mx > kRescaleSlack : mx != -INFINITY;
  if (__any(need)) {
    if (need) {
      const float mc = started ? st.m : 0.f;    // reference baked into the seed
      const float m_new = mc + mx;
      const float alpha = started ? fast_exp2(st.m - m_new) : 0.f;
      st.l *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st.o0[r] *= alpha;
        st.o1[r] *= alpha;
        s0[r] -= mx;
        s1[r] -= mx;
        st.cinit[r] = -m_new;
      }
      st.m = m_new;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = fast_exp2(s0[r]);
    s1[r] = fast_exp2(s1[r]);
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
}

// O^T += V^T P^T; V is the natural LDS tile sV, its transposed operand comes from
// ds_read_b64_tr_b16 reads.  pv_load issues the reads (early, so that their latency
// hides behind the softmax), pv_mma the MFMAs.
__device__ __forceinline__ void pv_load(const uint16_t* sV, int lane, bf16x8 (&v)[8]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[2 * c] = ld_tr8(sV, 0, c, lane);
    v[2 * c + 1] = ld_tr8(sV, 1, c, lane);
  }
}

__device__ __forceinline__ void pv_mma(const bf16x8 (&v)[8], const bf16x8 (&pc)[4], FwdState& st) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    st.o0 = mfma32(v[2 * c], pc[c], st.o0);
    st.o1 = mfma32(v[2 * c + 1], pc[c], st.o1);
  }
}

__device__ __forceinline__ void pv_tile(const uint16_t* sV, const bf16x8 (&pc)[4], int lane,
                                        FwdState& st) {
  bf16x8 v[8];
  pv_load(sV, lane, v);
  pv_mma(v, pc, st);
}

// Final write of a finished row: O (bf16, normalised) and lse (natural log).
// orow points at this lane's query row of O; lse_out may be null.  l_tot is the
// row's full sum (both half-lanes, partner_sum).
__device__ __forceinline__ void write_o_bf16(const FwdState& st, float l_tot, int hl,
                                             uint16_t* orow, float* lse_out) {
  const float inv = 1.f / l_tot;
  uint16_t* op = orow + 4 * hl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x2 w0, w1;
    w0[0] = pack_bf16x2(st.o0[4 * j] * inv, st.o0[4 * j + 1] * inv);
    w0[1] = pack_bf16x2(st.o0[4 * j + 2] * inv, st.o0[4 * j + 3] * inv);
    w1[0] = pack_bf16x2(st.o1[4 * j] * inv, st.o1[4 * j + 1] * inv);
    w1[1] = pack_bf16x2(st.o1[4 * j + 2] * inv, st.o1[4 * j + 3] * inv);
    *reinterpret_cast<u32x2*>(op + 8 * j) = w0;
    *reinterpret_cast<u32x2*>(op + 32 + 8 * j) = w1;
  }
  if (lse_out != nullptr && hl == 0) *lse_out = (st.m + __log2f(l_tot)) * kLn2;
}

// Partial record of a split full row: O unnormalised [64][64] fp32, then m[64],
// then l[64] (both log2 units / plain sums), row qr of the query tile.
constexpr int kPartFloats = kBlock * kHead + 2 * kBlock;

__device__ __forceinline__ void write_partial(const FwdState& st, float l_tot, int hl, int qr,
                                              float* rec) {
  float* orow = rec + qr * kHead + 4 * hl;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = st.o0[4 * j + e];
      w1[e] = st.o1[4 * j + e];
    }
    *reinterpret_cast<f32x4*>(orow + 8 * j) = w0;
    *reinterpret_cast<f32x4*>(orow + 32 + 8 * j) = w1;
  }
  if (hl == 0) {
    rec[kBlock * kHead + qr] = st.m;
    rec[kBlock * kHead + kBlock + qr] = l_tot;
  }
}

// Merge nseg partial records (stride kPartFloats) for row `row`, columns dq..dq+15,
// in segment order: M = max m_s, L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M) / L.
// Up to kMergeBatch records are read with all their loads in flight together (one
// memory round trip: these merges run on few work-groups and are latency-bound);
// the arithmetic is the same, in the same order, either way.
constexpr int kMergeBatch = 8;

__device__ __forceinline__ void merge_partials(const float* base, int nseg, int row, int dq,
                                               float (&acc)[16], float& M, float& L) {
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  L = 0.f;
  if (nseg <= kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    f32x4 x[kMergeBatch][4];
#pragma unroll
    for (int s = 0; s < kMergeBatch; ++s) {
      if (s < nseg) {
        const float* ps = base + (size_t)s * kPartFloats;
        mv[s] = ps[kBlock * kHead + row];
        lv[s] = ps[kBlock * kHead + kBlock + row];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[s][q] = *reinterpret_cast<const f32x4*>(ps + row * kHead + dq + 4 * q);
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
  for (int s = 0; s < nseg; ++s) M = fmaxf(M, base[(size_t)s * kPartFloats + kBlock * kHead + row]);
  const float Mref = M == -INFINITY ? 0.f : M;
#pragma unroll 4
  for (int s = 0; s < nseg; ++s) {
    const float* ps = base + (size_t)s * kPartFloats;
    const float f = fast_exp2(ps[kBlock * kHead + row] - Mref);
    L += ps[kBlock * kHead + kBlock + row] * f;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(ps + row * kHead + dq + e);
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
