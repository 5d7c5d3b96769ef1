// Shared device and host helpers for the gfx950 attention kernels.
//
// Tile conventions used by every kernel in this library (CDNA4, wave64):
//
// * One 32x32x16 bf16 MFMA computes C[m][n] += sum_k A[m][k] B[k][n].  Lane l
//   supplies A row (l % 32) and B column (l % 32), eight k-values each, taken
//   from k-slots (l / 32, e), e = 0..7.  Which k index a slot stands for does not
//   matter as long as A and B agree, because the product sums over all slots.
// * The 16 accumulator registers of lane l hold column (l % 32) and rows
//   8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
// * A contraction over a 64-long block dimension (keys or queries) whose
//   operand comes out of a previous MFMA accumulator therefore pairs register
//   r = 8c' + e of tile t with k-slot e of chunk c = 2t + c'.  The index it stands
//   for is 16c + 8(e/4) + 4h + (e%4), h = l / 32.  The matching other operand is
//   read from a natural LDS tile (row = contraction index, 64 columns) with two
//   ds_read_b64_tr_b16: within each 16-lane group, lane 16g + 4a + b receives
//   element b of the 8-byte chunks addressed by lanes 16g + a + 4j, j = 0..3.
//   Lane s therefore addresses row 16c + 8t + 4(s/32) + (s%16)/4 (t = 0, 1),
//   columns 16((s/16)%2) + 4(s%4) .. +3, and receives column (s % 32) of rows
//   16c + 8t + 4(s/32) + j: exactly k-slots e = 4t + j of the pairing above.
// * Every LDS tile is stored in natural layout with 16-byte stores; rows are
//   padded to 72 elements so that the row-strided 16-byte and 8-byte reads above
//   spread over the banks.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "shape.hpp"

namespace bsattn {

constexpr int kLdsStride = 72;  // bf16 elements per LDS tile row (64 + 8 pad)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// acc + (both bf16 values of the packed pair w), one v_dot2 with (1, 1): the
// products by one are exact and the sum is accumulated in fp32.
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Eight consecutive accumulator registers rounded to bf16 and packed in pairs.
__device__ __forceinline__ u32x4 pack8u(const f32x16& s, int base) {
  u32x4 u;
  u[0] = pack_bf16x2(s[base + 0], s[base + 1]);
  u[1] = pack_bf16x2(s[base + 2], s[base + 3]);
  u[2] = pack_bf16x2(s[base + 4], s[base + 5]);
  u[3] = pack_bf16x2(s[base + 6], s[base + 7]);
  return u;
}

// The same, as one MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  return __builtin_bit_cast(bf16x8, pack8u(s, base));
}

// Registers base .. base+7 of s replaced by what their bf16 rounding h (the
// operand pack8(s, base) made of them) left out: s - h, exact in fp32.
__device__ __forceinline__ void residue8(f32x16& s, const bf16x8& h, int base) {
  const u32x4 u = __builtin_bit_cast(u32x4, h);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[base + 2 * e] -= bf16_lo(u[e]);
    s[base + 2 * e + 1] -= bf16_hi(u[e]);
  }
}

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0).  Placed before a loop whose body first
// reads registers loaded ahead of it: the compiler's wait for them would otherwise
// stay inside the loop and, since the counter is shared, also wait for the loads
// each iteration issues for the next one.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------------------
// Cooperative 64 x D bf16 tile staging through LDS (128 threads, D = 64 or 128):
// LDS row x holds global row x (D values + an 8-element pad, so that the
// row-strided reads spread over the banks as described above).  Thread t moves
// 16-byte chunk (t % (D/8)) of rows t / (D/8) + (1024/D) u, u = 0 .. D/16 - 1,
// so D/8 consecutive lanes cover one row.
// ---------------------------------------------------------------------------

template <int D>
constexpr int kStrideOf = D + 8;   // bf16 elements per LDS tile row
static_assert(kStrideOf<kHead> == kLdsStride, "LDS row stride of the d = 64 tiles");

template <int D>
struct TileRegsT { u32x4 v[D / 16]; };
using TileRegs = TileRegsT<kHead>;

template <int D>
__device__ __forceinline__ void gload_nat(TileRegsT<D>& r, const uint16_t* g, int tid) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  const int c = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) r.v[u] = ldg16(g + (row + kRpp * u) * D + 8 * c);
}

// The same for the last block of a sequence that ends inside it: only its first
// `rows` rows are tokens; the others are not read and are staged as zeros.
template <int D>
__device__ __forceinline__ void gload_nat_rows(TileRegsT<D>& r, const uint16_t* g, int tid,
                                               int rows) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  const int c = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row + kRpp * u < rows) x = ldg16(g + (row + kRpp * u) * D + 8 * c);
    r.v[u] = x;
  }
}

template <int D>
__device__ __forceinline__ void lds_store_nat(uint16_t* s, const TileRegsT<D>& r, int tid) {
  constexpr int kCpr = D / 8, kRpp = 128 / kCpr, kShift = D == 64 ? 3 : 4;
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  const int c = tid & (kCpr - 1), row = tid >> kShift;
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
    *reinterpret_cast<u32x4*>(s + (row + kRpp * u) * kStrideOf<D> + 8 * c) = r.v[u];
}

// MFMA operand of 8 k-slots for chunk c of a contraction over the rows of the
// natural LDS tile s (row stride D + 8), for output rows/columns 32*tile ..
// 32*tile + 31 (the tile's columns).  See the lane mapping described at the top
// of this file.
template <int D = kHead>
__device__ __forceinline__ bf16x8 ld_tr8(const uint16_t* s, int tile, int c, int lane) {
  const int row = 16 * c + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = 32 * tile + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const lds_v4i16* p0 = (const lds_v4i16*)(s + row * kStrideOf<D> + col);
  const lds_v4i16* p1 = (const lds_v4i16*)(s + (row + 8) * kStrideOf<D> + col);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4i16*>(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4i16*>(p1));
  const v4i16 both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// max over lanes l and l ^ 32 (the two halves of one accumulator column)
__device__ __forceinline__ float partner_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float partner_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// XCD-aware work mapping: the dispatcher hands consecutive work-groups to the 8
// XCDs in turn; remap so that each XCD walks one contiguous range of items (and
// so reuses the K/V blocks of the same heads from its own L2).
__device__ __forceinline__ int xcd_remap(int g, int total) {
  const int per = (total + 7) / 8;
  return (g & 7) * per + (g >> 3);
}

// The same eighths, for a list made of consecutive groups of ipb items whose
// first ng are short and the rest long: each XCD runs the long items of its eighth
// before the short ones, so the longest work starts first.  Returns the item of
// work-group g, or -1 past the end of its eighth.
__device__ __forceinline__ int xcd_item_long_first(int g, int total, int ipb, int ng) {
  const int per = (total + 7) / 8;
  const int lo = (g & 7) * per, k = g >> 3;
  const int hi = min(total, lo + per);
  if (k >= hi - lo) return -1;
  const int nl = ipb - ng;
  auto longs_before = [&](int v) {
    const int b = v / ipb, r = v - b * ipb;
    return b * nl + max(0, r - ng);
  };
  const int l0 = longs_before(lo), nlong = longs_before(hi) - l0;
  if (k < nlong) {
    const int t = l0 + k;
    return (t / nl) * ipb + ng + t % nl;
  }
  const int b0 = lo / ipb, r0 = lo - b0 * ipb;
  const int t = b0 * ng + min(r0, ng) + (k - nlong);
  return (t / ng) * ipb + t % ng;
}

}  // namespace bsattn
