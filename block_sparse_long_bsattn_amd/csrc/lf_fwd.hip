// Longformer sliding-window + symmetric global attention forward on gfx950.
//
// Pattern ("Longformer: The Long-Document Transformer", §3.1 "Sliding Window" and
// "Global Attention"): token p attends to token q iff |p - q| <= w1, or p is
// global, or q is global.  Scores are scaled as in §3.1 eq. (1).  §3.2 and App. A
// describe the band as a banded matrix product that only computes a fixed number
// of diagonals; here the band is walked in 64x64 tiles.
//
// Kernels (per call):
//   lf_gather   packs the Q, K, V rows of the global tokens into 64-row tiles.
//   lf_band     one 128-thread work-group per 64-row query tile: the key tiles that
//               overlap the band, then the packed global-key tiles whose keys lie
//               outside those band tiles.  Only tiles the band cuts need an
//               element mask; keys that are global are allowed in every tile.
//               Rows of global tokens are skipped at write time.
//   lf_global   the global query rows are full rows ("a token with global
//               attention attends to all tokens"): packed query tiles times all key
//               tiles, split into kLfSeg-tile items writing partial records.
//   lf_combine  merges those partials in a fixed order and scatters O and lse back
//               to the global tokens' positions.

#include "attn_tile.hpp"
#include "internal.hpp"

namespace bsattn {
namespace {

constexpr int kThreads = 128;

struct LfArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const uint16_t* qg;   // packed global rows [B*H][ngt*64][64]
  const uint16_t* kg;
  const uint16_t* vg;
  float* part;          // [B*H*ngt*nseg] partial records
  const int32_t* gtok;  // [ng]
  const int32_t* gidx;  // [n]
  const uint64_t* tile_gmask;  // [nt] bit x set iff token 64u+x is global
  int heads, n, nt, ng, ngt, nseg, w1;
  int total_items;
  float sl2;
};

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__global__ __launch_bounds__(256) void lf_gather_kernel(LfArgs a) {
  const int idx = blockIdx.x;   // bh * ngt + gt
  const int bh = idx / a.ngt, gt = idx - bh * a.ngt;
  const int x = threadIdx.x >> 2, dq = (threadIdx.x & 3) * 16;
  const int j = gt * kBlock + x;
  const size_t src_bh = (size_t)bh * a.n * kHead;
  const size_t dst = ((size_t)bh * a.ngt * kBlock + j) * kHead + dq;
  uint16_t* qd = const_cast<uint16_t*>(a.qg) + dst;
  uint16_t* kd = const_cast<uint16_t*>(a.kg) + dst;
  uint16_t* vd = const_cast<uint16_t*>(a.vg) + dst;
  if (j < a.ng) {
    const size_t src = src_bh + (size_t)a.gtok[j] * kHead + dq;
#pragma unroll
    for (int e = 0; e < 16; e += 8) {
      *reinterpret_cast<u32x4*>(qd + e) = ldg16(a.q + src + e);
      *reinterpret_cast<u32x4*>(kd + e) = ldg16(a.k + src + e);
      *reinterpret_cast<u32x4*>(vd + e) = ldg16(a.v + src + e);
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; e += 8) {
      *reinterpret_cast<u32x4*>(qd + e) = z;
      *reinterpret_cast<u32x4*>(kd + e) = z;
      *reinterpret_cast<u32x4*>(vd + e) = z;
    }
  }
}

__global__ __launch_bounds__(kThreads) void lf_band_kernel(LfArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBlock * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBlock * kLdsStride];

  const int v = xcd_remap(blockIdx.x, a.total_items);
  if (v >= a.total_items) return;
  const int bh = v / a.nt, t = v - bh * a.nt;
  if (a.tile_gmask[t] == ~0ull) return;   // every row global: lf_global owns them
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)bh * a.n * kHead;
  const int i0 = t * kBlock;
  const int p = i0 + 32 * wave + col;   // this lane's query token

  bf16x8 qB[4];
  {
    const uint16_t* qp = a.q + bh_off + (size_t)p * kHead + 8 * hl;
#pragma unroll
    for (int c = 0; c < 4; ++c) qB[c] = ld16(qp + 16 * c);
  }
  const int lo_u = max(0, i0 - a.w1) / kBlock;
  const int hi_u = min(a.nt - 1, (i0 + kBlock - 1 + a.w1) / kBlock);
  const int nband = hi_u - lo_u + 1;
  const int ntile = nband + a.ngt;

  // A packed global tile gt contributes key j iff j < ng and the key's own tile
  // lies outside [lo_u, hi_u] (inside, the band tile already counts it).
  auto global_elig = [&](int gt) -> uint64_t {
    const int j = gt * kBlock + lane;
    bool ok = false;
    if (j < a.ng) {
      const int u = a.gtok[j] / kBlock;
      ok = u < lo_u || u > hi_u;
    }
    return ballot64(ok);
  };

  scale_operands(qB, a.sl2);
  FwdState st;
  fwd_state_init(st);
  const uint16_t* kg_bh = a.kg + (size_t)bh * a.ngt * kBlock * kHead;
  const uint16_t* vg_bh = a.vg + (size_t)bh * a.ngt * kBlock * kHead;
  auto tile_src = [&](int x, const uint16_t*& ks, const uint16_t*& vs) {
    if (x < nband) {
      ks = a.k + bh_off + (size_t)(lo_u + x) * kBlock * kHead;
      vs = a.v + bh_off + (size_t)(lo_u + x) * kBlock * kHead;
    } else {
      ks = kg_bh + (size_t)(x - nband) * kBlock * kHead;
      vs = vg_bh + (size_t)(x - nband) * kBlock * kHead;
    }
  };

  // skip packed tiles with no eligible key
  auto next_tile = [&](int x) -> int {
    while (x < ntile && x >= nband && global_elig(x - nband) == 0ull) ++x;
    return x;
  };

  int x = next_tile(0);
  TileRegs kr, vr;
  if (x < ntile) {
    const uint16_t *ks, *vs;
    tile_src(x, ks, vs);
    gload_nat(kr, ks, tid);
    gload_nat(vr, vs, tid);
    lds_store_nat(sK[0], kr, tid);
    lds_store_nat(sV[0], vr, tid);
  }
  int cur = 0;
  while (x < ntile) {
    __syncthreads();
    const int xn = next_tile(x + 1);
    if (xn < ntile) {
      const uint16_t *ks, *vs;
      tile_src(xn, ks, vs);
      gload_nat(kr, ks, tid);
      gload_nat(vr, vs, tid);
    }
    f32x16 s0, s1;
    qk_tile(sK[cur], qB, col, hl, st.cinit, s0, s1);
    if (x < nband) {
      const int u0 = (lo_u + x) * kBlock;
      // the whole tile lies in the band iff its farthest pair does
      const int far = max(abs(i0 - (u0 + kBlock - 1)), abs(i0 + kBlock - 1 - u0));
      if (far > a.w1) {
        const uint64_t gm = a.tile_gmask[lo_u + x];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kx = 8 * (r >> 2) + 4 * hl + (r & 3);
          const int q0 = u0 + kx, q1 = u0 + 32 + kx;
          if (abs(p - q0) > a.w1 && !((gm >> kx) & 1ull)) s0[r] = -INFINITY;
          if (abs(p - q1) > a.w1 && !((gm >> (32 + kx)) & 1ull)) s1[r] = -INFINITY;
        }
      }
    } else {
      const uint64_t el = global_elig(x - nband);
      if (el != ~0ull) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kx = 8 * (r >> 2) + 4 * hl + (r & 3);
          if (!((el >> kx) & 1ull)) s0[r] = -INFINITY;
          if (!((el >> (32 + kx)) & 1ull)) s1[r] = -INFINITY;
        }
      }
    }
    bf16x8 pc[4];
    softmax_step(s0, s1, st, pc, seed_ref(st));
    pv_tile(sV[cur], pc, lane, st);
    if (xn < ntile) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
    cur ^= 1;
    x = xn;
  }

  const float l_tot = partner_sum(st.l);
  if (a.gidx[p] < 0)
    write_o_bf16(st, l_tot, hl, a.o + bh_off + (size_t)p * kHead,
                 a.lse != nullptr ? a.lse + (size_t)bh * a.n + p : nullptr);
}

__global__ __launch_bounds__(kThreads) void lf_global_kernel(LfArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBlock * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBlock * kLdsStride];

  const int per_bh = a.ngt * a.nseg;
  const int v = xcd_remap(blockIdx.x, a.total_items);
  if (v >= a.total_items) return;
  const int bh = v / per_bh;
  const int rem = v - bh * per_bh;
  const int gt = rem / a.nseg, s = rem - gt * a.nseg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const size_t bh_off = (size_t)bh * a.n * kHead;
  const int qr = 32 * wave + col;

  bf16x8 qB[4];
  {
    const uint16_t* qp = a.qg + ((size_t)bh * a.ngt * kBlock + gt * kBlock + qr) * kHead + 8 * hl;
#pragma unroll
    for (int c = 0; c < 4; ++c) qB[c] = ld16(qp + 16 * c);
  }
  const int u_begin = s * kLfSeg;
  const int u_end = min(a.nt, u_begin + kLfSeg);
  scale_operands(qB, a.sl2);
  FwdState st;
  fwd_state_init(st);
  TileRegs kr, vr;
  gload_nat(kr, a.k + bh_off + (size_t)u_begin * kBlock * kHead, tid);
  gload_nat(vr, a.v + bh_off + (size_t)u_begin * kBlock * kHead, tid);
  lds_store_nat(sK[0], kr, tid);
  lds_store_nat(sV[0], vr, tid);
  for (int u = u_begin; u < u_end; ++u) {
    const int cur = (u - u_begin) & 1;
    __syncthreads();
    const bool more = u + 1 < u_end;
    if (more) {
      gload_nat(kr, a.k + bh_off + (size_t)(u + 1) * kBlock * kHead, tid);
      gload_nat(vr, a.v + bh_off + (size_t)(u + 1) * kBlock * kHead, tid);
    }
    f32x16 s0, s1;
    qk_tile(sK[cur], qB, col, hl, st.cinit, s0, s1);
    bf16x8 pc[4];
    softmax_step(s0, s1, st, pc, seed_ref(st));
    pv_tile(sV[cur], pc, lane, st);
    if (more) {
      lds_store_nat(sK[cur ^ 1], kr, tid);
      lds_store_nat(sV[cur ^ 1], vr, tid);
    }
  }
  const float l_tot = partner_sum(st.l);
  write_partial(st, l_tot, hl, qr, a.part + (size_t)v * kPartFloats);
}

__global__ __launch_bounds__(256) void lf_combine_kernel(LfArgs a) {
  const int idx = blockIdx.x;   // bh * ngt + gt
  const int bh = idx / a.ngt, gt = idx - bh * a.ngt;
  const int row = threadIdx.x >> 2, dq = (threadIdx.x & 3) * 16;
  const int j = gt * kBlock + row;
  if (j >= a.ng) return;
  float acc[16], M, L;
  merge_partials(a.part + (size_t)idx * a.nseg * kPartFloats, a.nseg, row, dq, acc, M, L);
  const int tok = a.gtok[j];
  store16_bf16(a.o + ((size_t)bh * a.n + tok) * kHead + dq, acc, 1.f / L);
  if (a.lse != nullptr && (threadIdx.x & 3) == 0)
    a.lse[(size_t)bh * a.n + tok] = (M + __log2f(L)) * kLn2;
}

struct LfWs {
  size_t qg, kg, vg, part, total;
};

LfWs lf_ws_layout(const lfattn_plan* P, int batch, int heads) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  LfWs w;
  const size_t bh = (size_t)batch * heads;
  const size_t tile_bytes = (size_t)P->ngt * kBlock * kHead * sizeof(uint16_t);
  w.qg = 0;
  w.kg = up(w.qg + bh * tile_bytes);
  w.vg = up(w.kg + bh * tile_bytes);
  w.part = up(w.vg + bh * tile_bytes);
  w.total = up(w.part + bh * P->ngt * P->nseg * kPartFloats * sizeof(float));
  return w;
}

}  // namespace

size_t lf_workspace_bytes(const lfattn_plan* P, int batch, int heads) {
  if (P->ng == 0) return 0;
  return lf_ws_layout(P, batch, heads).total;
}

int launch_lf_fwd(const lfattn_plan* P, int batch, int heads, float scale, const void* q,
                  const void* k, const void* v, void* o, float* lse, void* ws,
                  hipStream_t stream) {
  LfArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o; a.lse = lse;
  const bool has_g = P->ng > 0;
  LfWs w = lf_ws_layout(P, batch, heads);
  char* base = (char*)ws;
  a.qg = has_g ? (const uint16_t*)(base + w.qg) : nullptr;
  a.kg = has_g ? (const uint16_t*)(base + w.kg) : nullptr;
  a.vg = has_g ? (const uint16_t*)(base + w.vg) : nullptr;
  a.part = has_g ? (float*)(base + w.part) : nullptr;
  a.gtok = P->d_gtok; a.gidx = P->d_gidx; a.tile_gmask = P->d_tile_gmask;
  a.heads = heads; a.n = P->n; a.nt = P->nt; a.ng = P->ng; a.ngt = P->ngt;
  a.nseg = P->nseg; a.w1 = P->w1;
  a.sl2 = scale * kLog2e;
  const int bhn = batch * heads;
  int st;
  if (has_g) {
    {
    ProfScope prof_("lf_gather", stream);
    hipLaunchKernelGGL(lf_gather_kernel, dim3(bhn * P->ngt), dim3(256), 0, stream, a);
  }
    if ((st = check_hip(hipGetLastError(), "lf_gather launch"))) return st;
  }
  a.total_items = bhn * P->nt;
  {
    ProfScope prof_("lf_band", stream);
    hipLaunchKernelGGL(lf_band_kernel, dim3(8 * ((a.total_items + 7) / 8)), dim3(kThreads), 0,
                       stream, a);
  }
  if ((st = check_hip(hipGetLastError(), "lf_band launch"))) return st;
  if (!has_g) return 0;
  a.total_items = bhn * P->ngt * P->nseg;
  {
    ProfScope prof_("lf_global", stream);
    hipLaunchKernelGGL(lf_global_kernel, dim3(8 * ((a.total_items + 7) / 8)), dim3(kThreads), 0,
                       stream, a);
  }
  if ((st = check_hip(hipGetLastError(), "lf_global launch"))) return st;
  {
    ProfScope prof_("lf_combine", stream);
    hipLaunchKernelGGL(lf_combine_kernel, dim3(bhn * P->ngt), dim3(256), 0, stream, a);
  }
  return check_hip(hipGetLastError(), "lf_combine launch");
}

}  // namespace bsattn
