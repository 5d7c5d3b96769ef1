// Helpers shared by the Longformer forward and backward kernels: tiles whose rows
// are global tokens are gathered by index from the [n][64] tensors.
#pragma once

#include "common.hpp"

namespace bsattn {

// Token behind row x of global tile gt: the (gt*64 + x)-th global token; rows past
// the last one repeat it (their keys or queries are masked out or not written).
__device__ __forceinline__ int global_token(const int32_t* gtok, int ng, int gt, int x) {
  return gtok[min(gt * kBlock + x, ng - 1)];
}

// gload_nat for a tile of global tokens, rows gathered from `base` ([n][64]).
__device__ __forceinline__ void gload_gather(TileRegs& r, const uint16_t* base,
                                             const int32_t* gtok, int ng, int gt, int tid) {
  const int c = tid & 7, row = tid >> 3;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    r.v[u] = ldg16(base + (size_t)global_token(gtok, ng, gt, row + 16 * u) * kHead + 8 * c);
}

// Which rows of global tile gt are global tokens whose own 64-token tile lies
// outside [lo, hi] (inside, a natural tile of that range already holds them):
// bit x <-> row x.  Every lane of the wave must call it.
__device__ __forceinline__ uint64_t global_rows_outside(const int32_t* gtok, int ng, int gt,
                                                        int lo, int hi, int lane) {
  const int j = gt * kBlock + lane;
  bool ok = false;
  if (j < ng) {
    const int u = gtok[j] / kBlock;
    ok = u < lo || u > hi;
  }
  return __ballot(ok);
}

// Band tiles of tile t: the tiles holding a token within w1 of one of t's tokens.
__device__ __forceinline__ void band_range(int t, int w1, int nt, int& lo, int& hi) {
  const int i0 = t * kBlock;
  lo = max(0, i0 - w1) / kBlock;
  hi = min(nt - 1, (i0 + kBlock - 1 + w1) / kBlock);
}

}  // namespace bsattn
