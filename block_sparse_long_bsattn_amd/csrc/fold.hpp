// First level of a two-level sum of long lists of fp32 partials.
//
// The full rows of global queries and the full columns of key tiles that hold
// global keys are cut into segments, and each segment leaves an fp32 partial.  The
// work-group that owns an output tile merges its partials one after another, so
// with long sequences (hundreds of segments) that merge is bound by one
// work-group's memory round trips.  Past kFoldMin partials, a kernel first folds
// each run of `chunk` consecutive partials into one, over many work-groups at
// once, into an area of its own; the owning work-group then merges the nfold
// folded partials.  Both levels sum in a fixed order, so results stay bitwise
// reproducible (they differ from the one-level sum only in rounding order).
#pragma once

#include "attn_tile.hpp"

namespace bsattn {

constexpr int kFoldMin = 16;

// chunk = 0: no fold, the final merge reads the nseg partials.  Else runs of chunk
// partials (the smallest power of two from 8 that leaves at most 8 runs, so that
// the final merge reads all of them in one round trip) fold into
// nfold = ceil(nseg / chunk).
struct Fold {
  int chunk, nfold;
};

inline Fold fold_plan(int nseg) {
  if (nseg <= kFoldMin) return Fold{0, nseg};
  int c = 8;
  while ((int64_t)c * 8 < nseg) c *= 2;
  return Fold{c, (nseg + c - 1) / c};
}

namespace {

// Plain sums of one list: group g's partial s is `floats` floats at
// src + (g*nseg + s)*floats (floats a multiple of 1024); its fold c goes to
// dst + (g*nfold + c)*floats.  It takes groups * nfold * floats/1024 work-groups.
struct FoldSumJob {
  const float* src;
  float* dst;
  int nseg, chunk, nfold, floats, blocks;
};

inline FoldSumJob fold_sum_job(const float* src, float* dst, int groups, int nseg, Fold f,
                               int floats) {
  return FoldSumJob{src, dst, nseg, f.chunk, f.nfold, floats,
                    f.chunk ? groups * f.nfold * (floats >> 10) : 0};
}

// Two lists in one launch (a job with chunk 0 takes no work-groups): grid
// j0.blocks + j1.blocks work-groups of 256; thread t sums 4 floats.
__global__ __launch_bounds__(256) void fold_sum_kernel(FoldSumJob j0, FoldSumJob j1) {
  int b = blockIdx.x;
  const bool first = b < j0.blocks;
  if (!first) b -= j0.blocks;
  const FoldSumJob& j = first ? j0 : j1;
  const int slices = j.floats >> 10;
  const int sl = b % slices;
  b /= slices;
  const int c = b % j.nfold, g = b / j.nfold;
  const size_t e = ((size_t)sl << 10) + 4 * threadIdx.x;
  const int s0 = c * j.chunk, cnt = min(j.chunk, j.nseg - s0);
  const float* p = j.src + ((size_t)g * j.nseg + s0) * j.floats + e;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < cnt; s += 16) {
    f32x4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)   // clamped: every load is issued, none under a branch
      x[i] = *reinterpret_cast<const f32x4*>(p + (size_t)min(s + i, cnt - 1) * j.floats);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s + i < cnt) acc += x[i];
  }
  *reinterpret_cast<f32x4*>(j.dst + ((size_t)g * j.nfold + c) * j.floats + e) = acc;
}

// Softmax records (kPartFloatsOf<D> floats: O[64][D], then the row maxima m, sums
// l and lb, all in the base-2 units of the forward): the fold of a run is the
// record of the union of its segments, m = the run's maximum M, l = sum of
// l_s 2^(m_s - M), lb likewise, O = sum of O_s 2^(m_s - M); a row no segment saw
// keeps m = -inf and zeros.  Grid: groups * nfold * D/16 work-groups of 256, each
// on 1024/D rows of one record.
template <int D>
__global__ __launch_bounds__(256) void fold_softmax_kernel(const float* __restrict__ src,
                                                           float* __restrict__ dst, int nseg,
                                                           int chunk, int nfold) {
  constexpr int kPart = kPartFloatsOf<D>;
  constexpr int kM = kBlock * D, kL = kM + kBlock, kLb = kM + 2 * kBlock;
  constexpr int kRows = 1024 / D, kSlices = kBlock / kRows;
  int b = blockIdx.x;
  const int sl = b % kSlices;
  b /= kSlices;
  const int c = b % nfold, g = b / nfold;
  const int row = sl * kRows + (int)threadIdx.x / (D / 4), col = 4 * ((int)threadIdx.x % (D / 4));
  const int s0 = c * chunk, cnt = min(chunk, nseg - s0);
  const float* p = src + ((size_t)g * nseg + s0) * kPart;
  float M = -INFINITY;
  for (int s = 0; s < cnt; s += 16) {
    float mv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) mv[i] = p[(size_t)min(s + i, cnt - 1) * kPart + kM + row];
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, mv[i]);   // repeats of the last change nothing
  }
  const float Mref = M == -INFINITY ? 0.f : M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f, Lb = 0.f;
  for (int s = 0; s < cnt; s += 8) {
    f32x4 x[8];
    float mv[8], lv[8], lbv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* ps = p + (size_t)min(s + i, cnt - 1) * kPart;
      x[i] = *reinterpret_cast<const f32x4*>(ps + row * D + col);
      mv[i] = ps[kM + row];
      lv[i] = ps[kL + row];
      lbv[i] = ps[kLb + row];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s + i < cnt) {
        const float f = fast_exp2(mv[i] - Mref);
        L += lv[i] * f;
        Lb += lbv[i] * f;
        acc += x[i] * f;
      }
    }
  }
  float* q = dst + ((size_t)g * nfold + c) * kPart;
  *reinterpret_cast<f32x4*>(q + row * D + col) = acc;
  if (col == 0) {
    q[kM + row] = M;
    q[kL + row] = L;
    q[kLb + row] = Lb;
  }
}

}  // namespace
}  // namespace bsattn
