// Block layout builder for BigBird-ITC attention (integer work, bit-exact).
//
// Pattern ("Big Bird: Transformers for Longer Sequences", §2 and App. D, Fig. 6;
// Chinese Big Bird walkthrough, §2.1-2.3): query block i sees the global blocks
// G, the window blocks |i - j| <= (w-1)/2 and r random blocks drawn without
// replacement from the remaining blocks; a global query block sees every block.
// The random draw is a partial Fisher-Yates over the ascending candidate list
// driven by SplitMix64 (Steele, Lea & Flood 2014) output number
// (h*nb + i)*r + t + 1 of the stream seeded with the layout seed.
//
// Two kernels, one work-group per head:
//   layout_rows: row lengths -> row_ptr (block scan), then every row's sorted list.
//   layout_cols: column counts (LDS integer atomics) -> csc_ptr, then every
//                column's ascending list of query blocks.

#include "common.hpp"
#include "internal.hpp"

namespace bsattn {
namespace {

constexpr int kBuildThreads = 256;
constexpr int kMaxR = 64;

__device__ __forceinline__ uint64_t splitmix64_draw(uint64_t seed, uint64_t k) {
  uint64_t z = seed + k * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// number of entries of the sorted array a[0..n) that are <= x
__device__ int count_le(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ bool contains(const int32_t* a, int n, int x) {
  int c = count_le(a, n, x);
  return c > 0 && a[c - 1] == x;
}

struct RowCtx {
  const int32_t* G;
  int g, nb, lo, hi;   // window [lo, hi]
  // |E intersect [0, y]| with E = G U [lo, hi]
  __device__ int excl_le(int y) const {
    int cg = count_le(G, g, y);
    int cw = 0, cgw = 0;
    if (y >= lo) {
      int top = y < hi ? y : hi;
      cw = top - lo + 1;
      cgw = count_le(G, g, top) - count_le(G, g, lo - 1);
    }
    return cg + cw - cgw;
  }
  // x-th (0-based) block that is neither global nor in the window
  __device__ int cand(int x) const {
    int y = x;
    for (;;) {
      int ny = x + excl_le(y);
      if (ny == y) return y;
      y = ny;
    }
  }
  __device__ int excl_size() const { return excl_le(nb - 1); }
};

__device__ int row_length(const int32_t* G, int g, int nb, int w, int r, int i, bool& is_global) {
  is_global = contains(G, g, i);
  if (is_global) return nb;
  const int half = (w - 1) / 2;
  RowCtx c{G, g, nb, i - half < 0 ? 0 : i - half, i + half > nb - 1 ? nb - 1 : i + half};
  const int e = c.excl_size();
  const int m = nb - e;
  return e + (r < m ? r : m);
}

__global__ __launch_bounds__(kBuildThreads) void layout_rows_kernel(
    const int32_t* __restrict__ G, int g, int nb, int w, int r, uint64_t seed,
    int64_t nnz_per_head, int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
  __shared__ int part[kBuildThreads];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int i0 = tid * per;
  const int i1 = min(nb, i0 + per);

  int local = 0;
  for (int i = i0; i < i1; ++i) {
    bool gl;
    local += row_length(G, g, nb, w, r, i, gl);
  }
  part[tid] = local;
  __syncthreads();
  // inclusive scan of the per-thread sums
  for (int off = 1; off < kBuildThreads; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int64_t head_base = (int64_t)h * nnz_per_head;
  int64_t pos = head_base + (part[tid] - local);

  for (int i = i0; i < i1; ++i) {
    bool gl;
    const int len = row_length(G, g, nb, w, r, i, gl);
    row_ptr[(int64_t)h * nb + i] = (int32_t)pos;
    int32_t* out = col_idx + pos;
    if (gl) {
      for (int j = 0; j < nb; ++j) out[j] = j;
    } else {
      const int half = (w - 1) / 2;
      RowCtx c{G, g, nb, i - half < 0 ? 0 : i - half, i + half > nb - 1 ? nb - 1 : i + half};
      const int m = nb - c.excl_size();
      const int take = r < m ? r : m;
      // partial Fisher-Yates on the virtual candidate array; only positions > t
      // can still be touched after step t, so keep a small map of moved entries
      int mkey[2 * kMaxR], mval[2 * kMaxR];
      int nmap = 0;
      int rnd[kMaxR];
      for (int t = 0; t < take; ++t) {
        const uint64_t u = splitmix64_draw(seed, (uint64_t)((int64_t)h * nb + i) * (uint64_t)r + t + 1);
        const int s = t + (int)(u % (uint64_t)(m - t));
        int vt = -1, vs = -1, slot_s = -1;
        for (int q = 0; q < nmap; ++q) {
          if (mkey[q] == t) vt = mval[q];
          if (mkey[q] == s) { vs = mval[q]; slot_s = q; }
        }
        if (vt < 0) vt = c.cand(t);
        if (vs < 0) vs = c.cand(s);
        rnd[t] = vs;                    // position t is final now
        if (s != t) {
          if (slot_s >= 0) mval[slot_s] = vt;
          else { mkey[nmap] = s; mval[nmap] = vt; ++nmap; }
        }
      }
      // sort the random blocks (insertion sort, take <= 64)
      for (int a = 1; a < take; ++a) {
        int x = rnd[a], b2 = a - 1;
        while (b2 >= 0 && rnd[b2] > x) { rnd[b2 + 1] = rnd[b2]; --b2; }
        rnd[b2 + 1] = x;
      }
      // three-way merge of G, the window [lo, hi] and the random blocks
      int pg = 0, pw = c.lo, pr = 0, nout = 0, last = -1;
      const int big = 1 << 30;
      while (nout < len) {
        int vg = pg < g ? G[pg] : big;
        int vw = pw <= c.hi ? pw : big;
        int vr = pr < take ? rnd[pr] : big;
        int v = vg < vw ? vg : vw;
        v = v < vr ? v : vr;
        if (v == vg) ++pg;
        if (v == vw) ++pw;
        if (v == vr) ++pr;
        if (v != last) { out[nout++] = v; last = v; }
      }
    }
    pos += len;
  }
  if (h == gridDim.x - 1 && tid == kBuildThreads - 1) row_ptr[(int64_t)gridDim.x * nb] = (int32_t)(head_base + nnz_per_head);
}

__global__ __launch_bounds__(kBuildThreads) void layout_cols_kernel(
    int nb, int64_t nnz_per_head, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int32_t* __restrict__ csc_ptr,
    int32_t* __restrict__ csc_idx) {
  extern __shared__ int cnt[];   // [nb]
  __shared__ int part[kBuildThreads];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  for (int j = tid; j < nb; j += kBuildThreads) cnt[j] = 0;
  __syncthreads();
  const int32_t* rp = row_ptr + (int64_t)h * nb;
  for (int i = tid; i < nb; i += kBuildThreads) {
    for (int e = rp[i]; e < rp[i + 1]; ++e) atomicAdd(&cnt[col_idx[e]], 1);
  }
  __syncthreads();
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int j0 = tid * per, j1 = min(nb, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) local += cnt[j];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kBuildThreads; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t pos = (int64_t)h * nnz_per_head + (part[tid] - local);
  for (int j = j0; j < j1; ++j) {
    csc_ptr[(int64_t)h * nb + j] = (int32_t)pos;
    int32_t* out = csc_idx + pos;
    int k = 0;
    for (int i = 0; i < nb; ++i) {
      if (contains(col_idx + rp[i], rp[i + 1] - rp[i], j)) out[k++] = i;
    }
    pos += k;
  }
  if (h == gridDim.x - 1 && tid == kBuildThreads - 1)
    csc_ptr[(int64_t)gridDim.x * nb] = (int32_t)((int64_t)gridDim.x * nnz_per_head);
}

}  // namespace

int launch_layout_build(bsattn_layout* L, hipStream_t stream) {
  hipLaunchKernelGGL(layout_rows_kernel, dim3(L->heads), dim3(kBuildThreads), 0, stream,
                     L->d_gblk, L->g, L->nb, L->w, L->r, L->seed, L->nnz_per_head,
                     L->d_row_ptr, L->d_col_idx);
  int st = check_hip(hipGetLastError(), "layout_rows launch");
  if (st) return st;
  hipLaunchKernelGGL(layout_cols_kernel, dim3(L->heads), dim3(kBuildThreads),
                     (size_t)L->nb * sizeof(int), stream, L->nb, L->nnz_per_head,
                     L->d_row_ptr, L->d_col_idx, L->d_csc_ptr, L->d_csc_idx);
  return check_hip(hipGetLastError(), "layout_cols launch");
}

}  // namespace bsattn
