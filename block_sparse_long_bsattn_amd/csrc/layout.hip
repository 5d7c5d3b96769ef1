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
// Kernels:
//   layout_rowptr (at build only): row lengths -> row offsets (block scan); they do
//                 not depend on the draws, so a redraw keeps them.
//   layout_head   (n/b <= 512): one work-group per head does everything: rows,
//                 random picks marked in an LDS bitmap, column lengths, column
//                 offsets (block scan) and column lists.
//   layout_rows + layout_cols (larger n/b): the same two phases as separate
//                 kernels with the bitmap in global memory (cleared after use).
// Row lists are written by rank: the position of a key block in the sorted union
// G U W_i U R_i is the number of union members below it, so no merge buffers are
// needed.  Random draws for r <= 8 stay in registers.

#include "common.hpp"
#include "internal.hpp"

namespace bsattn {
namespace {

constexpr int kBuildThreads = 256;
constexpr int kMaxR = 64;      // largest r accepted by the C ABI
constexpr int kFastR = 8;      // draws held in registers up to this r
constexpr int kLdsBitmapNb = 512;

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

__device__ RowCtx row_ctx(const int32_t* G, int g, int nb, int w, int i) {
  const int half = (w - 1) / 2;
  return RowCtx{G, g, nb, i - half < 0 ? 0 : i - half, i + half > nb - 1 ? nb - 1 : i + half};
}

__device__ int row_length(const int32_t* G, int g, int nb, int w, int r, int i, bool& is_global) {
  is_global = contains(G, g, i);
  if (is_global) return nb;
  const RowCtx c = row_ctx(G, g, nb, w, i);
  const int e = c.excl_size();
  const int m = nb - e;
  return e + (r < m ? r : m);
}

// Writes row i's sorted key blocks G U [lo, hi] U R (R sorted, disjoint from the
// rest) by rank.  cnt_r_below(x) = #{y in R : y < x}; rnd_at(t) = t-th of R.
template <typename CountR, typename AtR>
__device__ void write_row(const RowCtx& c, int take, CountR cnt_r_below, AtR rnd_at, int32_t* out) {
  const int32_t* G = c.G;
  const int g = c.g;
  // window members that are not global, below x
  auto win_below = [&](int x) -> int {
    if (x <= c.lo) return 0;
    const int top = x - 1 < c.hi ? x - 1 : c.hi;
    return (top - c.lo + 1) - (count_le(G, g, top) - count_le(G, g, c.lo - 1));
  };
  for (int a = 0; a < g; ++a) {
    const int x = G[a];
    out[a + win_below(x) + cnt_r_below(x)] = x;
  }
  for (int x = c.lo; x <= c.hi; ++x) {
    if (contains(G, g, x)) continue;
    out[count_le(G, g, x - 1) + win_below(x) + cnt_r_below(x)] = x;
  }
  for (int t = 0; t < take; ++t) {
    const int x = rnd_at(t);
    out[count_le(G, g, x - 1) + win_below(x) + t] = x;
  }
}

// Random blocks of one row for r <= kFastR, kept in registers: a partial
// Fisher-Yates whose swaps are logged per step (position written, value); the
// value at a position is the latest logged write to it, else the untouched
// candidate.  Positions below the current step are never read again.
__device__ void draw_fast(const RowCtx& c, int m, int take, uint64_t seed, uint64_t k0,
                          int (&rnd)[kFastR]) {
  int key[kFastR], val[kFastR];
#pragma unroll
  for (int t = 0; t < kFastR; ++t) {
    key[t] = -1;
    val[t] = 0;
    rnd[t] = 0x7fffffff;
  }
#pragma unroll
  for (int t = 0; t < kFastR; ++t) {
    if (t < take) {
      const uint64_t u = splitmix64_draw(seed, k0 + t);
      const int s = t + (int)(u % (uint64_t)(m - t));
      int vt = -1, vs = -1;
#pragma unroll
      for (int q = 0; q < t; ++q) {
        if (key[q] == t) vt = val[q];
        if (key[q] == s) vs = val[q];
      }
      if (vt < 0) vt = c.cand(t);
      if (vs < 0) vs = c.cand(s);
      rnd[t] = vs;
      key[t] = s != t ? s : -1;
      val[t] = vt;
    }
  }
  // sorting network (odd-even transposition) on the padded array
#pragma unroll
  for (int pass = 0; pass < kFastR; ++pass) {
#pragma unroll
    for (int q = pass & 1; q + 1 < kFastR; q += 2) {
      const int a = rnd[q], b = rnd[q + 1];
      rnd[q] = a < b ? a : b;
      rnd[q + 1] = a < b ? b : a;
    }
  }
}

// General r (up to kMaxR): the same algorithm with per-thread arrays.
__device__ void draw_any(const RowCtx& c, int m, int take, uint64_t seed, uint64_t k0,
                         int* rnd) {
  int key[kMaxR], val[kMaxR];
  for (int t = 0; t < take; ++t) {
    const uint64_t u = splitmix64_draw(seed, k0 + t);
    const int s = t + (int)(u % (uint64_t)(m - t));
    int vt = -1, vs = -1;
    for (int q = 0; q < t; ++q) {
      if (key[q] == t) vt = val[q];
      if (key[q] == s) vs = val[q];
    }
    if (vt < 0) vt = c.cand(t);
    if (vs < 0) vs = c.cand(s);
    rnd[t] = vs;
    key[t] = s != t ? s : -1;
    val[t] = vt;
  }
  for (int a = 1; a < take; ++a) {
    int x = rnd[a], b = a - 1;
    while (b >= 0 && rnd[b] > x) { rnd[b + 1] = rnd[b]; --b; }
    rnd[b + 1] = x;
  }
}

// Build row i of head h: its sorted list at out and its random picks marked in
// the column-major bitmap (word (j, i/32) of head h's bitmap `hb`, wpc words per
// column; atomics on LDS or global memory).
__device__ void build_row(const int32_t* G, int g, int nb, int w, int r, uint64_t seed, int h,
                          int i, int32_t* out, uint32_t* hb, int wpc) {
  if (contains(G, g, i)) {
    for (int j = 0; j < nb; ++j) out[j] = j;
    return;
  }
  const RowCtx c = row_ctx(G, g, nb, w, i);
  const int m = nb - c.excl_size();
  const int take = r < m ? r : m;
  const uint64_t k0 = (uint64_t)((int64_t)h * nb + i) * (uint64_t)r + 1;
  if (r <= kFastR) {
    int rnd[kFastR];
    draw_fast(c, m, take, seed, k0, rnd);
    auto cnt = [&](int x) {
      int n = 0;
#pragma unroll
      for (int t = 0; t < kFastR; ++t) n += rnd[t] < x;
      return n;
    };
    auto at = [&](int t) {
      int v = 0;
#pragma unroll
      for (int q = 0; q < kFastR; ++q) v = q == t ? rnd[q] : v;
      return v;
    };
    write_row(c, take, cnt, at, out);
#pragma unroll
    for (int t = 0; t < kFastR; ++t)
      if (t < take) atomicOr(&hb[(int64_t)rnd[t] * wpc + (i >> 5)], 1u << (i & 31));
  } else {
    int rnd[kMaxR];
    draw_any(c, m, take, seed, k0, rnd);
    auto cnt = [&](int x) {
      int n = 0;
      for (int t = 0; t < take; ++t) n += rnd[t] < x;
      return n;
    };
    auto at = [&](int t) { return rnd[t]; };
    write_row(c, take, cnt, at, out);
    for (int t = 0; t < take; ++t) atomicOr(&hb[(int64_t)rnd[t] * wpc + (i >> 5)], 1u << (i & 31));
  }
}

// Column j: length, and the ascending list.  The query blocks seeing key block j
// are all blocks when j is global, otherwise the global blocks, the non-global
// blocks within the window of j, and the blocks whose random draw picked j; the
// three sets are disjoint.
__device__ int col_length(const int32_t* G, int g, int nb, int w, int j, const uint32_t* bits,
                          int wpc) {
  if (contains(G, g, j)) return nb;
  const int half = (w - 1) / 2;
  const int lo = j - half < 0 ? 0 : j - half, hi = j + half > nb - 1 ? nb - 1 : j + half;
  int n = g + (hi - lo + 1) - (count_le(G, g, hi) - count_le(G, g, lo - 1));
  for (int x = 0; x < wpc; ++x) n += __popc(bits[x]);
  return n;
}

__device__ void write_col(const int32_t* G, int g, int nb, int w, int j, uint32_t* bits, int wpc,
                          int32_t* out) {
  int k = 0;
  if (contains(G, g, j)) {
    for (int i = 0; i < nb; ++i) out[k++] = i;
  } else {
    const int half = (w - 1) / 2;
    const int lo = j - half < 0 ? 0 : j - half, hi = j + half > nb - 1 ? nb - 1 : j + half;
    int pg = 0, pw = lo, x = 0;
    uint32_t word = wpc > 0 ? bits[0] : 0u;
    const int big = 1 << 30;
    for (;;) {
      while (pw <= hi && contains(G, g, pw)) ++pw;       // window rows exclude G
      while (word == 0u && x + 1 < wpc) word = bits[++x];
      const int vg = pg < g ? G[pg] : big;
      const int vw = pw <= hi ? pw : big;
      const int vr = word ? 32 * x + __builtin_ctz(word) : big;
      int v = vg < vw ? vg : vw;
      v = v < vr ? v : vr;
      if (v == big) break;
      out[k++] = v;
      if (v == vg) ++pg;
      else if (v == vw) ++pw;
      else word &= word - 1u;
    }
  }
  for (int y = 0; y < wpc; ++y) bits[y] = 0u;          // ready for the next draw
}

// inclusive Hillis-Steele scan of part[0..kBuildThreads) in LDS
__device__ void block_scan(int* part, int tid) {
  for (int off = 1; off < kBuildThreads; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBuildThreads) void layout_rowptr_kernel(
    const int32_t* __restrict__ G, int g, int nb, int w, int r, int heads,
    int64_t nnz_per_head, int32_t* __restrict__ row_ptr) {
  __shared__ int part[kBuildThreads];
  const int tid = threadIdx.x;
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    bool gl;
    local += row_length(G, g, nb, w, r, i, gl);
  }
  part[tid] = local;
  __syncthreads();
  block_scan(part, tid);
  int pos = part[tid] - local;
  for (int i = i0; i < i1; ++i) {
    for (int h = 0; h < heads; ++h) row_ptr[(int64_t)h * nb + i] = (int32_t)(h * nnz_per_head + pos);
    bool gl;
    pos += row_length(G, g, nb, w, r, i, gl);
  }
  if (tid == 0) row_ptr[(int64_t)heads * nb] = (int32_t)(heads * nnz_per_head);
}

// One work-group per head, nb <= kLdsBitmapNb: bitmap (nb x wpc words) in LDS.
__global__ __launch_bounds__(kBuildThreads) void layout_head_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int r, uint64_t seed,
    int64_t nnz_per_head, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ csc_ptr, int32_t* __restrict__ csc_idx) {
  extern __shared__ int32_t dyn[];          // G[g] then bitmap[nb * wpc]
  __shared__ int part[kBuildThreads];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int wpc = (nb + 31) / 32;
  int32_t* sG = dyn;
  uint32_t* bm = reinterpret_cast<uint32_t*>(dyn + g);
  for (int x = tid; x < g; x += kBuildThreads) sG[x] = Gglob[x];
  for (int x = tid; x < nb * wpc; x += kBuildThreads) bm[x] = 0u;
  __syncthreads();
  for (int i = tid; i < nb; i += kBuildThreads)
    build_row(sG, g, nb, w, r, seed, h, i, col_idx + row_ptr[(int64_t)h * nb + i], bm, wpc);
  __syncthreads();
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int j0 = min(nb, tid * per), j1 = min(nb, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) local += col_length(sG, g, nb, w, j, bm + j * wpc, wpc);
  part[tid] = local;
  __syncthreads();
  block_scan(part, tid);
  int64_t pos = (int64_t)h * nnz_per_head + (part[tid] - local);
  for (int j = j0; j < j1; ++j) {
    csc_ptr[(int64_t)h * nb + j] = (int32_t)pos;
    const int len = col_length(sG, g, nb, w, j, bm + j * wpc, wpc);
    write_col(sG, g, nb, w, j, bm + j * wpc, wpc, csc_idx + pos);
    pos += len;
  }
  if (h == gridDim.x - 1 && tid == kBuildThreads - 1)
    csc_ptr[(int64_t)gridDim.x * nb] = (int32_t)((int64_t)gridDim.x * nnz_per_head);
}

// Larger layouts, phase 1: one thread per (head, query block); bitmap in global
// memory, zero on entry (cleared by phase 2 of the previous build).
__global__ __launch_bounds__(64) void layout_rows_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int r, int heads, uint64_t seed,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    uint32_t* __restrict__ rbits, int wpc) {
  extern __shared__ int32_t sG[];
  for (int x = threadIdx.x; x < g; x += 64) sG[x] = Gglob[x];
  __syncthreads();
  const int idx = blockIdx.x * 64 + threadIdx.x;
  if (idx >= heads * nb) return;
  const int h = idx / nb, i = idx - h * nb;
  build_row(sG, g, nb, w, r, seed, h, i, col_idx + row_ptr[idx], rbits + (int64_t)h * nb * wpc,
            wpc);
}

// Larger layouts, phase 2: one work-group per head; clears the bitmap.
__global__ __launch_bounds__(kBuildThreads) void layout_cols_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int64_t nnz_per_head,
    uint32_t* __restrict__ rbits, int wpc, int32_t* __restrict__ csc_ptr,
    int32_t* __restrict__ csc_idx) {
  __shared__ int part[kBuildThreads];
  extern __shared__ int32_t sG[];
  const int h = blockIdx.x, tid = threadIdx.x;
  for (int x = tid; x < g; x += kBuildThreads) sG[x] = Gglob[x];
  __syncthreads();
  uint32_t* hb = rbits + (int64_t)h * nb * wpc;
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int j0 = min(nb, tid * per), j1 = min(nb, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) local += col_length(sG, g, nb, w, j, hb + (int64_t)j * wpc, wpc);
  part[tid] = local;
  __syncthreads();
  block_scan(part, tid);
  int64_t pos = (int64_t)h * nnz_per_head + (part[tid] - local);
  for (int j = j0; j < j1; ++j) {
    csc_ptr[(int64_t)h * nb + j] = (int32_t)pos;
    const int len = col_length(sG, g, nb, w, j, hb + (int64_t)j * wpc, wpc);
    write_col(sG, g, nb, w, j, hb + (int64_t)j * wpc, wpc, csc_idx + pos);
    pos += len;
  }
  if (h == gridDim.x - 1 && tid == kBuildThreads - 1)
    csc_ptr[(int64_t)gridDim.x * nb] = (int32_t)((int64_t)gridDim.x * nnz_per_head);
}

}  // namespace

int launch_layout_rowptr(bsattn_layout* L, hipStream_t stream) {
  {
    ProfScope prof_("layout_rowptr", stream);
    hipLaunchKernelGGL(layout_rowptr_kernel, dim3(1), dim3(kBuildThreads), 0, stream, L->d_gblk,
                       L->g, L->nb, L->w, L->r, L->heads, L->nnz_per_head, L->d_row_ptr);
  }
  return check_hip(hipGetLastError(), "layout_rowptr launch");
}

int launch_layout_build(bsattn_layout* L, hipStream_t stream) {
  const int wpc = (L->nb + 31) / 32;
  if (L->nb <= kLdsBitmapNb) {
    const size_t lds = ((size_t)L->g + (size_t)L->nb * wpc) * sizeof(int32_t);
    {
      ProfScope prof_("layout_head", stream);
      hipLaunchKernelGGL(layout_head_kernel, dim3(L->heads), dim3(kBuildThreads), lds, stream,
                         L->d_gblk, L->g, L->nb, L->w, L->r, L->seed, L->nnz_per_head,
                         L->d_row_ptr, L->d_col_idx, L->d_csc_ptr, L->d_csc_idx);
    }
    return check_hip(hipGetLastError(), "layout_head launch");
  }
  {
    ProfScope prof_("layout_rows", stream);
    hipLaunchKernelGGL(layout_rows_kernel, dim3((L->heads * L->nb + 63) / 64), dim3(64),
                       (size_t)L->g * sizeof(int32_t), stream, L->d_gblk, L->g, L->nb, L->w,
                       L->r, L->heads, L->seed, L->d_row_ptr, L->d_col_idx, L->d_rbits, wpc);
  }
  int st = check_hip(hipGetLastError(), "layout_rows launch");
  if (st) return st;
  {
    ProfScope prof_("layout_cols", stream);
    hipLaunchKernelGGL(layout_cols_kernel, dim3(L->heads), dim3(kBuildThreads),
                       (size_t)L->g * sizeof(int32_t), stream, L->d_gblk, L->g, L->nb, L->w,
                       L->nnz_per_head, L->d_rbits, wpc, L->d_csc_ptr, L->d_csc_idx);
  }
  return check_hip(hipGetLastError(), "layout_cols launch");
}

}  // namespace bsattn
