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
//   layout_head   (n/b <= 512): one work-group per head.  Rows and columns are
//                 bitmaps in registers (row i = G | window | R_i; column j = G |
//                 window | rows that drew j), the lists are their set bits in
//                 ascending order, the column offsets a block scan.
//   layout_rows + layout_cols + layout_info (larger n/b): one thread per row
//                 (its list written by rank: the position of a block in the sorted
//                 union is the number of union members below it), the random picks
//                 in a global bitmap with a count per column; then a work-group per
//                 64 columns (each column's list read off its bitmap words in one
//                 pass); then the work records.  Bitmap and counts are cleared after
//                 use; global rows and columns are written by whole work-groups.

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

// The global block set, searched many times per row and column.  GReg keeps up to
// kRegG entries in registers (uniform, padded with INT_MAX), so every query is a
// few independent compares; GLds searches a sorted copy in LDS.
constexpr int kRegG = 8;

struct GReg {
  int v[kRegG];
  int g;
  __device__ int count_le(int x) const {
    int c = 0;
#pragma unroll
    for (int a = 0; a < kRegG; ++a) c += v[a] <= x;
    return c;
  }
  __device__ bool contains(int x) const {
    bool f = false;
#pragma unroll
    for (int a = 0; a < kRegG; ++a) f |= v[a] == x;
    return f;
  }
  template <typename F> __device__ void for_each(F f) const {
#pragma unroll
    for (int a = 0; a < kRegG; ++a)
      if (a < g) f(a, v[a]);
  }
};

struct GLds {
  const int32_t* p;
  int g;
  __device__ int count_le(int x) const {
    int lo = 0, hi = g;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (p[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
  }
  __device__ bool contains(int x) const {
    const int c = count_le(x);
    return c > 0 && p[c - 1] == x;
  }
  template <typename F> __device__ void for_each(F f) const {
    for (int a = 0; a < g; ++a) f(a, p[a]);
  }
};

template <typename GS>
struct RowCtx {
  GS G;
  int nb, lo, hi;   // window [lo, hi]
  // |E intersect [0, y]| with E = G U [lo, hi]
  __device__ int excl_le(int y) const {
    int cg = G.count_le(y);
    int cw = 0, cgw = 0;
    if (y >= lo) {
      int top = y < hi ? y : hi;
      cw = top - lo + 1;
      cgw = G.count_le(top) - G.count_le(lo - 1);
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
  // window members that are not global, below x
  __device__ int win_below(int x) const {
    if (x <= lo) return 0;
    const int top = x - 1 < hi ? x - 1 : hi;
    return (top - lo + 1) - (G.count_le(top) - G.count_le(lo - 1));
  }
};

template <typename GS>
__device__ RowCtx<GS> row_ctx(const GS& G, int nb, int w, int i) {
  const int half = (w - 1) / 2;
  return RowCtx<GS>{G, nb, i - half < 0 ? 0 : i - half, i + half > nb - 1 ? nb - 1 : i + half};
}

template <typename GS>
__device__ int row_length(const GS& G, int nb, int w, int r, int i) {
  if (G.contains(i)) return nb;
  const RowCtx<GS> c = row_ctx(G, nb, w, i);
  const int e = c.excl_size();
  const int m = nb - e;
  return e + (r < m ? r : m);
}

// Writes row i's sorted key blocks G U [lo, hi] U R (R sorted, disjoint from the
// rest) by rank.  cnt_r_below(x) = #{y in R : y < x}; rnd_at(t) = t-th of R.
template <typename GS, typename CountR, typename AtR>
__device__ void write_row(const RowCtx<GS>& c, int take, CountR cnt_r_below, AtR rnd_at,
                          int32_t* out) {
  c.G.for_each([&](int a, int x) { out[a + c.win_below(x) + cnt_r_below(x)] = x; });
  for (int x = c.lo; x <= c.hi; ++x) {
    if (c.G.contains(x)) continue;
    out[c.G.count_le(x - 1) + c.win_below(x) + cnt_r_below(x)] = x;
  }
  for (int t = 0; t < take; ++t) {
    const int x = rnd_at(t);
    out[c.G.count_le(x - 1) + c.win_below(x) + t] = x;
  }
}

// Random blocks of one row for r <= kFastR, kept in registers: a partial
// Fisher-Yates whose swaps are logged per step (position written, value); the
// value at a position is the latest logged write to it, else the untouched
// candidate.  Positions below the current step are never read again.
template <typename GS>
__device__ void draw_fast(const RowCtx<GS>& c, int m, int take, uint64_t seed, uint64_t k0,
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
template <typename GS>
__device__ void draw_any(const RowCtx<GS>& c, int m, int take, uint64_t seed, uint64_t k0,
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
template <typename GS>
__device__ void build_row(const GS& G, int nb, int w, int r, uint64_t seed, int h, int i,
                          int32_t* out, uint32_t* hb, int wpc, int32_t* hcnt) {
  if (G.contains(i)) return;   // a global row lists every block: written by layout_cols
  const RowCtx<GS> c = row_ctx(G, nb, w, i);
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
      if (t < take) {
        atomicOr(&hb[(int64_t)rnd[t] * wpc + (i >> 5)], 1u << (i & 31));
        atomicAdd(&hcnt[rnd[t]], 1);
      }
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
    for (int t = 0; t < take; ++t) {
      atomicOr(&hb[(int64_t)rnd[t] * wpc + (i >> 5)], 1u << (i & 31));
      atomicAdd(&hcnt[rnd[t]], 1);
    }
  }
}

// The list of a non-global column j (global columns list every block and are
// written by the whole work-group): the set bits, in ascending order, of the union
// of the global blocks (gbits), the window of j and the rows that drew j (bits),
// three disjoint sets.  One pass over the column's words, which it also clears for
// the next draw.
__device__ __forceinline__ void write_col(const uint32_t* gbits, int nb, int w, int j,
                                          uint32_t* bits, int wpc, int32_t* out) {
  const int half = (w - 1) / 2;
  const int lo = max(0, j - half), hi = min(nb - 1, j + half);
  int q = 0;
  // the words are read eight at a time (clamped reads, all in flight together); a
  // column holds a few picks, so only the words that had one are cleared
  for (int y0 = 0; y0 < wpc; y0 += 8) {
    uint32_t pw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pw[u] = bits[min(y0 + u, wpc - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int y = y0 + u;
      if (y >= wpc) break;
      if (pw[u]) bits[y] = 0u;
      const int a = max(lo - 32 * y, 0), b = min(hi - 32 * y, 31);
      const uint32_t win = a > b ? 0u : (b == 31 ? ~0u : (2u << b) - 1u) & ~((1u << a) - 1u);
      uint32_t word = pw[u] | gbits[y] | win;
      while (word) {
        out[q++] = 32 * y + __builtin_ctz(word);
        word &= word - 1u;
      }
    }
  }
}

// exclusive scan of v within each wave (no work-group barrier): for values that
// only the first wave holds
__device__ __forceinline__ int wave_exclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x - v;
}

// exclusive scan of v over the work-group (any multiple of 64 threads); `part` holds
// one int per wave.  Returns the exclusive prefix.
__device__ int block_exclusive_scan(int v, int* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < wave; ++q) base += part[q];
  __syncthreads();
  return base + x - v;
}

// sum of v over the work-group (any multiple of 64 threads); `part` one int per wave
__device__ int block_sum(int v, int* part) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
  for (int q = 0; q < (int)(blockDim.x >> 6); ++q) t += part[q];
  __syncthreads();
  return t;
}

template <typename GS>
__device__ GS load_gset(const int32_t* Gglob, int g, int32_t* lds);

template <>
__device__ GReg load_gset<GReg>(const int32_t* Gglob, int g, int32_t*) {
  GReg G;
  G.g = g;
#pragma unroll
  for (int a = 0; a < kRegG; ++a) G.v[a] = a < g ? Gglob[a] : 0x7fffffff;
  return G;
}

template <>
__device__ GLds load_gset<GLds>(const int32_t* Gglob, int g, int32_t* lds) {
  for (int x = threadIdx.x; x < g; x += blockDim.x) lds[x] = Gglob[x];
  __syncthreads();
  return GLds{lds, g};
}

__global__ __launch_bounds__(kBuildThreads) void layout_rowptr_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int r, int heads,
    int64_t nnz_per_head, int32_t* __restrict__ row_ptr) {
  extern __shared__ int32_t sG[];
  __shared__ int part[kBuildThreads / 64];
  const GLds G = load_gset<GLds>(Gglob, g, sG);
  const int tid = threadIdx.x;
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += row_length(G, nb, w, r, i);
  int pos = block_exclusive_scan(local, part);
  for (int i = i0; i < i1; ++i) {
    for (int h = 0; h < heads; ++h) row_ptr[(int64_t)h * nb + i] = (int32_t)(h * nnz_per_head + pos);
    pos += row_length(G, nb, w, r, i);
  }
  if (tid == 0) row_ptr[(int64_t)heads * nb] = (int32_t)(heads * nnz_per_head);
}

// ---------------------------------------------------------------------------
// One work-group per head for n/b <= 512.  Every row and column of the head is a
// bitmap of W 64-bit words in registers: row i is G | window(i) | R_i, column j is
// G | window(j) | {i : j in R_i} (all rows when j is global), and the sorted
// lists come out of a lowest-set-bit walk.  The i-th entry of the ascending
// candidate list is the i-th set bit of the row's free-block bitmap.
// ---------------------------------------------------------------------------

// bits lo..hi of the whole bitmap (inclusive; may be empty or reach past either
// end) that fall in word k
__device__ __forceinline__ uint64_t span_bits(int k, int lo, int hi) {
  const int a = max(lo - 64 * k, 0), b = min(hi - 64 * k, 63);
  if (a > b) return 0ull;
  const uint64_t upto = b == 63 ? ~0ull : (2ull << b) - 1ull;
  return upto & ~((1ull << a) - 1ull);
}

template <int W>
__device__ __forceinline__ bool bit_of(const uint64_t (&b)[W], int x) {
  uint64_t v = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) v = (x >> 6) == k ? b[k] : v;
  return (v >> (x & 63)) & 1ull;
}

// every word is updated (with a zero mask where x is not), so the array stays in
// registers: a store under a data-dependent condition sends it to per-lane memory
template <int W>
__device__ __forceinline__ void set_bit(uint64_t (&b)[W], int x) {
  const uint64_t m = 1ull << (x & 63);
#pragma unroll
  for (int k = 0; k < W; ++k) b[k] |= (x >> 6) == k ? m : 0ull;
}

// position of the x-th (0-based) set bit; x < popcount(f)
template <int W>
__device__ __forceinline__ int select_bit(const uint64_t (&f)[W], int x) {
  uint64_t word = 0;
  int base = 0;
  bool found = false;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const int c = __popcll(f[k]);
    const bool here = !found && x < c;
    word = here ? f[k] : word;
    base = here ? 64 * k : base;
    x = (found || here) ? x : x - c;
    found = found || here;
  }
  int pos = 0;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int c = __popcll(word & ((1ull << s) - 1ull));
    if (x >= c) {
      x -= c;
      word >>= s;
      pos += s;
    }
  }
  return base + pos;
}

// u mod d for 1 <= d < 2^15 with 32-bit remainders only:
// u = hi 2^32 + lo, so u mod d = ((hi mod d)(2^32 mod d) + lo mod d) mod d
__device__ __forceinline__ uint32_t mod_small(uint64_t u, uint32_t d) {
  const uint32_t hi = (uint32_t)(u >> 32), lo = (uint32_t)u;
  const uint32_t p32 = (0u - d) % d;   // (2^32 - d) mod d = 2^32 mod d
  return ((hi % d) * p32 + lo % d) % d;
}

// lowest set bit (the bitmap is not empty)
template <int W>
__device__ __forceinline__ int first_bit(const uint64_t (&b)[W]) {
  int pos = -1;
#pragma unroll
  for (int k = W - 1; k >= 0; --k)
    if (b[k]) pos = 64 * k + __builtin_ctzll(b[k]);
  return pos;
}

// number of set bits below position x
template <int W>
__device__ __forceinline__ int bits_below(const uint64_t (&b)[W], int x) {
  int c = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) c += __popcll(b[k] & span_bits(k, 0, x - 1));
  return c;
}

template <int W>
__device__ __forceinline__ int write_bits(const uint64_t (&b)[W], int32_t* out) {
  int q = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    uint64_t x = b[k];
    while (x) {
      out[q++] = 64 * k + __builtin_ctzll(x);
      x &= x - 1ull;
    }
  }
  return q;
}

// RMAX bounds r: the swap log of the partial Fisher-Yates lives in registers for
// RMAX <= 8 (fully unrolled), in per-thread memory otherwise.
template <int W, int RMAX>
__global__ __launch_bounds__(kBuildThreads) void layout_head_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int r, uint64_t seed,
    int64_t nnz_per_head, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ csc_ptr, int32_t* __restrict__ csc_idx, int32_t* __restrict__ kv_order,
    int32_t* __restrict__ row_info, int32_t* __restrict__ col_info) {
  // dynamic LDS: random picks per key block (nb x wpc words, bit i = query block
  // i), the global list G[g], every column's offset within the head, every
  // column's length, columns by length, first rank per length, every column's
  // first query block, columns per length, list offsets of the global rows
  extern __shared__ __attribute__((aligned(16))) int32_t dyn[];
  __shared__ uint32_t sGb[2 * W];
  __shared__ int part[kBuildThreads / 64];
  const int h = blockIdx.x, tid = threadIdx.x;
  // the first row's list offset is loaded before anything else, so that its
  // latency overlaps that of the global list
  const int rp0 = tid < nb ? row_ptr[(int64_t)h * nb + tid] : 0;
  const int wpc = (nb + 31) / 32;
  uint32_t* colmap = reinterpret_cast<uint32_t*>(dyn);
  int32_t* sG = dyn + nb * wpc;
  int32_t* sColPos = sG + g;
  int32_t* sColLen = sColPos + nb;                 // column lengths
  uint32_t* sBk = reinterpret_cast<uint32_t*>(sColLen + nb);   // [nb + 1][wpc] columns by length
  int32_t* sBase = reinterpret_cast<int32_t*>(sBk + (nb + 1) * wpc);   // [nb + 1] first rank
  int32_t* sColFirst = sBase + nb + 1;                 // [nb] first query block
  int32_t* sLenCnt = sColFirst + nb;                   // [nb + 1] columns per length
  int32_t* sGrp = sLenCnt + nb + 1;                    // [g] global rows' list offsets
  for (int x = tid; x < nb * wpc; x += kBuildThreads) colmap[x] = 0u;
  for (int x = tid; x < (nb + 1) * wpc; x += kBuildThreads) sBk[x] = 0u;
  for (int x = tid; x <= nb; x += kBuildThreads) sLenCnt[x] = 0;
  for (int x = tid; x < g; x += kBuildThreads) sG[x] = Gglob[x];
  if (tid < 2 * W) sGb[tid] = 0u;
  __syncthreads();
  for (int x = tid; x < g; x += kBuildThreads) atomicOr(&sGb[sG[x] >> 5], 1u << (sG[x] & 31));
  __syncthreads();
  uint64_t gb[W], valid[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    gb[k] = sGb[2 * k] | ((uint64_t)sGb[2 * k + 1] << 32);
    valid[k] = span_bits(k, 0, nb - 1);
  }
  const int half = (w - 1) / 2;

  // rows (global rows are written by the whole group at the end)
  for (int i = tid; i < nb; i += kBuildThreads) {
    const int rp = i == tid ? rp0 : row_ptr[(int64_t)h * nb + i];
    if (bit_of(gb, i)) {
      sGrp[bits_below(gb, i)] = rp;
      continue;
    }
    uint64_t row[W], freeb[W];
    int m = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      row[k] = (gb[k] | span_bits(k, i - half, i + half)) & valid[k];
      freeb[k] = valid[k] & ~row[k];
      m += __popcll(freeb[k]);
    }
    const int take = r < m ? r : m;
    const uint64_t k0 = (uint64_t)((int64_t)h * nb + i) * (uint64_t)r + 1;
    int key[RMAX], val[RMAX];
    constexpr int kUnroll = RMAX <= kFastR ? RMAX : 1;
#pragma unroll kUnroll
    for (int t = 0; t < RMAX; ++t) {
      if (t < take) {
        const uint64_t u = splitmix64_draw(seed, k0 + t);
        const int s = t + (int)mod_small(u, (uint32_t)(m - t));
        // the log holds candidate positions, not blocks: only the pick itself is
        // turned into a block (one bit select per draw)
        int pt = t, ps = s;
#pragma unroll kUnroll
        for (int q = 0; q < t; ++q) {
          if (key[q] == t) pt = val[q];
          if (key[q] == s) ps = val[q];
        }
        key[t] = s != t ? s : -1;
        val[t] = pt;
        const int vs = select_bit(freeb, ps);
        set_bit(row, vs);
        atomicOr(&colmap[vs * wpc + (i >> 5)], 1u << (i & 31));
      }
    }
    const int len = write_bits(row, col_idx + rp);
    // the row's work-item record, at its rank among the non-global rows
    int32_t* rec = row_info + 4 * ((int64_t)h * (nb - g) + i - bits_below(gb, i));
    rec[0] = i; rec[1] = rp; rec[2] = len; rec[3] = first_bit(row);
  }
  __syncthreads();

  // columns: lengths, offsets (block scan), lists
  auto col_bits = [&](int j, uint64_t (&c)[W]) {
    const bool global = bit_of(gb, j);
    int len = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const uint32_t lo = 2 * k < wpc ? colmap[j * wpc + 2 * k] : 0u;
      const uint32_t hi = 2 * k + 1 < wpc ? colmap[j * wpc + 2 * k + 1] : 0u;
      const uint64_t picked = lo | ((uint64_t)hi << 32);
      c[k] = global ? valid[k] : (gb[k] | span_bits(k, j - half, j + half) | picked) & valid[k];
      len += __popcll(c[k]);
    }
    return len;
  };
  const int per = (nb + kBuildThreads - 1) / kBuildThreads;
  const int j0 = min(nb, tid * per), j1 = min(nb, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) {
    uint64_t c[W];
    local += col_bits(j, c);
  }
  // up to 64 blocks every column sits in the first wave: no work-group scan
  int pos = nb <= 64 ? wave_exclusive_scan(local) : block_exclusive_scan(local, part);
  for (int j = j0; j < j1; ++j) {
    uint64_t c[W];
    const int len = col_bits(j, c);
    const int64_t p = (int64_t)h * nnz_per_head + pos;
    csc_ptr[(int64_t)h * nb + j] = (int32_t)p;
    sColPos[j] = pos;
    sColLen[j] = len;
    sColFirst[j] = first_bit(c);
    if (!bit_of(gb, j)) {
      atomicOr(&sBk[len * wpc + (j >> 5)], 1u << (j & 31));
      atomicAdd(&sLenCnt[len], 1);
      write_bits(c, csc_idx + p);
    }
    pos += len;
  }
  if (h == (int)gridDim.x - 1 && tid == kBuildThreads - 1)
    csc_ptr[(int64_t)gridDim.x * nb] = (int32_t)((int64_t)gridDim.x * nnz_per_head);
  __syncthreads();

  // work order of the non-global key blocks for dK/dV: longest column first, ties
  // by block index.  sBk[L] holds the columns of length L as a bitmap; the rank of
  // column j is the count of longer columns plus the columns of its length before
  // it.
  {
    // the first rank of each length is an exclusive scan of the column counts
    // over descending lengths (up to 63 blocks all lengths sit in the first wave)
    const int bper = (nb + 1 + kBuildThreads - 1) / kBuildThreads;
    const int d0 = min(nb + 1, tid * bper), d1 = min(nb + 1, d0 + bper);   // L = nb - d
    int cnt = 0;
    for (int d = d0; d < d1; ++d) cnt += sLenCnt[nb - d];
    int base = nb < 64 ? wave_exclusive_scan(cnt) : block_exclusive_scan(cnt, part);
    for (int d = d0; d < d1; ++d) {
      sBase[nb - d] = base;
      base += sLenCnt[nb - d];
    }
  }
  __syncthreads();
  for (int j = tid; j < nb; j += kBuildThreads) {
    if (bit_of(gb, j)) continue;
    const uint32_t* bk = sBk + sColLen[j] * wpc;
    int rank = sBase[sColLen[j]];
    for (int x = 0; x < (j >> 5); ++x) rank += __popc(bk[x]);
    rank += __popc(bk[j >> 5] & ((1u << (j & 31)) - 1u));
    kv_order[(int64_t)h * (nb - g) + rank] = j;
    int32_t* rec = col_info + 4 * ((int64_t)h * (nb - g) + rank);
    rec[0] = j; rec[1] = (int32_t)((int64_t)h * nnz_per_head + sColPos[j]);
    rec[2] = sColLen[j]; rec[3] = sColFirst[j];
  }

  // global rows and columns hold every block
  for (int e = tid; e < g * nb; e += kBuildThreads) {
    const int a = e / nb, j = e - a * nb;
    col_idx[sGrp[a] + j] = j;
    csc_idx[(int64_t)h * nnz_per_head + sColPos[sG[a]] + j] = j;
  }
}

// Larger layouts, phase 1: one thread per (head, query block); bitmap in global
// memory, zero on entry (cleared by phase 2 of the previous build).
template <typename GS>
__global__ __launch_bounds__(64) void layout_rows_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int r, int heads, uint64_t seed,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    uint32_t* __restrict__ rbits, int32_t* __restrict__ counts, int wpc) {
  extern __shared__ int32_t sG[];
  const GS G = load_gset<GS>(Gglob, g, sG);
  const int idx = blockIdx.x * 64 + threadIdx.x;
  if (idx >= heads * nb) return;
  const int h = idx / nb, i = idx - h * nb;
  build_row(G, nb, w, r, seed, h, i, col_idx + row_ptr[idx], rbits + (int64_t)h * nb * wpc, wpc,
            counts + (int64_t)h * nb);
}

// Larger layouts, phase 2: a work-group per kColThreads columns of a head (a column
// per thread).  A column's length is g (or every block for a global column), its
// non-global window rows and the rows that drew it (counted by phase 1), so each
// work-group finds its offset by summing the lengths of the head's earlier columns.
// Writes the column lists (clearing the pick bitmap), then with all threads the
// global columns it owns and its slice of every global row.
constexpr int kColThreads = 64;

template <typename GS>
__global__ __launch_bounds__(kColThreads) void layout_cols_kernel(
    const int32_t* __restrict__ Gglob, int g, int nb, int w, int64_t nnz_per_head,
    uint32_t* __restrict__ rbits, const int32_t* __restrict__ counts, int wpc,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    int32_t* __restrict__ csc_ptr, int32_t* __restrict__ csc_idx) {
  // dynamic LDS: [g] global blocks (GLds), then [wpc] the global blocks as a bitmap
  extern __shared__ int32_t sG[];
  uint32_t* sGbits = reinterpret_cast<uint32_t*>(sG + g);
  __shared__ int part[kColThreads / 64];
  __shared__ int sPos[kColThreads];
  const int chunks = (nb + kColThreads - 1) / kColThreads;
  const int h = blockIdx.x / chunks, c = blockIdx.x - h * chunks, tid = threadIdx.x;
  for (int y = tid; y < wpc; y += kColThreads) sGbits[y] = 0u;
  const GS G = load_gset<GS>(Gglob, g, sG);   // (GLds: ends with a barrier)
  __syncthreads();
  for (int a = tid; a < g; a += kColThreads) atomicOr(&sGbits[Gglob[a] >> 5], 1u << (Gglob[a] & 31));
  __syncthreads();
  const int32_t* hcnt = counts + (int64_t)h * nb;
  auto is_global = [&](int j) { return (sGbits[j >> 5] >> (j & 31)) & 1u; };
  auto len_of = [&](int j, int picks) {
    if (is_global(j)) return nb;
    const RowCtx<GS> rc = row_ctx(G, nb, w, j);
    return G.g + rc.win_below(rc.hi + 1) + picks;
  };
  // lengths of the columns of the earlier chunks: their pick counts are read 16
  // chunks at a time (clamped reads, all in flight together), not one round trip
  // per chunk
  int before = 0;
  for (int k0 = 0; k0 < c; k0 += 16) {
    int pk[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) pk[u] = hcnt[min(k0 + u, c - 1) * kColThreads + tid];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (k0 + u < c) before += len_of((k0 + u) * kColThreads + tid, pk[u]);
  }
  const int base = block_sum(before, part);
  const int j = c * kColThreads + tid;
  const int len = j < nb ? len_of(j, hcnt[j]) : 0;
  const int pos = base + block_exclusive_scan(len, part);   // offset within the head
  const int64_t head0 = (int64_t)h * nnz_per_head;
  sPos[tid] = pos;
  if (j < nb) {
    csc_ptr[(int64_t)h * nb + j] = (int32_t)(head0 + pos);
    if (!is_global(j))
      write_col(sGbits, nb, w, j, rbits + ((int64_t)h * nb + j) * wpc, wpc, csc_idx + head0 + pos);
  }
  if (h == (int)gridDim.x / chunks - 1 && c == chunks - 1 && tid == 0)
    csc_ptr[(int64_t)(h + 1) * nb] = (int32_t)((int64_t)(h + 1) * nnz_per_head);
  __syncthreads();
  // the global columns of this chunk, then this chunk's slice of every global row
  for (int x = 0; x < kColThreads && c * kColThreads + x < nb; ++x)
    if (is_global(c * kColThreads + x))
      for (int e = tid; e < nb; e += kColThreads) csc_idx[head0 + sPos[x] + e] = e;
  if (j < nb)
    for (int a = 0; a < g; ++a) col_idx[row_ptr[(int64_t)h * nb + Gglob[a]] + j] = j;
}

}  // namespace

int launch_layout_rowptr(bsattn_layout* L, hipStream_t stream) {
  {
    ProfScope prof_("layout_rowptr", stream);
    hipLaunchKernelGGL(layout_rowptr_kernel, dim3(1), dim3(kBuildThreads),
                       (size_t)L->g * sizeof(int32_t), stream, L->d_gblk, L->g, L->nb, L->w,
                       L->r, L->heads, L->nnz_per_head, L->d_row_ptr);
  }
  return check_hip(hipGetLastError(), "layout_rowptr launch");
}

// Larger layouts, phase 3: the work-item records of the non-global rows (in block
// order) and columns (in dK/dV order), one thread per (head, rank); clears the
// per-column pick counts for the next draw (one thread per (head, block)).
__global__ __launch_bounds__(64) void layout_info_kernel(
    const int32_t* __restrict__ ngblk, const int32_t* __restrict__ kv_order, int nb, int g,
    int heads, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ csc_ptr, const int32_t* __restrict__ csc_idx,
    int32_t* __restrict__ row_info, int32_t* __restrict__ col_info,
    int32_t* __restrict__ counts) {
  const int ng = nb - g;
  const int idx = blockIdx.x * 64 + threadIdx.x;
  if (idx < heads * nb) counts[idx] = 0;
  if (idx >= heads * ng) return;
  const int h = idx / ng, r = idx - h * ng;
  const int i = ngblk[r];
  const int rp = row_ptr[(int64_t)h * nb + i];
  int32_t* rec = row_info + 4 * (int64_t)idx;
  rec[0] = i; rec[1] = rp; rec[2] = row_ptr[(int64_t)h * nb + i + 1] - rp; rec[3] = col_idx[rp];
  const int j = kv_order[idx];
  const int cp = csc_ptr[(int64_t)h * nb + j];
  rec = col_info + 4 * (int64_t)idx;
  rec[0] = j; rec[1] = cp; rec[2] = csc_ptr[(int64_t)h * nb + j + 1] - cp; rec[3] = csc_idx[cp];
}

namespace {
// Dynamic LDS of layout_head_kernel: random picks, global list, column offsets,
// lengths and first query blocks, columns by length, first rank per length,
// columns per length, global rows' list offsets.
size_t head_lds_bytes(const bsattn_layout* L) {
  const int wpc = (L->nb + 31) / 32;
  return ((size_t)L->nb * wpc + L->g + 3 * L->nb + (size_t)(L->nb + 1) * (wpc + 2) + L->g) *
         sizeof(int32_t);
}

template <int W, int RMAX>
int launch_head(bsattn_layout* L, hipStream_t stream) {
  const size_t lds = head_lds_bytes(L);
  {
    ProfScope prof_("layout_head", stream);
    hipLaunchKernelGGL((layout_head_kernel<W, RMAX>), dim3(L->heads), dim3(kBuildThreads), lds,
                       stream, L->d_gblk, L->g, L->nb, L->w, L->r, L->seed, L->nnz_per_head,
                       L->d_row_ptr, L->d_col_idx, L->d_csc_ptr, L->d_csc_idx, L->d_kv_order,
                       L->d_row_info, L->d_col_info);
  }
  return check_hip(hipGetLastError(), "layout_head launch");
}

template <int RMAX>
int launch_head_r(bsattn_layout* L, hipStream_t stream) {
  if (L->nb <= 64) return launch_head<1, RMAX>(L, stream);
  if (L->nb <= 128) return launch_head<2, RMAX>(L, stream);
  if (L->nb <= 256) return launch_head<4, RMAX>(L, stream);
  return launch_head<8, RMAX>(L, stream);
}

template <typename GS>
int launch_rows_cols(bsattn_layout* L, hipStream_t stream) {
  const int wpc = (L->nb + 31) / 32;
  const size_t g_lds = (size_t)L->g * sizeof(int32_t);
  // per-column pick counts after the pick bitmap (zero between builds, like it)
  int32_t* counts = reinterpret_cast<int32_t*>(L->d_rbits + (size_t)L->heads * L->nb * wpc);
  const int chunks = (L->nb + kColThreads - 1) / kColThreads;
  {
    ProfScope prof_("layout_rows", stream);
    hipLaunchKernelGGL(layout_rows_kernel<GS>, dim3((L->heads * L->nb + 63) / 64), dim3(64),
                       g_lds, stream, L->d_gblk, L->g, L->nb, L->w, L->r, L->heads, L->seed,
                       L->d_row_ptr, L->d_col_idx, L->d_rbits, counts, wpc);
  }
  int st = check_hip(hipGetLastError(), "layout_rows launch");
  if (st) return st;
  {
    ProfScope prof_("layout_cols", stream);
    hipLaunchKernelGGL(layout_cols_kernel<GS>, dim3(L->heads * chunks), dim3(kColThreads),
                       g_lds + (size_t)wpc * sizeof(uint32_t), stream, L->d_gblk, L->g, L->nb,
                       L->w, L->nnz_per_head, L->d_rbits, counts, wpc, L->d_row_ptr,
                       L->d_col_idx, L->d_csc_ptr, L->d_csc_idx);
  }
  st = check_hip(hipGetLastError(), "layout_cols launch");
  const int ng = L->nb - L->g;
  if (st || ng == 0) return st;
  {
    ProfScope prof_("layout_info", stream);
    hipLaunchKernelGGL(layout_info_kernel, dim3((L->heads * L->nb + 63) / 64), dim3(64), 0,
                       stream, L->d_ngblk, L->d_kv_order, L->nb, L->g, L->heads, L->d_row_ptr,
                       L->d_col_idx, L->d_csc_ptr, L->d_csc_idx, L->d_row_info, L->d_col_info,
                       counts);
  }
  return check_hip(hipGetLastError(), "layout_info launch");
}
}  // namespace

int launch_layout_build(bsattn_layout* L, hipStream_t stream) {
  if (L->nb <= kLdsBitmapNb && head_lds_bytes(L) <= (size_t)L->max_lds)
    return L->r <= kFastR ? launch_head_r<kFastR>(L, stream) : launch_head_r<kMaxR>(L, stream);
  return L->g <= kRegG ? launch_rows_cols<GReg>(L, stream) : launch_rows_cols<GLds>(L, stream);
}

}  // namespace bsattn
