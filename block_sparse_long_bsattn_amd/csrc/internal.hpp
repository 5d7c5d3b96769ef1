// Host-side internals shared by the translation units of libbsattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/bsattn.h"

struct bsattn_layout {
  int n = 0, b = 0, nb = 0, heads = 0, g = 0, w = 0, r = 0;
  uint64_t seed = 0;
  int device = 0;
  int64_t nnz_per_head = 0;      // same for every head (row lengths do not depend on h)
  std::vector<int32_t> gblk;     // global blocks (host copy)
  std::vector<int32_t> ngblk;    // non-global blocks ascending (host copy)
  std::vector<int32_t> row_len;  // length of each query-block row (host copy)
  int cus = 256;                 // compute units of the device (sizes the segment plan)
  int max_lds = 65536;           // LDS bytes one work-group may use on the device
  // device arrays (owned)
  int32_t* d_gblk = nullptr;     // [g]
  int32_t* d_ngblk = nullptr;    // [nb - g] non-global block ids, ascending
  int32_t* d_row_ptr = nullptr;  // [heads*nb + 1]
  int32_t* d_col_idx = nullptr;  // [heads*nnz_per_head]
  int32_t* d_csc_ptr = nullptr;  // [heads*nb + 1]
  int32_t* d_csc_idx = nullptr;  // [heads*nnz_per_head]
  uint32_t* d_rbits = nullptr;   // [heads][nb][ceil(nb/32)] random picks, then [heads][nb]
                                 // picks per column; zero between builds
  int32_t* d_kv_order = nullptr; // [heads][nb - g] non-global key blocks, longest column
                                 // first (the dK/dV work order; ascending until a build
                                 // kernel that sorts has run)
  // Work-item records {block, list start, list length, first listed block}, four
  // int32 each: [heads][nb - g] non-global rows in block order, and non-global
  // columns in d_kv_order's order.
  int32_t* d_row_info = nullptr;
  int32_t* d_col_info = nullptr;
  std::vector<int32_t> kv_order_init;
  hipEvent_t built = nullptr;     // recorded after the last build or redraw
};

// How one call cuts the full-length (global) rows and columns into work items:
// segments of `seg` blocks, `nseg` per global block (split = 0: one whole item).
struct SegPlan {
  int seg, nseg, split;
};
SegPlan seg_plan(const bsattn_layout* L, int batch);

// A 64-token tile of one residue class of one head's window pattern: with stride
// s (dilation + 1), class c holds tokens c, c + s, c + 2s, ... (nc of them); row x
// of tile t is class index 64*t + x, i.e. token c + s*(64*t + x), valid iff that
// index is below nc.  Stride 1 gives the natural tiles (c = 0, nc = n).
struct LfTileRef {
  int32_t h;        // head within the plan's head period
  int16_t c, s;     // residue class, stride
  int32_t t, nc;    // tile within the class, class length
};

struct lfattn_plan {
  int n = 0, w1 = 0, ng = 0, nt = 0, ngt = 0;  // tokens, window per side, globals,
                                               // 64-token tiles (the last may be partial)
  int heads = 0;                 // 0: any head count, one pattern; else the plan's heads
  int causal = 0;                // window of earlier tokens only
  int wb = 0, woff = 0, whalf = 0;   // blocked window: block size (0: sliding window),
                                     // first ordinary token, (w - 1) / 2
  int device = 0;
  int cus = 256;                 // compute units of the device (sizes the row segments)
  int nct = 0;                   // class tiles per head period (all heads, or one)
  int nct_plain = 0;             // ... of them holding no global key (listed first)
  int32_t* d_gtok = nullptr;     // [ng] global positions ascending
  int32_t* d_gidx = nullptr;     // [n] index into d_gtok, or -1 for non-global tokens
  uint64_t* d_tile_gmask = nullptr;  // [nt] bit x set iff token 64*t + x is global
  LfTileRef* d_ct = nullptr;     // [nct] class tiles, those without global keys first
  std::vector<int32_t> gtok;     // host copies backing the build-time uploads
  std::vector<int32_t> gidx;
  std::vector<uint64_t> tile_gmask;
  std::vector<int32_t> dil;      // dilation per head ([heads], or one value)
  std::vector<LfTileRef> ct;
  hipEvent_t built = nullptr;    // recorded after the build-time uploads
};

namespace bsattn {

// Brackets one kernel launch with hipEvents while profiling is enabled.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

// BSATTN_DEBUG, read once from the environment: 0 (unset) silent; 1 logs every
// compute call, kernel launch and error to stderr; 2 also synchronises the stream
// after each compute call (unless it is being captured into a graph) and reports a
// failed kernel, or a write past the workspace bytes the call needs (a canary
// placed after them when the caller's workspace has 64 spare bytes), as BSATTN_EHIP
// at the call that caused it.
int debug_level();

// The level-1 log and level-2 checks of one compute call, around its launches.
class DebugCall {
 public:
  DebugCall(const char* who, hipStream_t stream, void* ws, size_t ws_bytes, size_t need);
  int finish(int st);   // st, or the failure the level-2 checks found

 private:
  const char* who_;
  hipStream_t stream_;
  void* ws_;
  size_t need_;
  bool canary_ = false;
};

int set_error(int status, const std::string& msg);
void clear_error();
int check_hip(hipError_t e, const char* what);

// Launch helpers implemented in the kernel translation units.
int launch_layout_rowptr(bsattn_layout* L, hipStream_t stream);
int launch_layout_build(bsattn_layout* L, hipStream_t stream);
// o_lo (forward: written, backward: read) is the bf16 rounding residual of O, or
// null.  d: head dimension, 64 (any dtype) or 128 (bf16).
int launch_fwd(const bsattn_layout* L, int batch, bsattn_dtype dt, int d, float scale,
               const void* q, const void* k, const void* v, void* o, float* lse,
               void* o_lo, void* ws, hipStream_t stream);
int launch_bwd(const bsattn_layout* L, int batch, int d, float scale, const void* q,
               const void* k, const void* v, const void* o, const void* o_lo,
               const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
               hipStream_t stream);
// qg, kg, vg (and dqg, dkg, dvg) may be null: one projection set for every row.
int launch_lf_fwd(const lfattn_plan* P, int batch, int heads, int d, float scale, const void* q,
                  const void* k, const void* v, const void* qg, const void* kg,
                  const void* vg, void* o, float* lse, void* o_lo, void* ws,
                  hipStream_t stream);

size_t fwd_workspace_bytes(const bsattn_layout* L, int batch, int d);   // either dtype
size_t fwd_workspace_bytes_dt(const bsattn_layout* L, int batch, bsattn_dtype dt, int d);
size_t bwd_workspace_bytes(const bsattn_layout* L, int batch, int d);
size_t lf_workspace_bytes(const lfattn_plan* P, int batch, int heads, int d);
int launch_lf_bwd(const lfattn_plan* P, int batch, int heads, int d, float scale, const void* q,
                  const void* k, const void* v, const void* qg, const void* kg,
                  const void* vg, const void* o, const void* o_lo, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, void* dqg, void* dkg,
                  void* dvg, void* ws, hipStream_t stream);
size_t lf_bwd_workspace_bytes(const lfattn_plan* P, int batch, int heads, int d);

// The static device scratch of bsattn_bwd_noalloc: its address on the current
// device (looked up once per device) and its size.
int noalloc_scratch(void** out);
size_t noalloc_scratch_bytes();

}  // namespace bsattn
