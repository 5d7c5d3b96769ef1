// C ABI of libbsattn.so: argument checking, handle management and error reporting.
// Every compute call is checked completely on the host before anything is
// enqueued; the kernels assume the shapes checked here.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"
#include "shape.hpp"

namespace bsattn {

namespace {
thread_local std::string g_last_error;
constexpr int kMaxNb = 4096;
constexpr int kMaxR = 64;
constexpr int kMaxLfTokens = 262144;
constexpr int kMaxLfDilation = 1023;   // stride and class fit the int16 fields of LfTileRef
constexpr int kMaxLfHeads = 4096;
}  // namespace

namespace {
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
}  // namespace

int debug_level() {
  static const int level = [] {
    const char* s = std::getenv("BSATTN_DEBUG");
    return s != nullptr ? std::atoi(s) : 0;
  }();
  return level;
}

ProfScope::ProfScope(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (debug_level() >= 1) std::fprintf(stderr, "[bsattn] launch %s stream=%p\n", name, (void*)stream);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  if (hipEventCreate(&start_) != hipSuccess) { start_ = nullptr; return; }
  if (hipEventRecord(start_, stream_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (start_ == nullptr) return;
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) != hipSuccess || hipEventRecord(stop, stream_) != hipSuccess) {
    if (stop) (void)hipEventDestroy(stop);
    (void)hipEventDestroy(start_);
    return;
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({name_, start_, stop});
}

int set_error(int status, const std::string& msg) {
  g_last_error = msg;
  if (debug_level() >= 1) std::fprintf(stderr, "[bsattn] error %d: %s\n", status, msg.c_str());
  return status;
}

namespace {
constexpr size_t kCanaryBytes = 64;
constexpr unsigned char kCanary = 0xA5;
}  // namespace

DebugCall::DebugCall(const char* who, hipStream_t stream, void* ws, size_t ws_bytes,
                     size_t need)
    : who_(who), stream_(stream), ws_(ws), need_(need) {
  const int level = debug_level();
  if (level < 1) return;
  std::fprintf(stderr, "[bsattn] call %s stream=%p workspace=%zu of %zu bytes needed\n", who,
               (void*)stream, ws_bytes, need);
  if (level < 2 || ws == nullptr || ws_bytes < need + kCanaryBytes) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  static const std::vector<unsigned char> pattern(kCanaryBytes, kCanary);
  canary_ = hipMemcpyAsync(static_cast<char*>(ws) + need, pattern.data(), kCanaryBytes,
                           hipMemcpyHostToDevice, stream) == hipSuccess;
}

int DebugCall::finish(int st) {
  if (st != BSATTN_OK || debug_level() < 2) return st;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream_, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return st;
  const std::string w(who_);
  hipError_t e = hipStreamSynchronize(stream_);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(BSATTN_EHIP, w + ": kernel failed: " + hipGetErrorString(e));
  if (canary_) {
    std::vector<unsigned char> got(kCanaryBytes, 0);
    e = hipMemcpy(got.data(), static_cast<char*>(ws_) + need_, kCanaryBytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return check_hip(e, "debug canary read");
    for (unsigned char c : got)
      if (c != kCanary)
        return set_error(BSATTN_EHIP, w + ": workspace written past the " +
                                          std::to_string(need_) + " bytes the call needs");
  }
  if (debug_level() >= 1) std::fprintf(stderr, "[bsattn] done %s\n", who_);
  return st;
}

void clear_error() { g_last_error.clear(); }

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSATTN_OK;
  return set_error(BSATTN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Number of distinct blocks in G U [lo, hi].
int union_size(const std::vector<int32_t>& G, int lo, int hi) {
  int in_win = 0;
  for (int x : G) in_win += (x >= lo && x <= hi);
  return (hi - lo + 1) + (int)G.size() - in_win;
}

int check_device(int device) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (cur != device)
    return set_error(BSATTN_EINVAL, "current device differs from the device the handle was built on");
  return BSATTN_OK;
}

// d_max: the largest head dimension the caller's kernels are built for (64, or 128
// for the bf16 block-sparse forward and backward, which take d = 64 or 128).
int check_tensor_args(int batch, int d, float scale, std::initializer_list<const void*> ptrs,
                      const char* who, int d_max = kHead) {
  if (batch < 1) return set_error(BSATTN_EINVAL, std::string(who) + ": batch must be >= 1");
  if (d != kHead && !(d == 128 && d_max == 128))
    return set_error(BSATTN_EUNSUPPORTED,
                     std::string(who) + (d_max == 128 ? ": head dim must be 64 or 128"
                                                      : ": head dim must be 64"));
  if (!(scale > 0.f) || !std::isfinite(scale))
    return set_error(BSATTN_EINVAL, std::string(who) + ": scale must be finite and > 0");
  for (const void* p : ptrs) {
    if (p == nullptr) return set_error(BSATTN_EINVAL, std::string(who) + ": null tensor pointer");
    if (!aligned16(p)) return set_error(BSATTN_EINVAL, std::string(who) + ": tensor pointer not 16-byte aligned");
  }
  return BSATTN_OK;
}

// The rounding residual of O is a bf16 tensor like O; it has no meaning for fp32.
int check_o_lo(const void* o_lo, bsattn_dtype dt, const char* who) {
  if (o_lo == nullptr) return BSATTN_OK;
  if (dt != BSATTN_BF16)
    return set_error(BSATTN_EINVAL, std::string(who) + ": o_lo is for bf16 outputs only");
  if (!aligned16(o_lo)) return set_error(BSATTN_EINVAL, std::string(who) + ": o_lo not 16-byte aligned");
  return BSATTN_OK;
}

int check_workspace(void* ws, size_t ws_bytes, size_t need, const char* who) {
  if (ws_bytes < need)
    return set_error(BSATTN_EINVAL, std::string(who) + ": workspace too small (need " +
                                        std::to_string(need) + " bytes)");
  if (need > 0 && (ws == nullptr || !aligned16(ws)))
    return set_error(BSATTN_EINVAL, std::string(who) + ": workspace null or not 16-byte aligned");
  return BSATTN_OK;
}

void free_layout(bsattn_layout* L) {
  if (L->built != nullptr) (void)hipEventDestroy(L->built);
  (void)hipFree(L->d_gblk);
  (void)hipFree(L->d_ngblk);
  (void)hipFree(L->d_row_ptr);
  (void)hipFree(L->d_col_idx);
  (void)hipFree(L->d_csc_ptr);
  (void)hipFree(L->d_csc_idx);
  (void)hipFree(L->d_rbits);
  (void)hipFree(L->d_kv_order);
  (void)hipFree(L->d_row_info);
  (void)hipFree(L->d_col_info);
  delete L;
}

void free_plan(lfattn_plan* P) {
  if (P->built != nullptr) (void)hipEventDestroy(P->built);
  (void)hipFree(P->d_gtok);
  (void)hipFree(P->d_gidx);
  (void)hipFree(P->d_tile_gmask);
  (void)hipFree(P->d_ct);
  delete P;
}

template <typename T>
int dev_alloc(T** p, size_t count) {
  *p = nullptr;
  if (count == 0) count = 1;
  hipError_t e = hipMalloc((void**)p, count * sizeof(T));
  if (e != hipSuccess) {
    *p = nullptr;
    return set_error(BSATTN_ENOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  return BSATTN_OK;
}

}  // namespace
}  // namespace bsattn

SegPlan seg_plan(const bsattn_layout* L, int batch) {
  // A segment is one work item, scheduled first on its XCD, so it should end within
  // the run: no longer than about the average work of one work-group slot (4 per
  // compute unit), while longer segments mean fewer fp32 partial tiles to write
  // and merge.  The smallest power of two in 8..64 above that average, and short
  // enough that a full row still makes two segments (measured against the next
  // shorter one: 1.3 % faster at batch 4, n = 4096; 1.7 % and 2.9 % on the forward
  // at batch 2, n = 4096 and at n = 16,384; a 64-block row left whole ran 11 %
  // slower at batch 4, n = 4096).
  const int64_t pairs = (int64_t)batch * L->heads * L->nnz_per_head;
  const int64_t avg = pairs / (4 * (int64_t)(L->cus > 0 ? L->cus : 1));
  int seg = 8;
  while (seg < 64 && seg <= avg && 2 * seg < L->nb) seg *= 2;
  SegPlan p;
  p.split = L->nb > seg ? 1 : 0;
  p.seg = p.split ? seg : L->nb;
  p.nseg = p.split ? (L->nb + seg - 1) / seg : 1;
  return p;
}

using namespace bsattn;

extern "C" {

int bsattn_layout_build(int n, int b, int heads, const int32_t* global_blocks, int g, int w,
                        int r, uint64_t seed, hipStream_t stream, bsattn_layout** out) {
  clear_error();
  if (out == nullptr) return set_error(BSATTN_EINVAL, "layout_build: out is null");
  *out = nullptr;
  if (b != kBlock) return set_error(BSATTN_EUNSUPPORTED, "layout_build: block size must be 64");
  if (n <= 0) return set_error(BSATTN_EINVAL, "layout_build: n must be positive");
  if (n > kMaxNb * kBlock) return set_error(BSATTN_EUNSUPPORTED, "layout_build: n/b above 4096");
  // ceil(n / b) blocks ([BB] App. D eq. (13)); the last one is short when b does
  // not divide n, and its missing positions are not tokens (nothing is padded)
  const int nb = (n + b - 1) / b;
  if (nb > kMaxNb) return set_error(BSATTN_EUNSUPPORTED, "layout_build: n/b above 4096");
  if (heads < 1) return set_error(BSATTN_EINVAL, "layout_build: heads must be >= 1");
  if (w < 1 || w % 2 == 0) return set_error(BSATTN_EINVAL, "layout_build: w must be odd and >= 1");
  if (r < 0) return set_error(BSATTN_EINVAL, "layout_build: r must be >= 0");
  if (r > kMaxR) return set_error(BSATTN_EUNSUPPORTED, "layout_build: r above 64");
  if (g < 0 || g > nb) return set_error(BSATTN_EINVAL, "layout_build: g out of range");
  if (g > 0 && global_blocks == nullptr) return set_error(BSATTN_EINVAL, "layout_build: global_blocks is null");
  std::vector<int32_t> G(global_blocks, global_blocks + g);
  for (int x = 0; x < g; ++x) {
    if (G[x] < 0 || G[x] >= nb) return set_error(BSATTN_EINVAL, "layout_build: global block out of range");
    if (x > 0 && G[x] <= G[x - 1]) return set_error(BSATTN_EINVAL, "layout_build: global blocks not sorted and unique");
  }
  const int64_t nnz_limit = (int64_t)1 << 31;
  auto L = new bsattn_layout();
  L->n = n; L->b = b; L->nb = nb; L->heads = heads; L->g = g; L->w = w; L->r = r; L->seed = seed;
  L->gblk = G;
  std::vector<int32_t> ng;
  {
    size_t p = 0;
    for (int i = 0; i < nb; ++i) {
      if (p < G.size() && G[p] == i) { ++p; continue; }
      ng.push_back(i);
    }
  }
  L->row_len.resize(nb);
  int64_t nnz = 0;
  const int half = (w - 1) / 2;
  {
    size_t p = 0;
    for (int i = 0; i < nb; ++i) {
      bool gl = p < G.size() && G[p] == i;
      if (gl) ++p;
      int len;
      if (gl) {
        len = nb;
      } else {
        const int lo = i - half < 0 ? 0 : i - half;
        const int hi = i + half > nb - 1 ? nb - 1 : i + half;
        const int e = union_size(G, lo, hi);
        const int m = nb - e;
        len = e + (r < m ? r : m);
      }
      L->row_len[i] = len;
      nnz += len;
    }
  }
  L->nnz_per_head = nnz;
  if (nnz * heads >= nnz_limit) {
    delete L;
    return set_error(BSATTN_EUNSUPPORTED, "layout_build: too many block pairs");
  }
  hipError_t e = hipGetDevice(&L->device);
  if (e != hipSuccess) { delete L; return check_hip(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&L->cus, hipDeviceAttributeMultiprocessorCount, L->device);
  if (e != hipSuccess) { delete L; return check_hip(e, "hipDeviceGetAttribute"); }
  e = hipDeviceGetAttribute(&L->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, L->device);
  if (e != hipSuccess) { delete L; return check_hip(e, "hipDeviceGetAttribute"); }
  int st = BSATTN_OK;
  if ((st = dev_alloc(&L->d_gblk, (size_t)g)) || (st = dev_alloc(&L->d_ngblk, ng.size())) ||
      (st = dev_alloc(&L->d_row_ptr, (size_t)heads * nb + 1)) ||
      (st = dev_alloc(&L->d_col_idx, (size_t)(nnz * heads))) ||
      (st = dev_alloc(&L->d_csc_ptr, (size_t)heads * nb + 1)) ||
      (st = dev_alloc(&L->d_csc_idx, (size_t)(nnz * heads))) ||
      (st = dev_alloc(&L->d_rbits, (size_t)heads * nb * ((nb + 31) / 32 + 1))) ||
      (st = dev_alloc(&L->d_kv_order, (size_t)heads * ng.size())) ||
      (st = dev_alloc(&L->d_row_info, (size_t)heads * ng.size() * 4)) ||
      (st = dev_alloc(&L->d_col_info, (size_t)heads * ng.size() * 4))) {
    free_layout(L);
    return st;
  }
  if ((st = check_hip(hipMemsetAsync(L->d_rbits, 0, (size_t)heads * nb * ((nb + 31) / 32 + 1) * 4, stream),
                      "clear random-pick bitmap"))) {
    free_layout(L);
    return st;
  }
  // the uploads read host copies owned by the handle, so they stay valid for as
  // long as the asynchronous copies may run
  L->ngblk = ng;
  if (g > 0 && (st = check_hip(hipMemcpyAsync(L->d_gblk, L->gblk.data(), (size_t)g * 4,
                                              hipMemcpyHostToDevice, stream), "upload global blocks"))) {
    free_layout(L);
    return st;
  }
  if (!L->ngblk.empty() &&
      (st = check_hip(hipMemcpyAsync(L->d_ngblk, L->ngblk.data(), L->ngblk.size() * 4,
                                     hipMemcpyHostToDevice, stream), "upload blocks"))) {
    free_layout(L);
    return st;
  }
  for (int h = 0; h < heads; ++h) L->kv_order_init.insert(L->kv_order_init.end(), ng.begin(), ng.end());
  if (!L->kv_order_init.empty() &&
      (st = check_hip(hipMemcpyAsync(L->d_kv_order, L->kv_order_init.data(),
                                     L->kv_order_init.size() * 4, hipMemcpyHostToDevice, stream),
                      "upload work order"))) {
    free_layout(L);
    return st;
  }
  DebugCall dbg("layout_build", stream, nullptr, 0, 0);
  if ((st = launch_layout_rowptr(L, stream)) || (st = launch_layout_build(L, stream))) {
    free_layout(L);
    return st;
  }
  if ((st = check_hip(hipEventCreateWithFlags(&L->built, hipEventDisableTiming), "layout event")) ||
      (st = check_hip(hipEventRecord(L->built, stream), "layout event record")) ||
      (st = dbg.finish(BSATTN_OK))) {
    free_layout(L);
    return st;
  }
  *out = L;
  return BSATTN_OK;
}

int bsattn_layout_rebuild(bsattn_layout* L, uint64_t seed, hipStream_t stream) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "layout_rebuild: null layout");
  int st = check_device(L->device);
  if (st) return st;
  L->seed = seed;
  DebugCall dbg("layout_rebuild", stream, nullptr, 0, 0);
  if ((st = launch_layout_build(L, stream))) return st;
  return dbg.finish(check_hip(hipEventRecord(L->built, stream), "layout event record"));
}

int bsattn_layout_info(const bsattn_layout* L, int* nb, int* heads, int64_t* nnzb_total) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "layout_info: null layout");
  if (nb) *nb = L->nb;
  if (heads) *heads = L->heads;
  if (nnzb_total) *nnzb_total = L->nnz_per_head * L->heads;
  return BSATTN_OK;
}

int bsattn_layout_to_host(const bsattn_layout* L, int32_t* row_ptr, int32_t* col_idx,
                          int32_t* csc_ptr, int32_t* csc_idx) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "layout_to_host: null layout");
  int st = check_device(L->device);
  if (st) return st;
  // wait for this layout's last build or redraw only (not for the whole device),
  // then copy on a private stream that does not wait for other work either
  if ((st = check_hip(hipEventSynchronize(L->built), "layout_to_host wait"))) return st;
  hipStream_t s = nullptr;
  if ((st = check_hip(hipStreamCreateWithFlags(&s, hipStreamNonBlocking), "layout_to_host stream")))
    return st;
  const size_t np = ((size_t)L->heads * L->nb + 1) * 4;
  const size_t nz = (size_t)(L->nnz_per_head * L->heads) * 4;
  if (row_ptr) st = check_hip(hipMemcpyAsync(row_ptr, L->d_row_ptr, np, hipMemcpyDeviceToHost, s), "copy row_ptr");
  if (!st && col_idx) st = check_hip(hipMemcpyAsync(col_idx, L->d_col_idx, nz, hipMemcpyDeviceToHost, s), "copy col_idx");
  if (!st && csc_ptr) st = check_hip(hipMemcpyAsync(csc_ptr, L->d_csc_ptr, np, hipMemcpyDeviceToHost, s), "copy csc_ptr");
  if (!st && csc_idx) st = check_hip(hipMemcpyAsync(csc_idx, L->d_csc_idx, nz, hipMemcpyDeviceToHost, s), "copy csc_idx");
  const int st2 = check_hip(hipStreamSynchronize(s), "layout_to_host copy");
  (void)hipStreamDestroy(s);
  return st ? st : st2;
}

int bsattn_layout_destroy(bsattn_layout* L) {
  clear_error();
  if (L == nullptr) return BSATTN_OK;
  // the handle's own build work; releasing its arrays then follows hipFree's rules
  // for work still reading them (the caller orders its own calls before this one)
  int st = check_hip(hipEventSynchronize(L->built), "layout_destroy wait");
  free_layout(L);
  return st;
}

size_t bsattn_fwd_workspace(const bsattn_layout* L, int batch, int d) {
  if (L == nullptr || batch < 1 || (d != kHead && d != 128)) return 0;
  return fwd_workspace_bytes(L, batch, d);
}

size_t bsattn_bwd_workspace(const bsattn_layout* L, int batch, int d) {
  if (L == nullptr || batch < 1 || (d != kHead && d != 128)) return 0;
  return bwd_workspace_bytes(L, batch, d);
}

int bsattn_fwd(const bsattn_layout* L, int batch, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, void* o, float* lse, void* o_lo,
               void* workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "fwd: null layout");
  if (dt != BSATTN_F32 && dt != BSATTN_BF16) return set_error(BSATTN_EUNSUPPORTED, "fwd: unknown dtype");
  int st = check_tensor_args(batch, d, scale, {q, k, v, o}, "fwd",
                             dt == BSATTN_BF16 ? 128 : kHead);
  if (st) return st;
  if (lse != nullptr && !aligned16(lse)) return set_error(BSATTN_EINVAL, "fwd: lse not 16-byte aligned");
  if ((st = check_o_lo(o_lo, dt, "fwd"))) return st;
  if ((int64_t)batch * L->heads * L->n * d >= ((int64_t)1 << 40))
    return set_error(BSATTN_EUNSUPPORTED, "fwd: tensor too large");
  const size_t need = fwd_workspace_bytes_dt(L, batch, dt, d);
  if ((st = check_workspace(workspace, ws_bytes, need, "fwd"))) return st;
  if ((st = check_device(L->device))) return st;
  DebugCall dbg("fwd", stream, workspace, ws_bytes, need);
  return dbg.finish(launch_fwd(L, batch, dt, d, scale, q, k, v, o, lse, o_lo, workspace, stream));
}

int bsattn_bwd(const bsattn_layout* L, int batch, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, const void* o, const void* o_lo,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               void* workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "bwd: null layout");
  if (dt != BSATTN_BF16) return set_error(BSATTN_EUNSUPPORTED, "bwd: only bf16 is built");
  int st = check_tensor_args(batch, d, scale, {q, k, v, o, lse, dout, dq, dk, dv}, "bwd", 128);
  if (st) return st;
  if ((st = check_o_lo(o_lo, dt, "bwd"))) return st;
  if ((int64_t)batch * L->heads * L->n * d >= ((int64_t)1 << 40))
    return set_error(BSATTN_EUNSUPPORTED, "bwd: tensor too large");
  const size_t need = bwd_workspace_bytes(L, batch, d);
  if ((st = check_workspace(workspace, ws_bytes, need, "bwd"))) return st;
  if ((st = check_device(L->device))) return st;
  DebugCall dbg("bwd", stream, workspace, ws_bytes, need);
  return dbg.finish(
      launch_bwd(L, batch, d, scale, q, k, v, o, o_lo, lse, dout, dq, dk, dv, workspace, stream));
}

int bsattn_bwd_noalloc(const bsattn_layout* L, int batch, int d, bsattn_dtype dt, float scale,
                       const void* q, const void* k, const void* v, const void* o,
                       const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
                       void* dv, hipStream_t stream) {
  clear_error();
  if (L == nullptr) return set_error(BSATTN_EINVAL, "bwd_noalloc: null layout");
  if (dt != BSATTN_BF16) return set_error(BSATTN_EUNSUPPORTED, "bwd_noalloc: only bf16 is built");
  int st = check_tensor_args(batch, d, scale, {q, k, v, o, lse, dout, dq, dk, dv},
                             "bwd_noalloc", 128);
  if (st) return st;
  if ((st = check_o_lo(o_lo, dt, "bwd_noalloc"))) return st;
  if ((int64_t)batch * L->heads * L->n * d >= ((int64_t)1 << 40))
    return set_error(BSATTN_EUNSUPPORTED, "bwd_noalloc: tensor too large");
  const size_t need = bwd_workspace_bytes(L, batch, d);
  if (need > noalloc_scratch_bytes())
    return set_error(BSATTN_EINVAL, "bwd_noalloc: needs " + std::to_string(need) +
                                        " bytes of scratch, above the static " +
                                        std::to_string(noalloc_scratch_bytes()) +
                                        "; use bsattn_bwd with a workspace");
  if ((st = check_device(L->device))) return st;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  DebugCall dbg("bwd_noalloc", stream, ws, noalloc_scratch_bytes(), need);
  return dbg.finish(
      launch_bwd(L, batch, d, scale, q, k, v, o, o_lo, lse, dout, dq, dk, dv, ws, stream));
}

}  // extern "C"

namespace {

// Class tiles of one head period: for each head, each residue class modulo its
// stride and each 64-index tile of the class; tiles holding no global token
// first, then the others, each group in (head, class, tile) order.
void build_class_tiles(lfattn_plan* P) {
  const int ph = P->heads > 0 ? P->heads : 1;
  std::vector<LfTileRef> with_g;
  P->ct.clear();
  for (int h = 0; h < ph; ++h) {
    const int s = P->dil[h] + 1;
    for (int c = 0; c < s; ++c) {
      const int nc = (P->n - c + s - 1) / s;
      for (int t = 0; t * kBlock < nc; ++t) {
        LfTileRef r;
        r.h = h;
        r.c = (int16_t)c;
        r.s = (int16_t)s;
        r.t = t;
        r.nc = nc;
        bool g = false;
        for (int x = t * kBlock; x < std::min(nc, (t + 1) * kBlock) && !g; ++x)
          g = P->gidx[c + s * x] >= 0;
        (g ? with_g : P->ct).push_back(r);
      }
    }
  }
  P->nct_plain = (int)P->ct.size();
  P->ct.insert(P->ct.end(), with_g.begin(), with_g.end());
  P->nct = (int)P->ct.size();
}

// Blocked window of the ETC construction (block size wb > 0; 0: sliding window).
struct BlockedWindow {
  int wb = 0, woff = 0, whalf = 0;
};

int lf_plan_build(int n, int window_one_side, const int32_t* global_tokens, int n_global,
                  int heads, const int32_t* dilation, int causal, hipStream_t stream,
                  lfattn_plan** out, BlockedWindow bw = BlockedWindow()) {
  clear_error();
  if (out == nullptr) return set_error(BSATTN_EINVAL, "lf_plan_build: out is null");
  *out = nullptr;
  if (n <= 0) return set_error(BSATTN_EINVAL, "lf_plan_build: n must be positive");
  if (n > kMaxLfTokens) return set_error(BSATTN_EUNSUPPORTED, "lf_plan_build: n above 262144");
  if (window_one_side < 0) return set_error(BSATTN_EINVAL, "lf_plan_build: window must be >= 0");
  if (n_global < 0 || n_global > n) return set_error(BSATTN_EINVAL, "lf_plan_build: n_global out of range");
  if (n_global > 0 && global_tokens == nullptr) return set_error(BSATTN_EINVAL, "lf_plan_build: global_tokens is null");
  for (int x = 0; x < n_global; ++x) {
    if (global_tokens[x] < 0 || global_tokens[x] >= n) return set_error(BSATTN_EINVAL, "lf_plan_build: global token out of range");
    if (x > 0 && global_tokens[x] <= global_tokens[x - 1]) return set_error(BSATTN_EINVAL, "lf_plan_build: global tokens not sorted and unique");
  }
  if (heads < 0 || heads > kMaxLfHeads) return set_error(BSATTN_EINVAL, "lf_plan_build: heads out of range");
  if (causal != 0 && causal != 1) return set_error(BSATTN_EINVAL, "lf_plan_build: causal must be 0 or 1");
  if (causal && n_global > 0)
    return set_error(BSATTN_EINVAL, "lf_plan_build: the causal window takes no global tokens");
  for (int h = 0; dilation != nullptr && h < heads; ++h)
    if (dilation[h] < 0 || dilation[h] > kMaxLfDilation)
      return set_error(BSATTN_EINVAL, "lf_plan_build: dilation out of [0, 1023]");
  // the window span w1 * (d + 1) must stay an int
  int64_t span = window_one_side;
  for (int h = 0; dilation != nullptr && h < heads; ++h)
    span = std::max(span, (int64_t)window_one_side * (dilation[h] + 1));
  if (span > ((int64_t)1 << 30)) return set_error(BSATTN_EUNSUPPORTED, "lf_plan_build: window too long");

  auto P = new lfattn_plan();
  P->n = n;
  P->w1 = window_one_side;
  P->ng = n_global;
  P->nt = (n + kBlock - 1) / kBlock;
  P->ngt = (n_global + kBlock - 1) / kBlock;
  P->heads = heads;
  P->causal = causal;
  P->wb = bw.wb;
  P->woff = bw.woff;
  P->whalf = bw.whalf;
  if (heads == 0)
    P->dil.assign(1, 0);
  else if (dilation == nullptr)
    P->dil.assign(heads, 0);
  else
    P->dil.assign(dilation, dilation + heads);
  P->gtok.assign(global_tokens, global_tokens + n_global);
  P->gidx.assign(n, -1);
  P->tile_gmask.assign(P->nt, 0ull);
  for (int x = 0; x < n_global; ++x) {
    const int t = P->gtok[x];
    P->gidx[t] = x;
    P->tile_gmask[t / kBlock] |= 1ull << (t % kBlock);
  }
  build_class_tiles(P);
  hipError_t e = hipGetDevice(&P->device);
  if (e != hipSuccess) { delete P; return check_hip(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&P->cus, hipDeviceAttributeMultiprocessorCount, P->device);
  if (e != hipSuccess) { delete P; return check_hip(e, "hipDeviceGetAttribute"); }
  int st;
  if ((st = dev_alloc(&P->d_gtok, (size_t)n_global)) || (st = dev_alloc(&P->d_gidx, (size_t)n)) ||
      (st = dev_alloc(&P->d_tile_gmask, (size_t)P->nt)) ||
      (st = dev_alloc(&P->d_ct, (size_t)P->nct))) {
    free_plan(P);
    return st;
  }
  if ((n_global > 0 && (st = check_hip(hipMemcpyAsync(P->d_gtok, P->gtok.data(), (size_t)n_global * 4,
                                                      hipMemcpyHostToDevice, stream), "upload global tokens"))) ||
      (st = check_hip(hipMemcpyAsync(P->d_gidx, P->gidx.data(), (size_t)n * 4, hipMemcpyHostToDevice, stream),
                      "upload token index")) ||
      (st = check_hip(hipMemcpyAsync(P->d_tile_gmask, P->tile_gmask.data(), (size_t)P->nt * 8,
                                     hipMemcpyHostToDevice, stream), "upload tile masks")) ||
      (st = check_hip(hipMemcpyAsync(P->d_ct, P->ct.data(), (size_t)P->nct * sizeof(LfTileRef),
                                     hipMemcpyHostToDevice, stream), "upload class tiles")) ||
      (st = check_hip(hipEventCreateWithFlags(&P->built, hipEventDisableTiming), "plan event")) ||
      (st = check_hip(hipEventRecord(P->built, stream), "plan event record"))) {
    free_plan(P);
    return st;
  }
  *out = P;
  return BSATTN_OK;
}

// A plan fixed to a head count takes calls with that count only.
int check_plan_heads(const lfattn_plan* P, int heads, const char* who) {
  if (P->heads > 0 && heads != P->heads)
    return set_error(BSATTN_EINVAL, std::string(who) + ": heads differ from the plan's");
  return BSATTN_OK;
}

}  // namespace

extern "C" {

int lfattn_plan_build(int n, int window_one_side, const int32_t* global_tokens, int n_global,
                      hipStream_t stream, lfattn_plan** out) {
  return lf_plan_build(n, window_one_side, global_tokens, n_global, 0, nullptr, 0, stream, out);
}

int lfattn_plan_build_etc(int g, int n, int b, int w, hipStream_t stream, lfattn_plan** out) {
  clear_error();
  if (out == nullptr) return set_error(BSATTN_EINVAL, "lf_plan_build_etc: out is null");
  *out = nullptr;
  if (g < 0 || n < 1 || b < 1) return set_error(BSATTN_EINVAL, "lf_plan_build_etc: need g >= 0, n >= 1, b >= 1");
  if (w < 1 || w % 2 == 0) return set_error(BSATTN_EINVAL, "lf_plan_build_etc: w must be odd and >= 1");
  if ((int64_t)g + n > kMaxLfTokens) return set_error(BSATTN_EUNSUPPORTED, "lf_plan_build_etc: g + n above 262144");
  const int nb = (n + b - 1) / b;
  BlockedWindow bw;
  bw.wb = b;
  bw.woff = g;
  bw.whalf = std::min((w - 1) / 2, nb);   // a wider window holds the same blocks
  std::vector<int32_t> gt(g);
  for (int x = 0; x < g; ++x) gt[x] = x;
  return lf_plan_build(g + n, 0, gt.data(), g, 0, nullptr, 0, stream, out, bw);
}

int lfattn_plan_build_dilated(int n, int window_one_side, const int32_t* global_tokens,
                              int n_global, int heads, const int32_t* dilation, int causal,
                              hipStream_t stream, lfattn_plan** out) {
  if (heads < 1) {
    clear_error();
    if (out != nullptr) *out = nullptr;
    return set_error(BSATTN_EINVAL, "lf_plan_build: heads must be >= 1");
  }
  return lf_plan_build(n, window_one_side, global_tokens, n_global, heads, dilation, causal,
                       stream, out);
}

int lfattn_plan_destroy(lfattn_plan* P) {
  clear_error();
  if (P == nullptr) return BSATTN_OK;
  // the plan's uploads; releasing its arrays then follows hipFree's rules for work
  // still reading them (the caller orders its own calls before this one)
  int st = check_hip(hipEventSynchronize(P->built), "lf_plan_destroy wait");
  free_plan(P);
  return st;
}

size_t lfattn_fwd_workspace(const lfattn_plan* P, int batch, int heads, int d) {
  if (P == nullptr || batch < 1 || heads < 1 || (d != kHead && d != 128)) return 0;
  if (P->heads > 0 && heads != P->heads) return 0;
  return lf_workspace_bytes(P, batch, heads, d);
}

}  // extern "C"

namespace {

int lf_fwd_impl(const char* who, const lfattn_plan* P, int batch, int heads, int d,
                bsattn_dtype dt, float scale, const void* q, const void* k, const void* v,
                const void* qg, const void* kg, const void* vg, void* o, float* lse,
                void* o_lo, void* workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  const std::string w(who);
  if (P == nullptr) return set_error(BSATTN_EINVAL, w + ": null plan");
  if (heads < 1) return set_error(BSATTN_EINVAL, w + ": heads must be >= 1");
  int st = check_plan_heads(P, heads, who);
  if (st) return st;
  if (dt != BSATTN_BF16) return set_error(BSATTN_EUNSUPPORTED, w + ": only bf16 is built");
  if ((st = check_tensor_args(batch, d, scale, {q, k, v, o}, who, 128))) return st;
  if (qg != nullptr && (st = check_tensor_args(batch, d, scale, {qg, kg, vg}, who, 128))) return st;
  if (lse != nullptr && !aligned16(lse)) return set_error(BSATTN_EINVAL, w + ": lse not 16-byte aligned");
  if ((st = check_o_lo(o_lo, dt, who))) return st;
  if ((int64_t)batch * heads * P->n * d >= ((int64_t)1 << 40))
    return set_error(BSATTN_EUNSUPPORTED, w + ": tensor too large");
  const size_t need = lf_workspace_bytes(P, batch, heads, d);
  if ((st = check_workspace(workspace, ws_bytes, need, who))) return st;
  if ((st = check_device(P->device))) return st;
  DebugCall dbg(who, stream, workspace, ws_bytes, need);
  return dbg.finish(launch_lf_fwd(P, batch, heads, d, scale, q, k, v, qg, kg, vg, o, lse, o_lo,
                                  workspace, stream));
}

}  // namespace

extern "C" {

int lfattn_fwd(const lfattn_plan* P, int batch, int heads, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, void* o, float* lse, void* o_lo,
               void* workspace, size_t ws_bytes, hipStream_t stream) {
  return lf_fwd_impl("lf_fwd", P, batch, heads, d, dt, scale, q, k, v, nullptr, nullptr,
                     nullptr, o, lse, o_lo, workspace, ws_bytes, stream);
}

int lfattn_fwd_gproj(const lfattn_plan* P, int batch, int heads, int d, bsattn_dtype dt,
                     float scale, const void* q, const void* k, const void* v, const void* qg,
                     const void* kg, const void* vg, void* o, float* lse, void* o_lo,
                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (qg == nullptr || kg == nullptr || vg == nullptr) {
    clear_error();
    return set_error(BSATTN_EINVAL, "lf_fwd_gproj: null global projection");
  }
  return lf_fwd_impl("lf_fwd_gproj", P, batch, heads, d, dt, scale, q, k, v, qg, kg, vg, o, lse,
                     o_lo, workspace, ws_bytes, stream);
}

size_t lfattn_bwd_workspace(const lfattn_plan* P, int batch, int heads, int d) {
  if (P == nullptr || batch < 1 || heads < 1 || (d != kHead && d != 128)) return 0;
  if (P->heads > 0 && heads != P->heads) return 0;
  return lf_bwd_workspace_bytes(P, batch, heads, d);
}

}  // extern "C"

namespace {

int lf_bwd_impl(const char* who, const lfattn_plan* P, int batch, int heads, int d,
                bsattn_dtype dt, float scale, const void* q, const void* k, const void* v,
                const void* qg, const void* kg, const void* vg, const void* o, const void* o_lo,
                const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dqg,
                void* dkg, void* dvg, void* workspace, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  const std::string w(who);
  if (P == nullptr) return set_error(BSATTN_EINVAL, w + ": null plan");
  if (heads < 1) return set_error(BSATTN_EINVAL, w + ": heads must be >= 1");
  int st = check_plan_heads(P, heads, who);
  if (st) return st;
  if (dt != BSATTN_BF16) return set_error(BSATTN_EUNSUPPORTED, w + ": only bf16 is built");
  if ((st = check_tensor_args(batch, d, scale, {q, k, v, o, lse, dout, dq, dk, dv}, who, 128)))
    return st;
  if ((st = check_o_lo(o_lo, dt, who))) return st;
  if (qg != nullptr) {
    if ((st = check_tensor_args(batch, d, scale, {qg, kg, vg, dqg, dkg, dvg}, who, 128)))
      return st;
    const void* outs[6] = {dq, dk, dv, dqg, dkg, dvg};
    for (int x = 0; x < 6; ++x)
      for (int y = x + 1; y < 6; ++y)
        if (outs[x] == outs[y]) return set_error(BSATTN_EINVAL, w + ": output gradients alias");
  }
  if ((int64_t)batch * heads * P->n * d >= ((int64_t)1 << 40))
    return set_error(BSATTN_EUNSUPPORTED, w + ": tensor too large");
  const size_t need = lf_bwd_workspace_bytes(P, batch, heads, d);
  if ((st = check_workspace(workspace, ws_bytes, need, who))) return st;
  if ((st = check_device(P->device))) return st;
  DebugCall dbg(who, stream, workspace, ws_bytes, need);
  return dbg.finish(launch_lf_bwd(P, batch, heads, d, scale, q, k, v, qg, kg, vg, o, o_lo, lse,
                                  dout, dq, dk, dv, dqg, dkg, dvg, workspace, stream));
}

}  // namespace

extern "C" {

int lfattn_bwd(const lfattn_plan* P, int batch, int heads, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, const void* o, const void* o_lo,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               void* workspace, size_t ws_bytes, hipStream_t stream) {
  return lf_bwd_impl("lf_bwd", P, batch, heads, d, dt, scale, q, k, v, nullptr, nullptr, nullptr,
                     o, o_lo, lse, dout, dq, dk, dv, nullptr, nullptr, nullptr, workspace,
                     ws_bytes, stream);
}

int lfattn_bwd_gproj(const lfattn_plan* P, int batch, int heads, int d, bsattn_dtype dt,
                     float scale, const void* q, const void* k, const void* v, const void* qg,
                     const void* kg, const void* vg, const void* o, const void* o_lo,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* dqg, void* dkg, void* dvg, void* workspace, size_t ws_bytes,
                     hipStream_t stream) {
  if (qg == nullptr || kg == nullptr || vg == nullptr || dqg == nullptr || dkg == nullptr ||
      dvg == nullptr) {
    clear_error();
    return set_error(BSATTN_EINVAL, "lf_bwd_gproj: null global projection or gradient");
  }
  return lf_bwd_impl("lf_bwd_gproj", P, batch, heads, d, dt, scale, q, k, v, qg, kg, vg, o, o_lo,
                     lse, dout, dq, dk, dv, dqg, dkg, dvg, workspace, ws_bytes, stream);
}

const char* bsattn_status_str(int status) {
  switch (status) {
    case BSATTN_OK: return "BSATTN_OK";
    case BSATTN_EINVAL: return "BSATTN_EINVAL";
    case BSATTN_EUNSUPPORTED: return "BSATTN_EUNSUPPORTED";
    case BSATTN_EHIP: return "BSATTN_EHIP";
    case BSATTN_ENOMEM: return "BSATTN_ENOMEM";
    default: return "BSATTN_UNKNOWN";
  }
}

const char* bsattn_last_error(void) { return g_last_error.c_str(); }

const char* bsattn_version(void) { return "bsattn 0.1.0 (gfx950)"; }

int bsattn_profile_enable(int on) {
  clear_error();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return BSATTN_OK;
}

int bsattn_profile_read(int max_kernels, char* names, int64_t* counts, double* total_ms,
                        int* n_kernels) {
  clear_error();
  if (max_kernels < 0 || (max_kernels > 0 && (!names || !counts || !total_ms)) || !n_kernels)
    return set_error(BSATTN_EINVAL, "profile_read: bad arguments");
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof);
  }
  std::vector<std::string> keys;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  int st = BSATTN_OK;
  for (const ProfRecord& r : recs) {
    float t = 0.f;
    if (st == BSATTN_OK) st = check_hip(hipEventSynchronize(r.stop), "profile sync");
    if (st == BSATTN_OK) st = check_hip(hipEventElapsedTime(&t, r.start, r.stop), "profile elapsed");
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    if (st) continue;
    size_t k = 0;
    while (k < keys.size() && keys[k] != r.name) ++k;
    if (k == keys.size()) { keys.push_back(r.name); cnt.push_back(0); ms.push_back(0.0); }
    cnt[k] += 1;
    ms[k] += t;
  }
  if (st) return st;
  const int n = (int)keys.size() < max_kernels ? (int)keys.size() : max_kernels;
  for (int i = 0; i < n; ++i) {
    std::memset(names + 48 * i, 0, 48);
    std::strncpy(names + 48 * i, keys[i].c_str(), 47);
    counts[i] = cnt[i];
    total_ms[i] = ms[i];
  }
  *n_kernels = n;
  return BSATTN_OK;
}

}  // extern "C"
