// A host-only stand-in for the HIP runtime and for the library's kernel-side
// functions, so that the C ABI's host code (abi.cpp: argument checks, handle
// construction and teardown, the host-side Longformer plan tables, the error and
// debug paths) can be built with AddressSanitizer, LeakSanitizer and UBSan and run
// on a machine without a GPU.  "Device" memory is host memory, copies are memcpy,
// streams and events are small heap objects (so an unbalanced create/destroy shows
// up as a leak), and every launch succeeds without doing anything, except that a
// test can ask the forward to write past the workspace bytes it needs.

#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "../../block_sparse_long_bsattn_amd/csrc/internal.hpp"

struct ihipStream_t { int id; };
struct ihipEvent_t { int id; };

extern "C" {

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t attr, int) {
  *pi = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
  return hipSuccess;
}

hipError_t hipMalloc(void** p, size_t bytes) {
  *p = std::aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
  return *p != nullptr ? hipSuccess : hipErrorOutOfMemory;
}

hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}

hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  if (bytes) std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  if (bytes) std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipMemsetAsync(void* dst, int value, size_t bytes, hipStream_t) {
  if (bytes) std::memset(dst, value, bytes);
  return hipSuccess;
}

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  *s = new ihipStream_t{1};
  return hipSuccess;
}

hipError_t hipStreamDestroy(hipStream_t s) {
  delete s;
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* cs) {
  *cs = hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipEventCreate(hipEvent_t* e) {
  *e = new ihipEvent_t{1};
  return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = new ihipEvent_t{2};
  return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }

hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t) { return "fake HIP error"; }

}  // extern "C"

// Set by the driver: the next forward writes this many bytes past what it needs.
size_t g_fake_overrun = 0;

namespace bsattn {

namespace {
constexpr size_t kFakeFwd = 4096, kFakeBwd = 8192;
unsigned char g_scratch[1 << 16];
}  // namespace

int launch_layout_rowptr(bsattn_layout*, hipStream_t) { return BSATTN_OK; }
int launch_layout_build(bsattn_layout*, hipStream_t) { return BSATTN_OK; }

size_t fwd_workspace_bytes(const bsattn_layout*, int, int) { return kFakeFwd; }
size_t fwd_workspace_bytes_dt(const bsattn_layout*, int, bsattn_dtype, int) { return kFakeFwd; }
size_t bwd_workspace_bytes(const bsattn_layout*, int, int) { return kFakeBwd; }
size_t lf_workspace_bytes(const lfattn_plan*, int, int, int) { return kFakeFwd; }
size_t lf_bwd_workspace_bytes(const lfattn_plan*, int, int, int) { return kFakeBwd; }

int launch_fwd(const bsattn_layout*, int, bsattn_dtype, int, float, const void*, const void*,
               const void*, void*, float*, void*, void* ws, hipStream_t stream) {
  ProfScope prof_("fake_fwd", stream);
  if (g_fake_overrun) std::memset(static_cast<char*>(ws) + kFakeFwd, 0, g_fake_overrun);
  return BSATTN_OK;
}

int launch_bwd(const bsattn_layout*, int, int, float, const void*, const void*, const void*,
               const void*, const void*, const float*, const void*, void*, void*, void*, void*,
               hipStream_t stream) {
  ProfScope prof_("fake_bwd", stream);
  return BSATTN_OK;
}

int launch_lf_fwd(const lfattn_plan*, int, int, int, float, const void*, const void*, const void*,
                  const void*, const void*, const void*, void*, float*, void*, void*,
                  hipStream_t) {
  return BSATTN_OK;
}

int launch_lf_bwd(const lfattn_plan*, int, int, int, float, const void*, const void*, const void*,
                  const void*, const void*, const void*, const void*, const void*, const float*,
                  const void*, void*, void*, void*, void*, void*, void*, void*, hipStream_t) {
  return BSATTN_OK;
}

int noalloc_scratch(void** out) {
  *out = g_scratch;
  return BSATTN_OK;
}

size_t noalloc_scratch_bytes() { return sizeof(g_scratch); }

}  // namespace bsattn
