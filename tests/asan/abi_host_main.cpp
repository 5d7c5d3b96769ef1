// Drives every entry point of the C ABI through its host code, with the stand-in
// runtime of fake_hip.cpp, under AddressSanitizer, LeakSanitizer and UBSan: valid
// calls (handles built, queried, used and destroyed), every class of rejected
// argument, and the BSATTN_DEBUG paths (call and launch log, stream check,
// workspace canary).  Exits non-zero at the first unexpected return code; the
// sanitizers abort on their own findings.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/bsattn.h"

extern size_t g_fake_overrun;

namespace {

int g_fail = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: got %d want %d (%s)\n", what, got, want, bsattn_last_error());
    g_fail = 1;
  }
}

void* dev(size_t bytes) {
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) std::abort();
  return p;
}

void bigbird_calls() {
  const int32_t G[2] = {0, 63};
  bsattn_layout* L = nullptr;
  expect(bsattn_layout_build(4096, 64, 12, G, 2, 3, 3, 7, nullptr, &L), BSATTN_OK, "build");
  int nb = 0, heads = 0;
  int64_t nnz = 0;
  expect(bsattn_layout_info(L, &nb, &heads, &nnz), BSATTN_OK, "info");
  std::vector<int32_t> rp(heads * nb + 1), ci(nnz), cp(heads * nb + 1), cs(nnz);
  expect(bsattn_layout_to_host(L, rp.data(), ci.data(), cp.data(), cs.data()), BSATTN_OK, "to_host");
  expect(bsattn_layout_rebuild(L, 8, nullptr), BSATTN_OK, "rebuild");
  const int B = 2;
  const size_t elems = (size_t)B * 12 * 4096 * 128;
  void* t[12];
  for (auto& p : t) p = dev(elems * 2);
  float* lse = static_cast<float*>(dev((size_t)B * 12 * 4096 * 4));
  const size_t wf = bsattn_fwd_workspace(L, B, 64), wb = bsattn_bwd_workspace(L, B, 64);
  void* ws = dev(wf + wb + 64);
  expect(bsattn_fwd(L, B, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, t[4], ws,
                    wf + 64, nullptr), BSATTN_OK, "fwd");
  expect(bsattn_fwd(L, B, 128, BSATTN_BF16, 0.088f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf, nullptr), BSATTN_OK, "fwd d=128");
  expect(bsattn_fwd(L, B, 128, BSATTN_F32, 0.088f, t[0], t[1], t[2], t[3], lse, nullptr, ws, wf,
                    nullptr), BSATTN_EUNSUPPORTED, "fwd fp32 d=128");
  expect(bsattn_fwd(L, B, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf - 1, nullptr), BSATTN_EINVAL, "fwd short workspace");
  expect(bsattn_fwd(L, B, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2],
                    static_cast<char*>(t[3]) + 2, lse, nullptr, ws, wf, nullptr),
         BSATTN_EINVAL, "fwd misaligned");
  expect(bsattn_fwd(L, B, 64, BSATTN_F32, 0.125f, t[0], t[1], t[2], t[3], lse, t[4], ws, wf,
                    nullptr), BSATTN_EINVAL, "fwd fp32 with o_lo");
  expect(bsattn_bwd(L, B, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], t[4], lse, t[5], t[6],
                    t[7], t[8], ws, wb, nullptr), BSATTN_OK, "bwd");
  expect(bsattn_bwd(L, B, 64, BSATTN_F32, 0.125f, t[0], t[1], t[2], t[3], nullptr, lse, t[5],
                    t[6], t[7], t[8], ws, wb, nullptr), BSATTN_EUNSUPPORTED, "bwd fp32");
  expect(bsattn_bwd_noalloc(L, B, 128, BSATTN_BF16, 0.088f, t[0], t[1], t[2], t[3], nullptr, lse,
                            t[5], t[6], t[7], t[8], nullptr), BSATTN_OK, "bwd_noalloc");
  // a forward that writes past its workspace bytes: the level-2 canary reports it
  g_fake_overrun = 8;
  expect(bsattn_fwd(L, B, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf + 64, nullptr), BSATTN_EHIP, "fwd canary");
  g_fake_overrun = 0;
  if (std::strstr(bsattn_last_error(), "written past") == nullptr) {
    std::fprintf(stderr, "FAIL canary message: %s\n", bsattn_last_error());
    g_fail = 1;
  }
  expect(bsattn_layout_destroy(L), BSATTN_OK, "destroy");
  // a ragged sequence and a layout above 512 blocks (the multi-kernel build)
  const int32_t G2[2] = {0, 15};
  expect(bsattn_layout_build(1000, 64, 2, G2, 2, 3, 3, 1, nullptr, &L), BSATTN_OK, "ragged");
  expect(bsattn_layout_destroy(L), BSATTN_OK, "destroy ragged");
  const int32_t G3[3] = {0, 7, 599};
  expect(bsattn_layout_build(64 * 600, 64, 2, G3, 3, 3, 3, 1, nullptr, &L), BSATTN_OK, "600 blocks");
  expect(bsattn_layout_destroy(L), BSATTN_OK, "destroy 600");
  for (auto& p : t) (void)hipFree(p);
  (void)hipFree(lse);
  (void)hipFree(ws);
}

void bigbird_rejections() {
  struct Case { int n, b, heads; std::vector<int32_t> G; int w, r, code; };
  const Case cases[] = {
      {0, 64, 1, {}, 3, 3, BSATTN_EINVAL},        {500, 64, 1, {8}, 3, 3, BSATTN_EINVAL},
      {512, 32, 1, {0}, 3, 3, BSATTN_EUNSUPPORTED}, {512, 64, 0, {0}, 3, 3, BSATTN_EINVAL},
      {512, 64, 1, {0}, 2, 3, BSATTN_EINVAL},     {512, 64, 1, {0}, 3, -1, BSATTN_EINVAL},
      {512, 64, 1, {0}, 3, 65, BSATTN_EUNSUPPORTED}, {512, 64, 1, {7, 0}, 3, 3, BSATTN_EINVAL},
      {512, 64, 1, {3, 3}, 3, 3, BSATTN_EINVAL},  {64 * 4097, 64, 1, {0}, 3, 3, BSATTN_EUNSUPPORTED},
  };
  for (const Case& c : cases) {
    bsattn_layout* L = reinterpret_cast<bsattn_layout*>(1);
    expect(bsattn_layout_build(c.n, c.b, c.heads, c.G.empty() ? nullptr : c.G.data(),
                               (int)c.G.size(), c.w, c.r, 1, nullptr, &L), c.code, "reject");
    if (L != nullptr) { std::fprintf(stderr, "FAIL handle not cleared\n"); g_fail = 1; }
  }
  expect(bsattn_fwd(nullptr, 1, 64, BSATTN_BF16, 0.1f, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, 0, nullptr), BSATTN_EINVAL, "null layout");
  expect(bsattn_layout_destroy(nullptr), BSATTN_OK, "destroy null");
  expect(bsattn_profile_read(-1, nullptr, nullptr, nullptr, nullptr), BSATTN_EINVAL, "profile");
}

void longformer_calls() {
  std::vector<int32_t> G(64);
  for (int i = 0; i < 64; ++i) G[i] = i;
  lfattn_plan* P = nullptr;
  expect(lfattn_plan_build(4096, 256, G.data(), 64, nullptr, &P), BSATTN_OK, "lf plan");
  const int B = 1, H = 12;
  const size_t elems = (size_t)B * H * 4096 * 64;
  void* t[16];
  for (auto& p : t) p = dev(elems * 2);
  float* lse = static_cast<float*>(dev((size_t)B * H * 4096 * 4));
  const size_t wf = lfattn_fwd_workspace(P, B, H, 64), wb = lfattn_bwd_workspace(P, B, H, 64);
  void* ws = dev(wf + wb + 64);
  expect(lfattn_fwd(P, B, H, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, t[4], ws,
                    wf + 64, nullptr), BSATTN_OK, "lf fwd");
  expect(lfattn_fwd_gproj(P, B, H, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[9], t[10], t[11],
                          t[3], lse, nullptr, ws, wf, nullptr), BSATTN_OK, "lf fwd gproj");
  expect(lfattn_bwd(P, B, H, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], t[4], lse, t[5],
                    t[6], t[7], t[8], ws, wb, nullptr), BSATTN_OK, "lf bwd");
  expect(lfattn_bwd_gproj(P, B, H, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[9], t[10], t[11],
                          t[3], nullptr, lse, t[5], t[6], t[7], t[8], t[12], t[13], t[6], ws, wb,
                          nullptr), BSATTN_EINVAL, "lf bwd gproj aliasing");
  expect(lfattn_fwd(P, B, H, 128, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf, nullptr), BSATTN_OK, "lf d=128");
  expect(lfattn_fwd(P, B, H, 96, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf, nullptr), BSATTN_EUNSUPPORTED, "lf d=96");
  expect(lfattn_bwd(P, B, H, 128, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], t[4], lse, t[5],
                    t[6], t[7], t[8], ws, wb, nullptr), BSATTN_OK, "lf bwd d=128");
  expect(lfattn_plan_destroy(P), BSATTN_OK, "lf destroy");
  // per-head dilation with a causal window; the ETC construction
  const int32_t dil[8] = {3, 3, 0, 0, 0, 0, 0, 0};
  expect(lfattn_plan_build_dilated(23040, 256, nullptr, 0, 8, dil, 1, nullptr, &P), BSATTN_OK,
         "dilated");
  expect(lfattn_fwd(P, 1, 8, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf, nullptr), BSATTN_OK, "dilated fwd");
  expect(lfattn_fwd(P, 1, 7, 64, BSATTN_BF16, 0.125f, t[0], t[1], t[2], t[3], lse, nullptr, ws,
                    wf, nullptr), BSATTN_EINVAL, "dilated head count");
  expect(lfattn_plan_destroy(P), BSATTN_OK, "dilated destroy");
  expect(lfattn_plan_build_etc(256, 4096, 84, 3, nullptr, &P), BSATTN_OK, "etc");
  expect(lfattn_plan_destroy(P), BSATTN_OK, "etc destroy");
  for (auto& p : t) (void)hipFree(p);
  (void)hipFree(lse);
  (void)hipFree(ws);
}

void longformer_rejections() {
  lfattn_plan* P = reinterpret_cast<lfattn_plan*>(1);
  const int32_t bad[2] = {5, 1};
  expect(lfattn_plan_build(512, 16, bad, 2, nullptr, &P), BSATTN_EINVAL, "lf unsorted");
  const int32_t g1[1] = {0};
  const int32_t dil[2] = {0, 1};
  expect(lfattn_plan_build_dilated(512, 8, g1, 1, 2, dil, 1, nullptr, &P), BSATTN_EINVAL,
         "causal with global");
  const int32_t dil_max[1] = {1023};
  expect(lfattn_plan_build_dilated(512, 1 << 21, nullptr, 0, 1, dil_max, 0, nullptr, &P),
         BSATTN_EUNSUPPORTED, "window span");
  expect(lfattn_plan_build_etc(200000, 62145, 84, 3, nullptr, &P), BSATTN_EUNSUPPORTED, "etc size");
  expect(lfattn_plan_build_etc(4, 100, 8, 2, nullptr, &P), BSATTN_EINVAL, "etc even window");
  if (P != nullptr) { std::fprintf(stderr, "FAIL plan not cleared\n"); g_fail = 1; }
  expect(lfattn_plan_destroy(nullptr), BSATTN_OK, "lf destroy null");
}

}  // namespace

int main() {
  setenv("BSATTN_DEBUG", "2", 1);   // read once, at the first call
  if (std::strcmp(bsattn_status_str(BSATTN_EINVAL), "BSATTN_EINVAL") != 0) g_fail = 1;
  if (std::strstr(bsattn_version(), "gfx950") == nullptr) g_fail = 1;
  expect(bsattn_profile_enable(1), BSATTN_OK, "profile on");
  bigbird_rejections();
  bigbird_calls();
  longformer_rejections();
  longformer_calls();
  char names[48 * 8];
  int64_t counts[8];
  double ms[8];
  int nk = -1;
  expect(bsattn_profile_read(8, names, counts, ms, &nk), BSATTN_OK, "profile read");
  expect(bsattn_profile_enable(0), BSATTN_OK, "profile off");
  std::printf("%s\n", g_fail ? "FAILED" : "ok");
  return g_fail;
}
