// Host-side checks of libkmip's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (the library sources compiled
// host-only).  Workspace sizes over a grid of shapes; every class of invalid
// argument, which must be refused before any HIP call; and, only when no GPU
// is present, valid calls with stand-in pointers, which validate, lay out
// the workspace and then fail to launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "kmip.h"

static int failures = 0;

static void expect(bool ok, const char* what, long a = 0, long b = 0) {
  if (!ok) {
    std::printf("FAIL %s (%ld, %ld)\n", what, a, b);
    ++failures;
  }
}

int main() {
  void* F = reinterpret_cast<void*>(uintptr_t(1) << 20);   // aligned, never dereferenced
  int32_t* Fi = static_cast<int32_t*>(F);
  float* Ff = static_cast<float*>(F);

  // Workspace sizes: positive for valid shapes, zero for invalid ones, the
  // fp32 forward at least the bf16 one, and growth with N.
  const int64_t Ns[] = {1, 7, 31, 32, 33, 1000, 8191, 32768, 100000, 500000};
  const int Hs[] = {1, 2, 3, 4, 8};
  const int ds[] = {32, 64};
  const int ks[] = {1, 5, 15, 16, 17, 45, 64};
  const int Bs[] = {0, 1, 3, 64};
  for (int64_t N : Ns)
    for (int H : Hs)
      for (int d : ds)
        for (int k : ks)
          for (int B : Bs) {
            const size_t f = kmip_forward_workspace_bytes(N, H, d, k, B);
            const size_t f32 = kmip_forward_f32_workspace_bytes(N, H, d, k, B);
            const size_t b = kmip_backward_workspace_bytes(N, H, d, k, B);
            expect(f > 0 && b > 0 && f32 > 0, "sizes of a valid shape", (long)N, k);
            // one graph, lists of at most 16: the pruned selection's buffers
            // (about 2d + 5 bytes per row) are held up to N = 2^19 only
            const bool prune_edge = B <= 1 && k <= 16 && N <= (1 << 19) && 2 * N > (1 << 19);
            if (!prune_edge)
              expect(kmip_forward_workspace_bytes(2 * N, H, d, k, B) >= f, "forward grows", (long)N, k);
            expect(kmip_backward_workspace_bytes(2 * N, H, d, k, B) >= b, "backward grows", (long)N, k);
          }
  expect(kmip_forward_workspace_bytes(0, 4, 32, 15, 0) == 0, "N = 0");
  expect(kmip_forward_workspace_bytes(10, 4, 48, 15, 0) == 0, "d = 48");
  expect(kmip_backward_workspace_bytes(10, 4, 32, 65, 0) == 0, "k = 65");
  expect(kmip_forward_workspace_bytes(int64_t(1) << 30, 4, 32, 15, 0) == 0, "N H k too large");

  // Invalid arguments.
  const size_t big = size_t(1) << 40;
  auto fwd = [&](void* q, int64_t N, int H, int d, int k, const int32_t* offs, int B, void* ws,
                 size_t wsb) {
    return kmip_forward(q, F, F, N, H, d, k, offs, B, Ff, Fi, Ff, ws, wsb, nullptr);
  };
  expect(fwd(nullptr, 128, 2, 32, 15, nullptr, 0, F, big) == KMIP_ERR_INVALID_VALUE, "null q");
  expect(fwd(F, 0, 2, 32, 15, nullptr, 0, F, big) == KMIP_ERR_INVALID_VALUE, "N = 0");
  expect(fwd(F, 128, 2, 32, 15, nullptr, 3, F, big) == KMIP_ERR_INVALID_VALUE, "B without offsets");
  expect(fwd(F, 128, 2, 32, 15, nullptr, -1, F, big) == KMIP_ERR_INVALID_VALUE, "B < 0");
  expect(fwd(static_cast<char*>(F) + 8, 128, 2, 32, 15, nullptr, 0, F, big) ==
             KMIP_ERR_INVALID_VALUE, "misaligned q");
  expect(fwd(F, 128, 2, 48, 15, nullptr, 0, F, big) == KMIP_ERR_UNSUPPORTED, "d = 48");
  expect(fwd(F, 128, 2, 32, 0, nullptr, 0, F, big) == KMIP_ERR_UNSUPPORTED, "k = 0");
  expect(fwd(F, 128, 2, 32, 65, nullptr, 0, F, big) == KMIP_ERR_UNSUPPORTED, "k = 65");
  expect(fwd(F, 128, 2, 32, 15, nullptr, 0, nullptr, 0) == KMIP_ERR_WORKSPACE, "no workspace");
  expect(fwd(F, 128, 2, 32, 15, nullptr, 0, F, 1020) == KMIP_ERR_WORKSPACE, "small workspace");
  expect(fwd(F, 128, 2, 32, 15, nullptr, 0, static_cast<char*>(F) + 8, big) ==
             KMIP_ERR_INVALID_VALUE, "misaligned workspace");
  auto bwd = [&](int64_t N, int d, int k, void* ws, size_t wsb, float* dq) {
    return kmip_backward(F, F, F, N, 2, d, k, nullptr, 0, Fi, Ff, Ff, dq, Ff, Ff, ws, wsb,
                         nullptr);
  };
  expect(bwd(128, 32, 15, F, big, nullptr) == KMIP_ERR_INVALID_VALUE, "null dq");
  expect(bwd(-5, 32, 15, F, big, Ff) == KMIP_ERR_INVALID_VALUE, "N < 0");
  expect(bwd(128, 16, 15, F, big, Ff) == KMIP_ERR_UNSUPPORTED, "d = 16");
  expect(bwd(128, 32, 100, F, big, Ff) == KMIP_ERR_UNSUPPORTED, "k = 100");
  expect(bwd(128, 32, 15, nullptr, big, Ff) == KMIP_ERR_WORKSPACE, "no workspace");
  expect(bwd(128, 32, 15, F, 100, Ff) == KMIP_ERR_WORKSPACE, "small workspace");
  expect(bwd(128, 32, 15, static_cast<char*>(F) + 16, big, Ff) == KMIP_ERR_INVALID_VALUE,
         "misaligned backward workspace");
  expect(kmip_forward_no_workspace(F, F, F, 4000000, 4, 32, 15, nullptr, 0, Ff, Fi, Ff,
                                   nullptr) == KMIP_ERR_WORKSPACE,
         "no-workspace forward beyond the scratch");
  expect(kmip_forward_no_workspace(nullptr, F, F, 1000, 4, 32, 15, nullptr, 0, Ff, Fi, Ff,
                                   nullptr) == KMIP_ERR_INVALID_VALUE,
         "no-workspace forward, null q");
  expect(kmip_status_string(KMIP_OK) != nullptr && kmip_version() >= 10000, "strings");

  // Valid calls reach the workspace layout and the launches; run them only
  // where there is no GPU (the stand-in pointers must never be dereferenced).
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    const int64_t shapes[][4] = {{128, 2, 32, 15}, {100000, 4, 32, 15}, {5000, 4, 64, 45},
                                 {33, 1, 32, 64}};
    for (auto& sh : shapes) {
      const int64_t N = sh[0];
      const int H = (int)sh[1], d = (int)sh[2], k = (int)sh[3];
      kmip_status_t st = kmip_forward(F, F, F, N, H, d, k, nullptr, 0, Ff, Fi, Ff, F, big, nullptr);
      expect(st == KMIP_ERR_LAUNCH, "forward without a GPU", (long)N, st);
      st = kmip_backward(F, F, F, N, H, d, k, nullptr, 0, Fi, Ff, Ff, Ff, Ff, Ff, F, big, nullptr);
      expect(st == KMIP_ERR_LAUNCH, "backward without a GPU", (long)N, st);
      st = kmip_forward_f32(Ff, Ff, Ff, N, H, d, k, nullptr, 0, Ff, Fi, Ff, F, big, nullptr);
      expect(st == KMIP_ERR_LAUNCH, "fp32 forward without a GPU", (long)N, st);
    }
    std::printf("valid calls checked without a GPU\n");
  }
  std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
