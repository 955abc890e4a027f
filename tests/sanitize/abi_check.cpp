// Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
// library's host code (eviction_fed_weight_amd/csrc/tc_api.hip), run by
// tests/test_sanitizers.py on the host only.  It exercises every check the C
// ABI makes before it touches a device: workspace sizes over many shapes,
// bad shapes, null and overlapping pointers, short workspaces, each entry
// point's rejection codes and the status query's validation.  The kernel
// launchers are replaced by stubs that abort, so a call that passed
// validation by mistake fails loudly instead of reaching a GPU.  Exit
// status 0 and the line "ok" on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/tc.h"
#include "../../eviction_fed_weight_amd/csrc/tc_launch.h"

namespace tck {
[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "validation let a call through to %s\n", what);
  abort();
}
hipError_t launch_continue_prep(const ContArgs&, hipStream_t) { reached("launch_continue_prep"); }
hipError_t launch_continue_finish(const ContArgs&, hipStream_t) { reached("launch_continue_finish"); }
hipError_t launch_delta_memory(const DeltaArgs&, int, bool, hipStream_t) { reached("launch_delta_memory"); }
hipError_t launch_forward_bf16(const FwdArgs&, int, hipStream_t) { reached("launch_forward_bf16"); }
hipError_t launch_forward_f32(const FwdArgs&, int, hipStream_t) { reached("launch_forward_f32"); }
hipError_t launch_forward_rows(const FwdArgs&, int, bool, hipStream_t) { reached("launch_forward_rows"); }
hipError_t launch_decode(const DecArgs&, int, bool, hipStream_t) { reached("launch_decode"); }
hipError_t launch_backward_bf16(const BwdArgs&, int, hipStream_t) { reached("launch_backward_bf16"); }
hipError_t launch_backward_f32(const BwdArgs&, int, hipStream_t) { reached("launch_backward_f32"); }
}  // namespace tck

static int fails = 0;
#define EXPECT(cond)                                          \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "line %d: %s\n", __LINE__, #cond);      \
      ++fails;                                                \
    }                                                         \
  } while (0)

static void* P(uint64_t x) { return (void*)(uintptr_t)x; }

int main() {
  const uint64_t G = 1ull << 32;  // spacing so the fake buffers never overlap (never dereferenced)
  // workspace sizes: valid shapes give positive, 256-byte multiples; invalid ones 0
  const int Ds[] = {16, 32, 64, 128, 48, 0, -1};
  const int Ts[] = {1, 63, 64, 65, 1000, 32768, 1 << 20, 0};
  const int Ws[] = {1, 8, 100, 4096, 1 << 20, 0};
  for (int D : Ds)
    for (int T : Ts)
      for (int W : Ws)
        for (int dt = 0; dt < 3; ++dt) {
          tc_shape_t s = {3, 5, T, D, W, 64, 0.0f, dt};
          const size_t f = tc_forward_workspace_size(&s), b = tc_backward_workspace_size(&s);
          const bool valid = (D == 16 || D == 32 || D == 64 || D == 128) && T >= 1 && W >= 1 && dt < 2 &&
                             (long long)(T + 128) * D * (dt ? 2 : 4) < (1ll << 31);
          EXPECT(valid ? (f > 0 && f % 256 == 0 && b > 0 && b % 256 == 0) : (f == 0 && b == 0));
          for (int64_t pos0 : {0ll, 1ll, 99ll, 1000000000007ll, -5ll}) {
            const size_t c = tc_continue_workspace_size(&s, pos0);
            EXPECT((valid && pos0 >= 0 && (long long)T + (pos0 < W ? pos0 : W) < (1ll << 30)) ? true : c == 0);
          }
        }
  EXPECT(tc_forward_workspace_size(nullptr) == 0 && tc_backward_workspace_size(nullptr) == 0);
  EXPECT(tc_continue_workspace_size(nullptr, 0) == 0);

  tc_shape_t ok = {2, 4, 1024, 64, 256, 64, 0.0f, TC_BF16};
  const size_t need = tc_forward_workspace_size(&ok);
  void *q = P(G), *k = P(2 * G), *v = P(3 * G), *y = P(5 * G), *ws = P(7 * G);
  float *lam = (float*)P(4 * G), *eta = (float*)P(4 * G + 256), *gate = (float*)P(4 * G + 512);
  float *A = (float*)P(6 * G), *lse = (float*)P(6 * G + (1 << 24));
  // forward
  EXPECT(tc_forward(nullptr, q, k, v, lam, eta, gate, y, A, lse, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward(&ok, nullptr, k, v, lam, eta, gate, y, A, lse, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward(&ok, q, k, v, lam, eta, gate, nullptr, A, lse, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward(&ok, q, k, v, lam, eta, gate, q, A, lse, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward(&ok, q, k, v, lam, eta, gate, y, A, lse, nullptr, 0, nullptr) == TC_ERR_WORKSPACE);
  EXPECT(tc_forward(&ok, q, k, v, lam, eta, gate, y, A, lse, ws, need - 1, nullptr) == TC_ERR_WORKSPACE);
  EXPECT(tc_forward(&ok, q, k, v, lam, eta, gate, y, A, lse, P(5 * G + 64), need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  tc_shape_t bad = ok;
  bad.D = 48;
  EXPECT(tc_forward(&bad, q, k, v, lam, eta, gate, y, A, lse, ws, need, nullptr) == TC_ERR_UNSUPPORTED);
  bad = ok;
  bad.scale = __builtin_nanf("");
  EXPECT(tc_forward(&bad, q, k, v, lam, eta, gate, y, A, lse, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.B = 1 << 20;
  bad.H = 1 << 10;
  EXPECT(tc_forward(&bad, q, k, v, lam, eta, gate, y, A, lse, ws, need, nullptr) == TC_ERR_UNSUPPORTED);
  // status query
  EXPECT(tc_forward_status(&ok, 0, nullptr, 0, nullptr) == TC_ERR_WORKSPACE);
  EXPECT(tc_forward_status(&ok, 0, ws, need - 1, nullptr) == TC_ERR_WORKSPACE);
  EXPECT(tc_forward_status(&ok, -1, ws, need, nullptr) == TC_ERR_INVALID_ARGUMENT);
  // backward
  const size_t bneed = tc_backward_workspace_size(&ok);
  void *dq = P(8 * G), *dk = P(9 * G), *dv = P(10 * G), *dy = P(11 * G);
  float *dl = (float*)P(12 * G), *de = (float*)P(12 * G + 256), *dg = (float*)P(12 * G + 512);
  EXPECT(tc_backward(&ok, q, k, v, y, dy, lse, lam, eta, gate, dq, dk, dv, dl, de, dg, nullptr, 0, nullptr) ==
         TC_ERR_WORKSPACE);
  EXPECT(tc_backward(&ok, q, k, v, y, dy, lse, lam, eta, gate, dq, dk, dv, dl, de, nullptr, ws, bneed, nullptr) ==
         TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_backward(&ok, q, k, v, y, dy, lse, lam, eta, gate, dq, q, dv, dl, de, dg, ws, bneed, nullptr) ==
         TC_ERR_INVALID_ARGUMENT);
  // decode
  tc_decode_shape_t ds = {4, 8, 128, 4096, 0.0f, TC_BF16};
  int64_t* pos = (int64_t*)P(13 * G);
  EXPECT(tc_decode_step(&ds, q, k, v, P(14 * G), P(15 * G), A, pos, lam, eta, gate, nullptr, nullptr) ==
         TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_decode_step(&ds, q, k, v, P(14 * G), P(14 * G + 64), A, pos, lam, eta, gate, y, nullptr) ==
         TC_ERR_INVALID_ARGUMENT);
  tc_decode_shape_t dbig = {1, 1, 128, 1 << 23, 0.0f, TC_BF16};
  EXPECT(tc_decode_step(&dbig, q, k, v, P(14 * G), P(15 * G), A, pos, lam, eta, gate, y, nullptr) ==
         TC_ERR_UNSUPPORTED);
  // continuation
  const size_t cneed = tc_continue_workspace_size(&ok, 300);
  EXPECT(tc_forward_continue(&ok, 300, q, k, v, lam, eta, gate, P(14 * G), P(15 * G), A, pos, y, lse, ws,
                             cneed - 1, nullptr) == TC_ERR_WORKSPACE);
  EXPECT(tc_forward_continue(&ok, 300, q, k, v, lam, eta, gate, P(14 * G), P(15 * G), A, pos, P(5 * G + 8), lse, ws,
                             cneed, nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward_continue(&ok, -3, q, k, v, lam, eta, gate, P(14 * G), P(15 * G), A, pos, y, lse, ws, cneed,
                             nullptr) == TC_ERR_INVALID_ARGUMENT);
  EXPECT(tc_forward_continue(&ok, 300, q, k, v, lam, eta, gate, k, P(15 * G), A, pos, y, lse, ws, cneed, nullptr) ==
         TC_ERR_INVALID_ARGUMENT);
  for (int st = -1; st < 8; ++st) EXPECT(tc_status_string((tc_status_t)st) != nullptr);
  EXPECT(tc_version() != nullptr);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
