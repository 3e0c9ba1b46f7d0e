// Host-side driver for the sanitizer build of the C ABI: every entry point
// with arguments its checks must refuse on the host, and the host-only model
// queries over their ranges.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only; run without a GPU, where
// an accepted call stops at the device check (ATTN_E_DEVICE).  Prints one
// line per failed expectation and exits non-zero if there was any.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/attnio.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static void* P(uintptr_t x) { return (void*)x; }

int main() {
  const uintptr_t G = 1ull << 30;
  // forward: every argument check, both precisions
  for (int f32 = 0; f32 < 2; ++f32) {
    auto fwd = f32 ? attn_fwd_f32 : attn_fwd;
    EXPECT(fwd(nullptr, P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, 0.125f, 0, nullptr, nullptr) == ATTN_E_NULL);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 96, 0.125f, 0, nullptr, nullptr) == ATTN_E_HEAD_DIM);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 0, 1, 16, 64, 0.125f, 0, nullptr, nullptr) == ATTN_E_SHAPE);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 1 << 12, 1 << 12, 1 << 12, 64, 0.125f, 0, nullptr, nullptr) ==
           ATTN_E_SHAPE);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 0x7fffffff, 0x7fffffff, 0x7fffffff, 128, 0.125f, 0, nullptr,
               nullptr) == ATTN_E_SHAPE);
    EXPECT(fwd(P(G + 8), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, 0.125f, 0, nullptr, nullptr) == ATTN_E_ALIGN);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(G + 64), 1, 1, 16, 64, 0.125f, 0, nullptr, nullptr) == ATTN_E_ALIAS);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, __builtin_nanf(""), 0, nullptr, nullptr) ==
           ATTN_E_ARG);
    EXPECT(fwd(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, 0.125f, 0, nullptr, nullptr) == ATTN_E_DEVICE);
  }
  float* lse = (float*)P(5 * G);
  EXPECT(attn_fwd_lse(P(G), P(2 * G), P(3 * G), P(4 * G), nullptr, 1, 1, 16, 64, 0.1f, 0, nullptr, nullptr) ==
         ATTN_E_NULL);
  EXPECT(attn_fwd_lse(P(G), P(2 * G), P(3 * G), P(4 * G), (float*)P(G + 4), 1, 1, 16, 64, 0.1f, 0, nullptr,
                      nullptr) == ATTN_E_ALIAS);
  EXPECT(attn_fwd_f32_lse(P(G), P(2 * G), P(3 * G), P(4 * G), lse, 1, 1, 16, 64, 0.1f, 1, nullptr, nullptr) ==
         ATTN_E_DEVICE);
  // explicit tilings
  const int nt = attn_tiling_count();
  EXPECT(nt >= 2);
  attn_tiling t;
  for (int i = -3; i < nt + 3; ++i) {
    const int rc = attn_tiling_get(i, &t);
    EXPECT((i >= 0 && i < nt) ? rc == ATTN_OK : rc == ATTN_E_ARG);
    const int d = (i >= 0 && i < nt) ? t.d : 64;
    const int rf = attn_fwd_tiled(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, d, 0.1f, 0, nullptr, i, nullptr);
    EXPECT((i >= 0 && i < nt) ? rf == ATTN_E_DEVICE : rf == ATTN_E_ARG);
  }
  EXPECT(attn_tiling_get(0, nullptr) == ATTN_E_NULL);
  // backward, with and without a workspace
  const uintptr_t bw[10] = {G, 2 * G, 3 * G, 4 * G, 5 * G, 6 * G, 7 * G, 8 * G, 9 * G, 10 * G};
  EXPECT(attn_bwd(P(bw[0]), P(bw[1]), P(bw[2]), P(bw[3]), P(bw[4]), (float*)P(bw[5]), P(bw[6]), P(bw[7]),
                  P(bw[8]), nullptr, 1, 1, 16, 64, 0.1f, 0, nullptr, nullptr) == ATTN_E_NULL);
  EXPECT(attn_bwd(P(bw[0]), P(bw[1]), P(bw[2]), P(bw[3]), P(bw[4]), (float*)P(bw[5]), P(bw[6]), P(bw[7]),
                  P(bw[0] + 16), P(bw[9]), 1, 1, 16, 64, 0.1f, 0, nullptr, nullptr) == ATTN_E_ALIAS);
  EXPECT(attn_bwd(P(bw[0]), P(bw[1]), P(bw[2]), P(bw[3]), P(bw[4]), (float*)P(bw[5]), P(bw[6]), P(bw[7]),
                  P(bw[8]), P(bw[9]), 1, 1, 16, 64, 0.1f, 0, nullptr, nullptr) == ATTN_E_DEVICE);
  EXPECT(attn_bwd_noalloc(P(bw[0]), P(bw[1]), P(bw[2]), P(bw[3]), P(bw[4]), (float*)P(bw[5]), P(bw[6]),
                          P(bw[7]), P(bw[8]), 1, 4097, 1024, 64, 0.1f, 0, nullptr, nullptr) == ATTN_E_SCRATCH);
  EXPECT(attn_bwd_noalloc(P(bw[0]), P(bw[1]), P(bw[2]), P(bw[3]), nullptr, (float*)P(bw[5]), P(bw[6]), P(bw[7]),
                          P(bw[8]), 1, 4097, 1024, 64, 0.1f, 0, nullptr, nullptr) == ATTN_E_NULL);
  EXPECT(attn_bwd_workspace_bytes(0x7fffffff, 0x7fffffff, 0x7fffffff) > 0);
  EXPECT(attn_bwd_workspace_bytes(-1, 1, 1) == 0);
  // unfused, fp8, row operators
  EXPECT(attn_fwd_unfused(P(G), P(2 * G), P(3 * G), P(4 * G), P(5 * G), 10, 1, 1, 16, 64, 0.1f, 0, nullptr,
                          nullptr) == ATTN_E_ARG);
  EXPECT(attn_fwd_unfused_workspace_bytes(0x7fffffff) > 0);
  EXPECT(attn_fwd_fp8(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, 0.1f, 1e30f, 1e30f, 1.f, 0, nullptr,
                      nullptr) == ATTN_E_ARG);
  EXPECT(attn_fwd_fp8(P(G), P(2 * G), P(3 * G), P(4 * G), 1, 1, 16, 64, 0.1f, 0.f, 1.f, 1.f, 0, nullptr,
                      nullptr) == ATTN_E_ARG);
  EXPECT(stream_softmax(P(G), P(G + 16), 4, 1024, 1.f, nullptr) == ATTN_E_ALIAS);
  EXPECT(stream_layernorm(P(G), P(3 * G), nullptr, P(2 * G), 1 << 20, 1 << 20, 1e-5f, nullptr) == ATTN_E_SHAPE);
  EXPECT(stream_rows_cached(0x7fffffff) == 0 && stream_rows_cached(-4) == 0);
  // host-only queries over their ranges
  for (int code = -20; code <= 5; ++code) EXPECT(attn_strerror(code) != nullptr && strlen(attn_strerror(code)) > 0);
  int bm = 0, bn = 0, st = 0;
  for (int d : {0, 32, 64, 96, 128, 256})
    for (int dtype = -1; dtype <= 3; ++dtype)
      for (int causal = 0; causal < 2; ++causal) {
        const int rc = attn_query_tiling(d, dtype, causal, &bm, &bn, &st);
        EXPECT(rc == ATTN_OK || rc == ATTN_E_HEAD_DIM || rc == ATTN_E_ARG);
        EXPECT(attn_query_tiling(d, dtype, causal, nullptr, nullptr, nullptr) == rc);
      }
  attn_tiling_eval ev[300];
  for (int d : {64, 128}) {
    const int n = attn_tiling_enumerate(d, ATTN_DTYPE_BF16, 1, ev, 300);
    EXPECT(n > 0 && n <= 300);
    EXPECT(attn_tiling_enumerate(d, ATTN_DTYPE_BF16, 0, ev, 1) == n);   // writes one, returns all
    EXPECT(attn_tiling_enumerate(d, ATTN_DTYPE_BF16, 0, nullptr, 0) == n);
    EXPECT(attn_tiling_enumerate(d, ATTN_DTYPE_F32, 0, ev, 300) == ATTN_E_ARG);
  }
  EXPECT(attn_tiling_enumerate(64, ATTN_DTYPE_BF16, 0, nullptr, 5) == ATTN_E_NULL);
  double a = 0, b = 0, c = 0, out[5];
  int32_t kv[4] = {-7, 0, 1 << 30, 513};
  EXPECT(attn_io_bound_bytes(4, 3, 1000, 128, ATTN_DTYPE_BF16, 1, kv, &a, &b, &c) == ATTN_OK && a > 0);
  EXPECT(attn_io_bound_bytes(1, 1, (1 << 24) - 1, 128, ATTN_DTYPE_FP8, 1, nullptr, &a, &b, &c) == ATTN_OK);
  EXPECT(attn_io_bound_bytes(1 << 20, 1 << 20, 1 << 20, 64, ATTN_DTYPE_BF16, 0, nullptr, &a, &b, &c) == ATTN_E_SHAPE);
  EXPECT(attn_io_model(4, 3, 1000, 64, 4, 0, kv, out) == ATTN_OK && out[4] > 0);
  EXPECT(attn_io_model(4, 3, 1000, 64, 3, 0, kv, out) == ATTN_E_ARG);
  EXPECT(attn_io_model(4, 3, 1000, 64, 2, 0, kv, nullptr) == ATTN_E_NULL);
  EXPECT(attn_version() > 0);
  if (failures) return 1;
  printf("abi driver: all checks passed\n");
  return 0;
}
