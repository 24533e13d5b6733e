// Host-logic checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer from a host-only compile of the library's
// sources (no device code): argument validation, workspace sizing and
// offsets, error strings, the timing switches, and the mapping of a failing
// HIP runtime call to NYS_EHIP.  It runs where no GPU is visible, so every
// call that passes validation fails at its first HIP call (the stream-ordered
// workspace allocation, or the launch) and nothing reaches a device.
// Exit status 0 when every expectation holds; the sanitizers abort on the
// first defect they see.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nystrom.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main() {
  // Fake device addresses: never dereferenced on the host, and with no GPU
  // visible no kernel runs.
  void* P = reinterpret_cast<void*>(uintptr_t(0x10000));
  const float* W = reinterpret_cast<const float*>(P);
  const int ds[] = {16, 32, 64, 128, 24, 0, -1};
  const int ms[] = {1, 8, 33, 64, 65, 128, 256, 257, 0};
  const int ns[] = {1, 64, 100, 8191, 8192, 1 << 24, (1 << 24) + 1};
  // Workspace sizes and offsets over a grid of shapes, valid and not.
  for (int d : ds)
    for (int m : ms)
      for (int n : ns) {
        const size_t ws = nystrom_attn_workspace_bytes(2, 3, n, d, m);
        const bool ok = (d == 16 || d == 32 || d == 64 || d == 128) && m >= 1 && m <= 256 && m <= n &&
                        n <= (1 << 24) && (long long)n * d < (1LL << 29);
        EXPECT((ws > 0) == ok);
        for (int which = -1; which <= NYS_WS_COUNT; ++which) {
          const long long off = nystrom_attn_workspace_offset(which, 2, 3, n, d, m);
          if (!ok || which < 0 || which >= NYS_WS_COUNT) {
            EXPECT(off == -1);
          } else {
            EXPECT(off >= 0 && off % 256 == 0 && (size_t)off < ws);
          }
        }
        (void)nystrom_attn_bwd_workspace_bytes(2, 3, n, d, m, 6, 33);
        (void)nystrom_layer_workspace_bytes(2, 3, n, d, m, NYS_BF16);
        (void)nystrom_attn_error_workspace_bytes(2, 3, n, d, m, NYS_F32);
      }
  // Validation: every invalid call returns its code and launches nothing.
  EXPECT(nystrom_attn_fwd(nullptr, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EINVAL);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 16, 129, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EINVAL);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 16, 8, 1, -1, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EINVAL);
  EXPECT(nystrom_attn_fwd(P, P, P, W, 128, 16, 8, 1, 6, P, 1, 4, NYS_F32, nullptr, 0, nullptr) == NYS_EINVAL);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, 7, nullptr, 0, nullptr) == NYS_EINVAL);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 24, 8, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EUNSUPPORTED);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 512, 16, 300, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EUNSUPPORTED);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, P, 16, nullptr) == NYS_EWORKSPACE);
  EXPECT(nystrom_attn_bwd(P, P, P, nullptr, P, 128, 16, 80, 1, 6, P, P, P, nullptr, 1, 0, NYS_F32, nullptr, 0,
                          nullptr) == NYS_EUNSUPPORTED);
  EXPECT(nystrom_attn_fwd_save(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EINVAL);
  EXPECT(nystrom_dconv_fwd(P, nullptr, 128, 16, 1, 1, 3, NYS_F32, P, nullptr) == NYS_EINVAL);
  EXPECT(nystrom_dconv_fwd(P, W, 128, 16, 1, 1, 2, NYS_F32, P, nullptr) == NYS_EINVAL);
  EXPECT(nystrom_attn_fwd_noalloc(P, P, P, nullptr, 32768, 128, 256, 12, 8, P, 8, 0, NYS_BF16, nullptr) ==
         NYS_EWORKSPACE);  // beyond NYS_NOALLOC_SCRATCH_BYTES
  EXPECT(nystrom_attn_fwd_noalloc(P, nullptr, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, nullptr) ==
         NYS_EINVAL);
  // Valid calls: with no device the first HIP call fails -> NYS_EHIP.
  EXPECT(nystrom_attn_fwd_noalloc(P, P, P, W, 128, 16, 8, 1, 6, P, 1, 3, NYS_F32, nullptr) == NYS_EHIP);
  EXPECT(nystrom_attn_fwd(P, P, P, W, 128, 16, 8, 1, 6, P, 1, 3, NYS_F32, nullptr, 0, nullptr) == NYS_EHIP);
  EXPECT(nystrom_attn_fwd(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_BF16, P, size_t(1) << 30, nullptr) ==
         NYS_EHIP);
  EXPECT(nystrom_attn_fwd_masked(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, nullptr, nullptr, 0,
                                 nullptr) == NYS_EHIP);
  EXPECT(nystrom_attn_bwd(P, P, P, W, P, 128, 16, 8, 1, 6, P, P, P, nullptr, 1, 3, NYS_F32, nullptr, 0, nullptr) ==
         NYS_EHIP);
  EXPECT(nystrom_layer_fwd(P, P, P, nullptr, 128, 16, 8, 1, 6, P, 1, 0, NYS_F32, nullptr, 0, nullptr) == NYS_EHIP);
  EXPECT(nystrom_attn_error(P, P, P, 128, 16, 8, 1, 6, reinterpret_cast<float*>(P), 1, NYS_F32, nullptr, 0,
                            nullptr) == NYS_EHIP);
  EXPECT(nystrom_dconv_fwd(P, W, 128, 16, 1, 1, 3, NYS_F32, P, nullptr) == NYS_EHIP);
  // Strings, version, timing switches.
  for (int code = -6; code <= 1; ++code) EXPECT(nystrom_strerror(code) && strlen(nystrom_strerror(code)) > 0);
  EXPECT(nystrom_abi_version() >= 100);
  EXPECT(nystrom_timing_enable(1) == 0);
  EXPECT(nystrom_timing_enable(0) == 1);
  const char* names[4];
  double total_ms[4];
  long long launches[4];
  EXPECT(nystrom_timing_read(4, names, total_ms, launches) >= 0);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
