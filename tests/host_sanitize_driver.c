/*
 * Drives the host side of libgmla (argument validation, kernel choice, launch) through
 * every C entry point, built with AddressSanitizer and UndefinedBehaviorSanitizer on
 * the host pass only.  Runs without a GPU: calls that pass validation must come back
 * GMLA_ERR_HIP from the failed launch.  Exit status 0 = all checks held and the
 * sanitizers found nothing.  Test infrastructure: built by tests/test_host_sanitized.py.
 */
#include <stdint.h>
#include <stdio.h>

#include "gmla.h"

static int failures = 0;
#define EXPECT(call, want)                                                      \
  do {                                                                          \
    const int got_ = (call);                                                    \
    if (got_ != (want)) {                                                       \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
              got_, (want));                                                    \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main(void) {
  void* F = (void*)(uintptr_t)(1 << 20); /* aligned, never dereferenced */
  const int64_t bad_strides[3] = {8 * 256, 256 + 4, 128};
  const int64_t neg_strides[3] = {-1, 256, 128};
  /* prefill */
  EXPECT(gmla_attend_prefill(GMLA_BF16, 0, 8, 2, 128, 0.1f, 1, F, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 2, F, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.0f, 1, F, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 1, 0, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 1, F, F, F, bad_strides, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 1, F, F, F, neg_strides, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 96, 0.1f, 1, F, F, F, 0, 0, F, 0), GMLA_ERR_UNSUPPORTED);
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 1, F, F, F, 0, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_prefill(GMLA_F32, 1, 8, 2, 64, 0.1f, 0, F, F, F, 0, 0, F, 0), GMLA_ERR_HIP);
  /* chunk */
  EXPECT(gmla_attend_chunk(GMLA_BF16, 1, 9, 8, 2, 128, 0.1f, 1, F, 0, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_chunk(GMLA_BF16, 1, 0, 8, 2, 128, 0.1f, 1, F, 0, F, F, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_chunk(GMLA_BF16, 1, 3, 8, 2, 128, 0.1f, 1, F, 0, F, F, 0, 0, F, 0), GMLA_ERR_HIP);
  /* decode */
  EXPECT(gmla_decode_workspace_bytes(2, 4, 100, 128, 4), (int)(2 * 4 * 4 * 130 * 4));
  EXPECT(gmla_attend_decode(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, 0, F, 0, 0, 4, 0), GMLA_ERR_WORKSPACE);
  EXPECT(gmla_attend_decode(GMLA_BF16, 2, 4, 100, 48, 0.1f, F, F, F, 0, 0, F, 0, 0, 1, 0), GMLA_ERR_UNSUPPORTED);
  EXPECT(gmla_attend_decode(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, 0, F, 0, 0, -1, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_decode(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, 0, F, 0, 0, 1, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_decode(GMLA_F32, 2, 4, 5000, 128, 0.1f, F, F, F, 0, 0, F, F, 1 << 20, 4, 0), GMLA_ERR_HIP);
  /* projections */
  EXPECT(gmla_linear(GMLA_BF16, 4, 4, 12, F, F, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_linear(GMLA_BF16, 64, 64, 64, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_linear(GMLA_BF16, 2048, 12288, 128, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_linear(GMLA_F32, 3, 5, 7, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_latent_expand(GMLA_BF16, 4, 8, 16, F, 0, F, F, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_latent_expand(GMLA_BF16, 64, 64, 128, F, F, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_gate_out(GMLA_BF16, 4, 16, 0, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_gate_out(GMLA_BF16, 64, 128, F, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_gate_out(GMLA_BF16, 64, 128, F, F, 0, F, 0), GMLA_ERR_HIP);
  if (gmla_status_string(GMLA_ERR_HIP)[0] != 'G') ++failures;
  printf("host sanitized run: %d failures\n", failures);
  return failures != 0;
}
