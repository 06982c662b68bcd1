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

/* from the HIP runtime (libamdhip64), declared here so the driver needs no HIP headers */
int hipGetDeviceCount(int* count);

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
  /* The calls below that pass validation reach a kernel launch with a fake pointer:
   * they may only ever run where no device is visible. */
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == 0 && ndev > 0) {
    printf("skipped: %d HIP device(s) visible\n", ndev);
    return 77;
  }
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
  {
    const int64_t wide[3] = {(int64_t)1 << 30, (int64_t)1 << 24, 128};
    EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 8, 2, 128, 0.1f, 1, F, F, F, wide, 0, F, 0), GMLA_ERR_UNSUPPORTED);
  }
  EXPECT(gmla_attend_prefill(GMLA_BF16, 1, 0x7fffffff, 2, 128, 0.1f, 1, F, F, F, 0, 0, F, 0), GMLA_ERR_UNSUPPORTED);
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
  EXPECT(gmla_attend_decode(GMLA_BF16, 2, 4, 0x7fffffff, 128, 0.1f, F, F, F, 0, 0, F, 0, 0, 1, 0), GMLA_ERR_UNSUPPORTED);
  /* decode without allocation */
  EXPECT(gmla_attend_decode_noalloc(GMLA_BF16, 8, 96, 4096, 128, 0.1f, F, F, F, 0, 0, F, 4096, 0), GMLA_ERR_TOO_LARGE);
  EXPECT(gmla_attend_decode_noalloc(GMLA_BF16, 2, 4, 100, 48, 0.1f, F, F, F, 0, 0, F, 1, 0), GMLA_ERR_UNSUPPORTED);
  EXPECT(gmla_attend_decode_noalloc(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, 0, F, 1, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_decode_noalloc(GMLA_BF16, 2, 4, 5000, 128, 0.1f, F, F, F, 0, 0, F, 4, 0), GMLA_ERR_HIP);
  if (gmla_decode_noalloc_scratch_bytes() != ((size_t)4 << 20)) ++failures;
  /* latent-fused prefill */
  {
    const size_t need = gmla_prefill_latent_workspace_bytes(1, 300, 2, 128);
    EXPECT(gmla_attend_prefill_latent(GMLA_BF16, 1, 300, 2, 128, 100, 0.1f, 1, F, 0, F, F, F, 0, F, F, need, 0), GMLA_ERR_UNSUPPORTED);
    EXPECT(gmla_attend_prefill_latent(GMLA_BF16, 1, 300, 2, 128, 512, 0.1f, 1, F, 0, F, F, F, 0, F, F, need - 1, 0), GMLA_ERR_WORKSPACE);
    EXPECT(gmla_attend_prefill_latent(GMLA_BF16, 1, 300, 2, 128, 512, 0.1f, 1, F, 0, F, F, F, F, F, F, need, 0), GMLA_ERR_HIP);
  }
  /* per-sequence lengths */
  EXPECT(gmla_attend_varlen(GMLA_BF16, 2, 4, 128, 0.1f, 1, F, 0, F, 0, F, F, 0, F, 10, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_varlen(GMLA_BF16, 2, 4, 96, 0.1f, 1, F, 0, F, 10, F, F, 0, F, 10, 0, F, 0), GMLA_ERR_UNSUPPORTED);
  EXPECT(gmla_attend_varlen(GMLA_BF16, 2, 4, 128, 0.1f, 1, F, 0, F, 10, F, F, 0, F, 10, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_varlen(GMLA_F32, 2, 4, 32, 0.1f, 0, F, 0, F, 10, F, F, 0, F, 0, 0, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_decode_varlen(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, 0, 0, F, 0, 0, 1, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_attend_decode_varlen(GMLA_BF16, 2, 4, 100, 128, 0.1f, F, F, F, 0, F, 0, F, 0, 0, 1, 0), GMLA_ERR_HIP);
  EXPECT(gmla_attend_decode_varlen(GMLA_BF16, 2, 4, 5000, 128, 0.1f, F, F, F, 0, F, F, F, F, 1 << 20, 3, 0), GMLA_ERR_HIP);
  /* decode over the latent cache */
  {
    const int64_t bad_c[2] = {100 * 512, 516};
    const size_t need = gmla_decode_latent_workspace_bytes(2, 4, 100, 512, 0);
    EXPECT(gmla_attend_decode_latent(GMLA_BF16, 2, 4, 100, 128, 512, 0.1f, F, F, bad_c, F, F, 0, F, F, need, 0, 0), GMLA_ERR_INVALID_ARG);
    EXPECT(gmla_attend_decode_latent(GMLA_BF16, 2, 4, 100, 128, 384, 0.1f, F, F, 0, F, F, 0, F, F, need, 0, 0), GMLA_ERR_UNSUPPORTED);
    EXPECT(gmla_attend_decode_latent(GMLA_BF16, 2, 4, 100, 128, 512, 0.1f, F, F, 0, F, F, 0, F, F, need - 1, 0, 0), GMLA_ERR_WORKSPACE);
    EXPECT(gmla_attend_decode_latent(GMLA_BF16, 2, 4, 100, 128, 512, 0.1f, F, F, 0, F, F, F, F, F, need, 0, 0), GMLA_ERR_HIP);
    EXPECT(gmla_attend_decode_latent(GMLA_BF16, 1, 40, 33, 128, 128, 0.1f, F, F, 0, F, F, 0, F, F, 1 << 20, 3, 0), GMLA_ERR_HIP);
    EXPECT(gmla_attend_decode_latent_varlen(GMLA_BF16, 2, 4, 100, 128, 512, 0.1f, F, F, 0, 0, F, F, 0, F, F, need, 0, 0), GMLA_ERR_INVALID_ARG);
    EXPECT(gmla_attend_decode_latent_varlen(GMLA_BF16, 2, 4, 100, 128, 512, 0.1f, F, F, 0, (const int*)F, F, F, 0, F, F, need, 0, 0), GMLA_ERR_HIP);
    if (gmla_decode_latent_num_splits(8, 96, 1001, 512) != 7) ++failures;
  }
  /* projections */
  EXPECT(gmla_linear(GMLA_BF16, 4, 4, 12, F, F, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_linear(GMLA_BF16, 64, 64, 64, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_linear(GMLA_BF16, 2048, 12288, 128, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_linear(GMLA_F32, 3, 5, 7, F, F, F, 0), GMLA_ERR_HIP);
  if (gmla_linear_workspace_bytes(2048, 512, 12288) != (size_t)8 * 2048 * 512 * 4) ++failures;
  EXPECT(gmla_linear_ws(GMLA_BF16, 2048, 512, 12288, F, F, F, F, (size_t)1 << 26, 0), GMLA_ERR_HIP);
  EXPECT(gmla_linear_ws(GMLA_BF16, 4, 4, 12, F, F, F, F, 0, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_latent_expand(GMLA_BF16, 4, 8, 16, F, 0, F, F, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_latent_expand(GMLA_BF16, 64, 64, 128, F, F, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_gate_out(GMLA_BF16, 4, 16, 0, 0, 0, F, 0), GMLA_ERR_INVALID_ARG);
  EXPECT(gmla_gate_out(GMLA_BF16, 64, 128, F, F, F, F, 0), GMLA_ERR_HIP);
  EXPECT(gmla_gate_out(GMLA_BF16, 64, 128, F, F, 0, F, 0), GMLA_ERR_HIP);
  EXPECT((int)gmla_gate_out_workspace_bytes(GMLA_BF16, 64, 128), 64 * 128 * 2);
  EXPECT(gmla_gate_out_ws(GMLA_BF16, 64, 128, F, F, F, F, (void*)((char*)F + (1 << 24)), 64 * 128 * 2, 0), GMLA_ERR_HIP);
  if (gmla_status_string(GMLA_ERR_HIP)[0] != 'G') ++failures;
  printf("host sanitized run: %d failures\n", failures);
  return failures != 0;
}
