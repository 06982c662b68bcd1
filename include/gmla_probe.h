/*
 * gmla_probe.h -- measurement aids for libgmla's benchmark (libgmla_probe.so).
 *
 * Two microbenchmarks give the rates the hot-path kernels can actually reach on
 * the device, beside the data-sheet peaks they are priced against: a matrix-core
 * loop with no memory traffic, and a plain streaming read of device memory.  They
 * compute nothing of the attention method and are not part of libgmla.
 *
 * Both take caller-owned device buffers, launch on `stream` (a hipStream_t, NULL for
 * the default stream), return 0 on success, -1 for invalid arguments (checked on the
 * host before any HIP call) and -4 if the launch fails.
 */
#ifndef GMLA_PROBE_H
#define GMLA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * `blocks` workgroups of 256 threads each run `iters` rounds of 16 dependent-chain
 * v_mfma_f32_32x32x16_bf16 (four independent accumulators per wave, register
 * operands only): blocks * 4 * iters * 16 * 32768 flop.  `out` receives one float per
 * thread (blocks * 256 floats) so the work cannot be elided.
 */
int gmla_probe_mfma(int blocks, int iters, float* out, void* stream);

/*
 * The same loop and work count, but each wave cycles through eight register sets of
 * random bf16 operands (signs and mantissas from an integer hash, magnitudes 2^-3 to
 * 2^2), so consecutive MFMAs see changing data as the attention's matrix products do.
 * The clock the chip holds depends on that switching: this is the matrix-core ceiling
 * for random data.
 */
int gmla_probe_mfma_random(int blocks, int iters, float* out, void* stream);

/*
 * Reads `bytes` (a multiple of 16 * 256 * 8) of device memory at `buf` once with
 * 16-byte non-temporal loads, eight in flight per lane, from `blocks` workgroups of
 * 256 threads; `out` (blocks unsigned ints) is written only where a lane's
 * checksum matches a fixed constant, so the kernel's traffic is essentially the read.
 */
int gmla_probe_read(const void* buf, size_t bytes, int blocks, unsigned* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMLA_PROBE_H */
