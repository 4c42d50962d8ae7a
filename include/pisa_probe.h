/* libpisa_probe: measurement helpers, not part of the attention library.
 *
 * Measures the HBM streaming-read rate, and the bf16 MFMA rate that gfx950 sustains for the per-chunk
 * instruction mix of libpisa's attention kernel (exact phase, d = 128,
 * 32-key chunks, three 4-wave workgroups per CU), on operands that toggle like
 * real activations.  The published dense peak assumes the nominal clock; under
 * sustained MFMA work on random data the chip holds a lower one, so this rate
 * is the attainable ceiling the kernel is compared with.
 */
#ifndef PISA_PROBE_H
#define PISA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of a `bytes`-byte device buffer (a multiple of 16, at least
 * 32 MiB; use far more than the 256 MB of on-chip caches, e.g. 2 GiB) by 8192
 * workgroups of 256 threads with 16-byte loads, timed over `reps` (>= 1)
 * launches after one warm-up.  gbs out: bytes read / time, GB/s (host
 * pointer).  Current device, null stream; allocates and frees the buffer;
 * synchronizes before returning.  Returns 0 (hipSuccess) or the first HIP
 * error code; invalid arguments give hipErrorInvalidValue and launch nothing. */
int pisa_probe_read_rate(size_t bytes, int reps, double* gbs);

/* mix    0: MFMAs only (S^T = K Q^T as 8 dependent 32x32x16 MFMAs, then
 *           O^T += V^T P^T as 8 MFMAs; P is S truncated to bf16);
 *        1: the full chunk step (the same MFMAs plus the softmax weights, one
 *           workgroup barrier and the global -> LDS copy of the next chunk);
 *        2: the 16 MFMAs per chunk alone with every operand in registers
 *           (eight A and eight B fragments cycled, four independent
 *           accumulators; no LDS, no barrier, no copies).
 * zeros  0: N(0, 1)-like bf16 operands; 1: all operands zero.
 * iters  chunks per wave per launch (>= 1); reps timed launches (>= 1) after
 *        one warm-up launch.
 * tflops out: algorithmic MFMA rate, TFLOP/s (host pointer).
 * Runs on the current device and the null stream, allocates and frees its
 * own 2 MB source and output buffers, and synchronizes before returning.
 * Returns 0 (hipSuccess) or the first HIP error code; invalid arguments give
 * hipErrorInvalidValue and launch nothing. */
int pisa_probe_chunk_rate(int mix, int zeros, int iters, int reps, double* tflops);

#ifdef __cplusplus
}
#endif

#endif
