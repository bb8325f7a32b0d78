/*
 * beam_probe.h — measurement instruments of the library (gfx950 only).
 *
 * Two kernels that measure what one MI355X sustains, so that a kernel's rate
 * can be reported as a fraction of a measured ceiling beside the fraction of
 * the published peak (dense bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s):
 *   - the bf16 matrix-core rate on operands with random mantissas (the chip
 *     runs slower on random data than on constant data: it is power-limited),
 *     for the two bf16 MFMA shapes (the 16x16x32 instruction sustains about
 *     half as much again as 32x32x16 on the same loop);
 *   - the HBM read rate of a plain streaming read.
 * Neither is part of the attention path. Conventions as in beam_attn.h:
 * device pointers, work enqueued on `stream`, arguments checked on the host
 * (statuses of beam_attn.h, message in beam_last_error()).
 */
#ifndef BEAM_PROBE_H
#define BEAM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "beam_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Register-only loop of v_mfma_f32_32x32x16_bf16. n_blocks blocks of 256
 * threads; every wave keeps 8 A and 8 B operand fragments and 4 accumulators
 * in registers and issues 16 MFMAs per iteration, cycling through them.
 * `distinct` (1..8) of the 8 fragments are different values (the others
 * repeat them): 8 makes the operands change on every MFMA, as they do in the
 * attention kernels; fewer repeat them (less switching activity).
 * operands: device uint32 [n_blocks * 256 * 64] (bf16 pairs; fill with random
 * normal values, or constants). out: device float [n_blocks * 256] (a checksum
 * per thread). Work: n_blocks * 4 waves * iters * 16 MFMAs * 32768 flop. The
 * chip boosts for a fraction of a millisecond: a sustained rate needs a run of
 * several milliseconds. */
beam_status beam_probe_mfma_bf16(const uint32_t *operands, int32_t n_blocks, int32_t iters, int32_t distinct,
                                 float *out, void *stream);

/* The same loop with v_mfma_f32_16x16x32_bf16: 32 MFMAs per iteration over 8
 * accumulators, the same operands and the same work (n_blocks * 4 waves *
 * iters * 32 MFMAs * 16384 flop = the figure above). */
beam_status beam_probe_mfma16_bf16(const uint32_t *operands, int32_t n_blocks, int32_t iters, int32_t distinct,
                                   float *out, void *stream);

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) with 16-byte
 * non-temporal loads, grid-stride over n_blocks blocks of 256 threads, eight
 * loads in flight per thread. out: device uint32 [n_blocks * 256] (an XOR
 * checksum per thread). */
beam_status beam_probe_stream_read(const void *buf, size_t bytes, int32_t n_blocks, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BEAM_PROBE_H */
