/*
 * moe_peak.h -- measurement kernels of libmoe.so that anchor the roofline.
 *
 * They are not part of the MoE block: they measure what this GPU sustains
 * for the two resources the block's kernels are bound by, a streaming read
 * from HBM (the weight stream of the expert GEMMs at decode) and back-to-back
 * bf16 MFMAs (the expert GEMMs at prefill), and for the two together in the
 * proportions of the prefill GEMMs, so the block's rates can be reported
 * against these achievable figures next to the published peaks.
 *
 * Same conventions as moe.h: caller-owned device memory, nothing allocated or
 * synchronised, work only enqueued on `stream`; arguments are checked on the
 * host first and nothing is enqueued on an error.  The time is the caller's
 * to take (events around the call).
 */
#ifndef MOE_PEAK_H
#define MOE_PEAK_H

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of `buf` once, with 16-byte loads spread over
 * `workgroups` workgroups of 256 threads (8 loads in flight per thread,
 * consecutive lanes on consecutive 16-byte chunks), nontemporal loads if
 * `nontemporal` is nonzero.  Writes at most one 32-bit value to sink[0] (and
 * almost never: only if the XOR of the buffer equals a fixed key).
 *   buf    16-byte aligned; bytes a positive multiple of 16
 * MOE_ERR_INVALID_ARG on a bad argument, MOE_ERR_HIP if the launch fails. */
moe_status moe_peak_stream_read(const void* buf, size_t bytes, int nontemporal, uint32_t* sink,
                                int workgroups, hipStream_t stream);

/* Every wave of `workgroups` workgroups of 256 threads (4 waves) runs `iters`
 * steps of 8 independent 32x32x16 bf16 MFMAs on register operands (no memory
 * traffic), then writes one float: sink[wave index], sink holding
 * 4 * workgroups floats.  moe_peak_mfma_bf16_flops gives the FLOPs of one
 * call (2 * 32 * 32 * 16 per MFMA).
 *   random_operands  0: one fixed operand pattern for every chain and step
 *                    (few bits change from one MFMA to the next);
 *                    nonzero: each chain of each lane holds its own
 *                    pseudo-random bf16 operands (random sign and mantissa,
 *                    magnitudes 2^-5 .. 2^-1, from the splitmix64 mix of the
 *                    thread and chain index), so the bits change at every
 *                    issue as they do in a GEMM on real data.  The matrix
 *                    pipes draw more power on changing bits; where the board
 *                    power limit binds, the random rate is the lower one and
 *                    is the ceiling a GEMM on such data can meet. */
moe_status moe_peak_mfma_bf16(int64_t iters, int random_operands, float* sink, int workgroups,
                              hipStream_t stream);

double moe_peak_mfma_bf16_flops(int64_t iters, int workgroups);

/* MFMAs with an HBM stream beside them, in the proportions of a GEMM: every
 * wave of `workgroups` workgroups of 256 threads runs `steps` steps, each
 * reading four A and four B bf16 fragments (16 bytes a lane each) of
 * pseudo-random values from LDS and issuing the 16 32x32x16 MFMAs of their
 * outer product, while every lane issues `loads_per_step` nontemporal 16-byte
 * loads of `buf`, each consumed 8 steps after it is issued.  One 16-byte load a
 * lane per step is 1.95 bytes per thousand FLOPs; 2 is 3.9, close to the
 * algorithmic intensity of the prefill gate/up GEMM.  The rate this reaches is
 * what the GPU sustains for that mix of matrix work, LDS reads and HBM bytes
 * within its power limit.
 *   loads_per_step  0, 1, 2 or 4
 *   steps           a positive multiple of 8
 *   buf             16-byte aligned, at least
 *                   (steps + 8) * loads_per_step * workgroups * 256 * 16 bytes
 *                   (unused when loads_per_step is 0); thread t reads chunk
 *                   t + n * (workgroups * 256) for n = 0 .. (steps + 8) *
 *                   loads_per_step - 1: one contiguous span, read once
 *   sink            4 * workgroups floats, one written per wave
 * moe_peak_mfma_stream_flops gives the FLOPs of one call and
 * moe_peak_mfma_stream_bytes the bytes its steps consume.
 * MOE_ERR_INVALID_ARG on a bad argument, MOE_ERR_HIP if the launch fails. */
moe_status moe_peak_mfma_stream(const void* buf, size_t bytes, int loads_per_step, int64_t steps,
                                float* sink, int workgroups, hipStream_t stream);

double moe_peak_mfma_stream_flops(int64_t steps, int workgroups);

double moe_peak_mfma_stream_bytes(int64_t steps, int loads_per_step, int workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAK_H */
