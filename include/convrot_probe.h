/*
 * convrot_probe.h - measurement probes of the ConvRot library (gfx950).
 *
 * Not part of the method: these kernels touch none of the linear's data.
 * They measure, on the machine at hand, the ceilings the benchmark reports
 * beside the spec peaks of the two rooflines the linear runs against:
 *   - the int8 matrix-core rate with no memory traffic (the large-M GEMM's
 *     bound: 2*M*N*K int ops on v_mfma_i32_32x32x32_i8), and the shader
 *     clock the chip holds under that load;
 *   - the rate of one kernel reading a cold buffer (the small-M GEMM's bound:
 *     its 4-bit weight stream, read once per call);
 *   - the rate of a plain device copy.
 * Conventions are those of convrot.h: device pointers owned by the caller,
 * work enqueued on `stream` with no synchronisation and no allocation,
 * argument errors returned before any launch.
 */
#ifndef CONVROT_PROBE_H
#define CONVROT_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "convrot.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe: `blocks` blocks of 8 waves; each wave runs `iters`
 * rounds of 4 independent v_mfma_i32_32x32x32_i8 (65536 int ops each) on
 * register operands, so the launch performs blocks * 8 * iters * 4 * 65536
 * int ops.  sink: int32 [blocks * 512] (out; a fold of the accumulators that
 * keeps the work live, meaningless otherwise).  stamps: uint64 [4] (out) =
 * shader clock counter at the start and the end of block 0's first wave,
 * then the constant-rate real-time counter at the same two points (its rate
 * from cr_probe_wall_clock_khz()).  1 <= blocks <= 65535, 1 <= iters <= 2^24. */
cr_status cr_probe_mfma_i8(int blocks, int iters, int32_t* sink, uint64_t* stamps, hipStream_t stream);

/* Read probe: one kernel reads `bytes` (a multiple of 16, at most 2^36) from
 * `src` with 16-byte loads, each thread issuing four before using any, and
 * writes one uint32 per block to `sink` (uint32 [4096]; out, meaningless). */
cr_status cr_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Copy probe: dst[0:bytes] = src[0:bytes] with 16-byte loads and stores
 * (bytes a multiple of 16, at most 2^36; the ranges must not overlap). */
cr_status cr_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Rate of the real-time counter of cr_probe_mfma_i8's stamps, in kHz, of the
 * current device (0 if it cannot be read). */
int cr_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif
#endif /* CONVROT_PROBE_H */
