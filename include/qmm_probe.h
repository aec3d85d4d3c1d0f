/*
 * qmm_probe.h -- measurement probes of the MI355X memory system and launch
 * path, used beside the product to say what its figures are measured against.
 *
 * FlashRT issue #153 (the Thor NVFP4 decode page, maintainer reply) checks a
 * product's bandwidth against the board itself: a device-to-device copy test
 * and a sustained read of the 635 MB lm_head in a tight loop, and it notes
 * that short reads are bound by launch overhead rather than by the memory.
 * These are the MI355X counterparts: a read-only streaming kernel (the
 * stream-read ceiling on a large buffer, or the sustained read of one
 * matrix) and an empty kernel (the launch gap between back-to-back launches
 * on one stream), plus a shader-clock probe, so that cycle counts and
 * per-CU rates can be stated at the clock the compute units actually ran.
 */
#ifndef QMM_PROBE_H
#define QMM_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of device memory at `buf` once with 128-bit non-temporal loads
 * (workgroup b reads a contiguous share; `grid` workgroups of `block`
 * threads, block a multiple of 64 up to 1024), enqueued on `stream`.
 * The loaded data is folded into one word per workgroup that is written to
 * sink[b] only in the (never generated) case that it equals a fixed magic
 * value, which keeps the loads from being optimized away; sink must hold
 * `grid` words. buf and bytes must be multiples of 16. Returns 0 (QMM_OK) or
 * QMM_ERR_INVALID_ARG / QMM_ERR_ALIGN / QMM_ERR_HIP as in qmm.h. */
int qmm_probe_read(const void* buf, uint64_t bytes, int grid, int block, uint32_t* sink,
                   hipStream_t stream);

/* Launch `grid` workgroups of 64 threads of an empty kernel on `stream`:
 * back-to-back launches of it measure the launch gap. Returns 0 or
 * QMM_ERR_INVALID_ARG / QMM_ERR_HIP. */
int qmm_probe_empty(int grid, hipStream_t stream);

/* Shader clock: `grid` workgroups of 64 threads (1 <= grid <= 2^20) each run
 * a dependent chain of `iters` fp32 FMAs (1 <= iters <= 2^26), and lane 0 of
 * workgroup b writes the shader clock counter (s_memtime) and the
 * constant-rate counter (s_memrealtime) read before and after the chain to
 * counts[4b], counts[4b+1], counts[4b+2], counts[4b+3] (device memory, 8-byte
 * aligned, 4 * grid words, owned by the caller). *wall_khz (host memory)
 * receives the constant counter's rate in kHz (the device attribute
 * hipDeviceAttributeWallClockRate of the current device), so that a
 * workgroup's clock is (counts[4b+2] - counts[4b]) / (counts[4b+3] -
 * counts[4b+1]) * wall_khz kHz. Enqueued on `stream`; the readings are valid
 * once it has completed. Returns 0 or QMM_ERR_INVALID_ARG / QMM_ERR_ALIGN /
 * QMM_ERR_HIP. */
int qmm_probe_clock(uint64_t* counts, int grid, int iters, int* wall_khz, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_PROBE_H */
