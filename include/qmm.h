/*
 * qmm.h -- C ABI of the skinny quantized matrix product on MI355X (gfx950).
 *
 *   y[M,N] = x[M,K] . dequant(W)[N,K]^T
 *
 * for skinny batches M = 1..32, where W is stored as 4.5-bit k-quant
 * super-blocks (Q4_K). This is the product that takes the time of a
 * speculative-decoding verify pass:
 *   - "sixi-asi 0.9", section "What I got wrong in 0.8": a verify step runs
 *     the target model over the anchor plus k drafts in one batched pass, and
 *     quantized matrix products take 83-92% of its GPU time; the per-row cost
 *     came from a kernel that decoded the 4-bit weights again for every row.
 *   - "sixi-asi 0.11", section "Why sixteen streams were the ceiling": several
 *     streams share one pass, and the pass reads the whole weight set once
 *     almost regardless of the number of rows (up to 32 streams).
 *   - "sixi-asi 0.9", section "The patch": the switch point between the
 *     row-vector and the tiled kernel and the occupancy of the tiled kernel
 *     decide the time; a time faster than reading the weights at full memory
 *     bandwidth is a bug, not a result.
 *
 * Weight format (one super-block = 256 consecutive weights along K, 144 bytes;
 * the Q4_K k-quant of the Q4_K_M GGUF files named in "sixi-asi 0.9", section
 * "Numbers"; the byte map is the public Q4_K layout):
 *   bytes 0..1   d     binary16, little-endian
 *   bytes 2..3   dmin  binary16, little-endian
 *   bytes 4..15  eight 6-bit scales sc_j and eight 6-bit mins m_j, packed:
 *                j < 4:  sc_j = s[j] & 63,  m_j = s[j+4] & 63
 *                j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4
 *                        m_j  = (s[j+4] >> 4) | (s[j]   >> 6) << 4
 *   bytes 16..143 quants: weight 64c + r (c = 0..3, r = 0..63) is the low
 *                nibble (r < 32) or high nibble (r >= 32) of byte
 *                16 + 32c + (r mod 32)
 *   weight i of the block: w = d * sc_j * q_i - dmin * m_j,  j = i / 32.
 * A matrix W[N,K] is N rows of K/256 consecutive blocks; rows are consecutive.
 * Block (n, b) starts at byte (n * (K/256) + b) * 144.
 *
 * Numerics: fp32 output. Activations are rounded once to binary16 inside the
 * kernels (the same rounded value feeds the quant term and the min term), the
 * products of quants and scales are exact, and all sums are fp32. Per element
 * |y - y_exact| <= 2e-3 * sum_k |w[n,k] * x[m,k]| holds for |x| < 65504 (the
 * binary16 range). The summation order is fixed by the launch plan, so repeated
 * calls with the same plan give bit-identical results.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. 0 is success; every error is negative and no kernel is
 * launched when a call returns an error. */
enum {
  QMM_OK = 0,
  QMM_ERR_INVALID_ARG = -1, /* null handle/pointer, bad override values */
  QMM_ERR_SHAPE = -2,       /* M outside 1..32, N < 1, K < 256 or K % 256 != 0 */
  QMM_ERR_ALIGN = -3,       /* x or W_blocks not 16-byte aligned, y not 4-byte aligned */
  QMM_ERR_NO_DEVICE = -4,   /* device index invalid or not gfx950 */
  QMM_ERR_OOM = -5,         /* workspace allocation failed in qmm_create */
  QMM_ERR_HIP = -6,         /* a HIP runtime call or a launch failed */
  QMM_ERR_OVERLAP = -7,     /* y overlaps x or W_blocks */
  QMM_ERR_SCRATCH = -8      /* qmm_run_static: the plan needs more scratch than it has */
};

/* Largest batch (rows of x) a call accepts: one row per stream for up to 32
 * concurrent streams ("sixi-asi 0.11", table and section "Why sixteen streams
 * were the ceiling"). */
#define QMM_MAX_M 32

typedef struct qmm_ctx* qmm_handle;

/* Create a handle on HIP device `device`. Queries the device (CU count, LDS,
 * architecture; only gfx950 is accepted), loads the launch table and allocates
 * the split-K workspace: 128 MiB of partial sums and 4 MiB of per-tile arrival
 * counters (device memory owned by the handle; the counters are zeroed here,
 * synchronously). device == -1 creates a planning-only handle: it plans and
 * checks arguments but never launches (qmm_run then returns
 * QMM_ERR_NO_DEVICE after its argument checks). On error *out is set to NULL.
 * A handle may be used by one stream at a time; create one handle per
 * concurrent stream. */
int qmm_create(qmm_handle* out, int device);

/* y = x . dequant(W_blocks)^T, enqueued on `stream`; returns at once and never
 * synchronizes.
 *   x        device pointer, fp32 [M][K] row-major, 16-byte aligned.
 *   W_blocks device pointer, N*K/256 super-blocks of 144 bytes in the layout
 *            above, 16-byte aligned.
 *   y        device pointer, fp32 [M][N] row-major, 4-byte aligned; it is
 *            overwritten (not accumulated into) and must not overlap x or W.
 *   M in 1..QMM_MAX_M, N >= 1, K >= 256 with K % 256 == 0.
 * All three buffers are owned by the caller, who keeps them alive until the
 * stream work completes; the library never frees or retains them. The pointers
 * must be on the handle's device (not checked). Argument errors are returned
 * before anything is launched; faults inside a kernel surface at the caller's
 * next synchronization. */
int qmm_run(qmm_handle h, const float* x, const void* W_blocks, float* y,
            int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Expert-indexed product (the MUL_MAT_ID case of the op test that the
 * launch-shape patch passes, "sixi-asi 0.9", section "The patch"):
 *
 *   y[m,:] = x[m,:] . dequant(W_experts[ids[m]])^T   for every row m,
 *
 * W_experts holds E matrices of N x K in the layout above, consecutively
 * (matrix e starts at byte e * qmm_weight_bytes(N, K)); ids is a device array of
 * M int32 expert indices. Rows that use the same expert share one pass over
 * its weights (each distinct expert is streamed once); rows whose id is
 * outside [0, E) are not written (y keeps their previous contents).
 *   x, y, M, N, K: as for qmm_run (ids 4-byte aligned, must not overlap y).
 * Enqueued on `stream`; never synchronizes. Always uses the tiled kernel.
 * Same status codes as qmm_run (E < 1 or a null ids: QMM_ERR_INVALID_ARG). */
int qmm_run_ids(qmm_handle h, const float* x, const void* W_experts, const int32_t* ids,
                int64_t E, float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Block-scaled FP4 weights ("NVFP4"), the second weight format. The pages
 * measure a W4A16 product over it (FlashRT issue #153: the NVFP4 W4A16 GEMM
 * and its per-shape bench of lm_head and gate+up at 1 and 7 rows) without
 * defining its bits; those are public: elements FP4 E2M1 (OCP Microscaling
 * Formats v1.0: sign, 2 exponent bits with bias 1, 1 mantissa bit), one FP8
 * E4M3 scale (OCP OFP8: bias 7, S.1111.111 = NaN) per 16 consecutive elements
 * of a row, one fp32 tensor scale; w = tensor_scale * scale * element.
 *
 * The library streams them in groups of 256 weights in 144 bytes, the
 * geometry of the 4.5-bit super-blocks: per row, K/256 groups in K order;
 * group bytes 0..15 are the scale codes of its 16 runs of 16 elements, bytes
 * 16..143 its element codes, element 64c + r (c = 0..3, r = 0..63) in byte
 * 16 + 32c + (r mod 32), low nibble for r < 32, high nibble for r >= 32.
 * qmm_weight_bytes(N, K) is the size of N rows of groups. NaN scale codes are
 * not supported (their weights are unspecified). */

/* Host-side repack from the usual layout: elems [N][K/2] bytes with element
 * 2i of a row in the low nibble of byte i and 2i+1 in the high nibble,
 * scales [N][K/16] codes (scale j covers elements 16j..16j+15), into
 * groups [N][K/256][144]. All three are host memory owned by the caller; K is
 * a multiple of 256. Returns QMM_OK, QMM_ERR_INVALID_ARG (null pointer) or
 * QMM_ERR_SHAPE. */
int qmm_nvfp4_repack(const uint8_t* elems, const uint8_t* scales, int64_t N, int64_t K,
                     uint8_t* groups);

/* y = x . w^T for block-scaled FP4 weights in groups (above), on `stream`;
 * never synchronizes. x, y, M, N, K, alignment, overlap and ownership as for
 * qmm_run (W_groups in place of W_blocks); tensor_scale must be finite, else
 * QMM_ERR_INVALID_ARG. The weights are
 * exact in the kernel's binary16 arithmetic; x is rounded to binary16 once,
 * as in qmm_run. Always uses the tiled kernel. */
int qmm_run_nvfp4(qmm_handle h, const float* x, const void* W_groups, float tensor_scale,
                  float* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Plain 4-bit integer weights, one scale per 128 columns. The "sixi-asi 0.11"
 * page (section "What did not work") names this layout as the plain
 * alternative to the k-quant files without fixing its bits; read here as:
 * elements 4-bit two's-complement integers q in [-8, 7] (no zero point), one
 * IEEE binary16 scale per 128 consecutive elements of a row;
 * w = scale * q.
 *
 * The library streams them in groups of 256 weights in 144 bytes, the
 * geometry of the 4.5-bit super-blocks: per row, K/256 groups in K order;
 * group bytes 0..1 and 2..3 are the binary16 scales (little-endian) of its
 * elements 0..127 and 128..255, bytes 4..15 are zero, bytes 16..143 hold the
 * codes offset by 8 (q + 8, 0..15), element 64c + r (c = 0..3, r = 0..63) in
 * byte 16 + 32c + (r mod 32), low nibble for r < 32, high nibble for r >= 32.
 * The 12 padding bytes make a group 4.5 bits per weight against the layout's
 * own 4.125; qmm_weight_bytes(N, K) is the size of N rows of groups. */

/* Host-side repack from the usual layout: codes [N][K/2] bytes, element 2i
 * of a row in the low nibble of byte i and 2i+1 in the high nibble, two's
 * complement; scales [N][K/128] binary16 bit patterns (scale j covers
 * elements 128j..128j+127), into groups [N][K/256][144]. All three are host
 * memory owned by the caller; K is a multiple of 256. Returns QMM_OK,
 * QMM_ERR_INVALID_ARG (null pointer) or QMM_ERR_SHAPE. */
int qmm_int4_repack(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                    uint8_t* groups);

/* y = x . w^T for plain INT4 weights in groups (above), on `stream`; never
 * synchronizes. x, y, M, N, K, alignment, overlap and ownership as for
 * qmm_run (W_groups in place of W_blocks). The codes are exact in the
 * kernel's binary16 arithmetic and the scales are applied in fp32, so zero
 * codes give exact zeros; x is rounded to binary16 once, as in qmm_run.
 * Infinite or NaN scales are not supported (their outputs are unspecified).
 * Always uses the tiled kernel. */
int qmm_run_int4(qmm_handle h, const float* x, const void* W_groups, float* y, int64_t M,
                 int64_t N, int64_t K, hipStream_t stream);

/* y = x . dequant(W_blocks)^T like qmm_run, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc. It takes no handle and calls no
 * allocating routine. Its split-K workspace is a static device array of the
 * library (32 MiB of partial sums and 65536 row-tile counters, 33 MiB per
 * device, held by each device the library runs on until the process ends),
 * set up at the first call on a device (that call also enqueues a small
 * kernel on `stream` that zeroes the counters). It runs on the current HIP
 * device, plans like a fresh handle (the launch table, no overrides) and
 * launches the same kernels, so it gives the same bits as qmm_run with the
 * same plan. A call whose plan needs more split-K workspace than the array
 * holds (e.g. a 151936-row matrix at more than 16 rows) returns
 * QMM_ERR_SCRATCH and launches nothing. Every call on one device shares that
 * device's array, so calls that overlap in time on one device (several
 * streams, or host threads) race on it and must be serialized by the caller.
 * Arguments, layouts, ownership, alignment and the other status codes are
 * those of qmm_run. */
int qmm_run_static(const float* x, const void* W_blocks, float* y, int64_t M, int64_t N,
                   int64_t K, hipStream_t stream);

/* Free the handle and its workspace. qmm_destroy(NULL) is a no-op returning
 * QMM_OK. The caller must make sure no work enqueued with the handle is still
 * running. */
int qmm_destroy(qmm_handle h);

/* Static, human-readable text for a status code. */
const char* qmm_status_string(int status);

/* Weight bytes of an N x K matrix in this format: 144 * N * K / 256 (the
 * weight-only byte count behind every bandwidth figure; "sixi-asi 0.9",
 * section "The patch": 15.8 GB per pass at 273 GB/s is the ~58 ms floor).
 * Returns 0 for invalid shapes. */
uint64_t qmm_weight_bytes(int64_t N, int64_t K);

/* Kernels of the launch table. */
enum {
  QMM_KERNEL_AUTO = 0,  /* let the launch table decide (for overrides) */
  QMM_KERNEL_VECTOR = 1, /* row-vector kernel: VALU dot products, x broadcast;
                            1..8 rows (its work grows with every row) */
  QMM_KERNEL_TILED = 2   /* tiled kernel: MFMA 16x16x32 f16 (rows padded to 16) */
};

/* One launch-table entry: which kernel, how the grid is shaped. */
typedef struct {
  int32_t kernel;        /* QMM_KERNEL_VECTOR or QMM_KERNEL_TILED */
  int32_t waves_per_wg;  /* wavefronts per workgroup: 1..8 */
  int32_t splits;        /* K split into this many slices (1 = no split-K) */
  int32_t grid_x;        /* workgroups per range of wave_splits slices; each tile
                            group of a workgroup walks the 16-row tiles
                            b*groups + t, + grid_x*groups, ..., so the table never
                            launches more workgroups than the device holds at
                            once (nor more than one tile per group needs) */
  int32_t blocks_per_split; /* super-blocks along K per slice */
  int32_t lds_bytes;     /* LDS per workgroup */
  int32_t wave_splits;   /* slices reduced inside one workgroup: its waves form
                            waves_per_wg / wave_splits tile groups, and the
                            wave_splits waves of a group sum their slices in LDS;
                            the remaining splits / wave_splits ranges are
                            summed across workgroups (split-K) */
  int64_t workspace_bytes; /* split-K partials used (0 without split-K across
                              workgroups) */
} qmm_plan;

/* The entry qmm_run would use for (M, N, K) with the handle's current
 * overrides. Returns a status like qmm_run's argument checks. */
int qmm_query_plan(qmm_handle h, int64_t M, int64_t N, int64_t K, qmm_plan* out);

/* Weight formats of the entry points: qmm_run / qmm_run_ids (4.5-bit
 * super-blocks), qmm_run_nvfp4, qmm_run_int4. */
enum {
  QMM_FORMAT_KQUANT = 0,
  QMM_FORMAT_NVFP4 = 1,
  QMM_FORMAT_INT4 = 2
};

/* The entry the call of that format would use, with the handle's current
 * overrides: expert_slots = 0 for a plain call, else the distinct experts an
 * expert-indexed call (qmm_run_ids) holds in its grid, min(M, E). For tests
 * that replay the kernels' index arithmetic on the host, and for sweeps.
 * QMM_ERR_INVALID_ARG for an unknown format, expert slots with a format other
 * than QMM_FORMAT_KQUANT, or slots outside 0..M; otherwise like
 * qmm_query_plan. */
int qmm_query_plan_format(qmm_handle h, int format, int expert_slots, int64_t M, int64_t N,
                          int64_t K, qmm_plan* out);

/* Force a kernel for every following call on this handle (QMM_KERNEL_AUTO
 * restores the table). For tests and sweeps. A call that forces the
 * row-vector kernel above 8 rows returns QMM_ERR_INVALID_ARG. */
int qmm_set_kernel(qmm_handle h, int kernel);

/* Override the grid shape for every following call: waves_per_wg (0 = table,
 * else 1..8), splits (0 = table), grid_x (0 = table; any positive count works:
 * with fewer workgroups each tile group walks more tiles, with more some stay
 * idle). Values that do not fit the call (LDS, workspace, K) make qmm_run
 * return QMM_ERR_INVALID_ARG. On a planning-only handle the table's grid_x is
 * one tile per tile group (the device's capacity is unknown there). For
 * sweeps. */
int qmm_set_shape(qmm_handle h, int waves_per_wg, int splits, int grid_x);

/* Override how many K slices one workgroup reduces itself for every following
 * call (0 = table, else 1..8; waves_per_wg must be a multiple and splits at
 * least this, or qmm_run returns QMM_ERR_INVALID_ARG). For sweeps. */
int qmm_set_wave_splits(qmm_handle h, int wave_splits);

/* For measurement: the next launch made through this handle (any qmm_run*
 * call) records `start` when its kernel begins executing and `stop` when it
 * ends (hipExtLaunchKernel), so that hipEventElapsedTime(start, stop) is the
 * kernel's own duration without the launch overhead around it; the events
 * are then forgotten (one launch only). Events are created by the caller on
 * the handle's device; NULL, NULL clears them. Not for use under graph
 * capture. Returns QMM_ERR_INVALID_ARG for a null handle. */
int qmm_set_launch_events(qmm_handle h, hipEvent_t start, hipEvent_t stop);

/* The row count from which the launch table switches from the row-vector to
 * the tiled kernel (M >= switch uses the tiled kernel). */
int qmm_switch_point(qmm_handle h, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
