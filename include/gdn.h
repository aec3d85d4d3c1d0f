/*
 * gdn.h -- C ABI of the Gated DeltaNet recurrent update with the replay of a
 * row log, on MI355X (gfx950). Part of libqmm.so; status codes are qmm.h's.
 *
 * What it computes. The other step of a hybrid model's verify pass besides
 * the quantized products: 48 of the model's 64 layers are Gated DeltaNet
 * layers whose recurrent state (3.1 MB per layer and sequence) is updated by
 * every row ("sixi-asi 0.11", section "What changed"; "sixi-asi 0.9", section
 * "What I got wrong in 0.8": about 3 ms of a pass). The update is a function
 * of the previous state and four per-row inputs, key, value, gate and beta;
 * instead of a snapshot after every row a sequence keeps one base state and
 * the inputs of its last few rows, and a rollback replays the kept rows on
 * the base state inside the kernel that processes the new rows ("sixi-asi
 * 0.11", section "A log instead of snapshots").
 *
 * The update rule is not on those pages; it is the gated delta rule of the
 * Gated DeltaNet paper (Yang, Kautz and Hatamizadeh, ICLR 2025). Per head,
 * with S the dv x dk state matrix:
 *
 *   S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T
 *   o_t = S_t q_t
 *
 * i.e. row i of S: s <- alpha s + beta (v_i - alpha (s . k)) k. The call
 * takes the keys and queries as given (a layer normalizes them before the
 * recurrence); the rule is a contraction, and the error bound below holds,
 * for keys of unit norm, alpha in [0, 1] and beta in [0, 1].
 *
 * One call processes B sequences of one layer. For sequence b the state
 * starts from its base state; the first n_log[b] rows of its log are applied
 * (no outputs), then its M new rows, each followed by its output. After the
 * first commit[b] rows of that walk (log rows first) the state at that point
 * overwrites the base state; commit[b] = 0 leaves it unchanged. (How the log
 * is kept, shifted or trimmed is the caller's bookkeeping.)
 *
 * Geometry: H heads of dk = dv = 128 (a reading: 48 heads give the pages'
 * 3 MiB per layer and sequence, 48 layers x 3 MiB the 144 MiB snapshot per
 * row); other head sizes return QMM_ERR_SHAPE.
 *
 * Layouts (fp32, row-major, device memory owned by the caller):
 *   state   [B][H][dk][dv]  element [b][h][e][i] = S_bh[i][e] (key index
 *                           outer, value index inner); read, and written
 *                           in place where commit[b] > 0
 *   k_log   [B][L][H][dk]   v_log [B][L][H][dv]
 *   gate_log, beta_log [B][L][H]
 *   n_log   [B] int32       kept rows per sequence
 *   q, k    [B][M][H][dk]   v [B][M][H][dv]   gate, beta [B][M][H]
 *   commit  [B] int32, or NULL (no commit)
 *   o       [B][M][H][dv]   overwritten
 * n_log[b] is clamped to [0, L] and commit[b] to [0, n_log[b] + M] (values
 * on the device cannot be checked before the launch).
 *
 * Numerics: fp32 state and arithmetic; per element of o after T rows,
 * |o - o_exact| <= (T + 1) (dk + 8) 2^-24 (R ||q|| + sum_e |S_ie q_e|), R the
 * largest |S_i.| + beta |v_i| along the walk, and the state likewise. The
 * summation order is fixed, so repeated calls give bit-identical results.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one call on `stream` (asynchronous; never synchronizes). B >= 1,
 * H >= 1, M >= 0, L >= 0. Pointers must be non-null except: the log arrays and
 * n_log when L = 0, the new-row arrays and o when M = 0, and commit. All
 * arrays 4-byte aligned. The state must not overlap any other array and o
 * must not overlap the inputs. Returns QMM_OK, or QMM_ERR_INVALID_ARG (null
 * pointer, negative sizes, more than 2^31 - 1 workgroups, more than 2^40 log
 * rows B L H or new rows B M H), QMM_ERR_SHAPE (dk
 * or dv not 128), QMM_ERR_ALIGN, QMM_ERR_OVERLAP, QMM_ERR_NO_DEVICE (no
 * current HIP device), QMM_ERR_HIP (launch failure); on an error nothing is
 * launched. */
int gdn_replay_update(float* state, const float* k_log, const float* v_log,
                      const float* gate_log, const float* beta_log, const int32_t* n_log,
                      int64_t L, const float* q, const float* k, const float* v,
                      const float* gate, const float* beta, const int32_t* commit, float* o,
                      int64_t B, int64_t M, int64_t H, int64_t dk, int64_t dv,
                      hipStream_t stream);

/* Algorithmic bytes of a call: the states read (B*H*dk*dv*4), the states
 * written (that again for each sequence with commit > 0, given as
 * `committing`), the log rows applied (`log_rows` in total over the
 * sequences) and new rows read, and the outputs written. */
uint64_t gdn_call_bytes(int64_t B, int64_t M, int64_t H, int64_t dk, int64_t dv,
                        int64_t log_rows, int64_t committing);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
