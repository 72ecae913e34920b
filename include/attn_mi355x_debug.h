/*
 * attn_mi355x_debug.h -- extra entry points of the debug build of the
 * library, libattn_mi355x_debug.so (compiled from the same sources with
 * ATTN_DEBUG_BUILD defined).  The release library libattn_mi355x.so exports
 * none of these.  Everything in attn_mi355x.h is exported by both builds and
 * behaves the same way.
 *
 * The debug build exists to observe what the release kernels cannot show in
 * their outputs: which branch of the rescale-threshold rule each query row
 * took on each KV step (release page "v1.7 / flash_attn 2.9.2.post1",
 * section 1.2: the rescale of O and the row sum is skipped while the row max
 * rises by at most the threshold, and the max then lags, so P stays at or
 * below exp2(threshold) = 256; release page "FA2 2.9.0 Kernel Changes in
 * v1.2", section 3: the first KV step never skips), to run the tile
 * shapes the release library's per-shape choice does not pick, and to
 * measure the matrix-core rate the board sustains.
 */
#ifndef ATTN_MI355X_DEBUG_H
#define ATTN_MI355X_DEBUG_H

#include <stdint.h>

#include "attn_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Tile-shape overrides for later forward / decode / backward launches of
 * this process (0 = the per-shape default the release library uses).
 * Forward, head_dim 128: 1 = 128 query rows per workgroup, 2 = 256 rows,
 * 3 = 32-key steps with four LDS stages, 4 = exp2 (and softcap's tanh) on
 * the FMA pipe, 5 = 128 rows of 32-key steps at three waves per SIMD,
 * 6 = 256 rows storing O straight from the accumulators; head_dim 256:
 * 1 = 128 rows, 2 = 256 rows, 3 = 128 rows at two waves per SIMD, 4 = 256
 * rows with the operand reads four ahead; head_dim 64: 1 = two waves per
 * SIMD.  Decode: 1 = 32-key steps with four stages, 2 = K/V copies with the
 * default cache policy.  Backward: 1 = dK/dV in two passes (head_dim 64 /
 * 128), 2 / 3 = dQ with 256 / 128 queries per workgroup (64 / 128), 4 = dK/dV
 * at one wave per SIMD (one pass at 64 / 128, two walks at 256).  Unknown
 * values select the default.  Not thread-safe; the setting is process-wide.
 */
void attn_debug_set_variants(int32_t fwd, int32_t dec, int32_t bwd);

/* KV step (keys per tile) of the last forward tile kernel launched. */
int32_t attn_debug_last_block_k(void);

/*
 * attn_fwd plus per-row counters of the rescale-threshold rule.
 *   args: as for attn_fwd (same validation, same outputs, same bits).
 *   row_stats: device uint32 [batch, heads_q, seqlen_q, 4], 16-byte aligned,
 *     written for every query row: [0] KV steps on which the row's running
 *     max left -inf (1 if the row sees any key, else 0), [1] later steps
 *     with a visible key that skipped the rescale (the max lagged), [2]
 *     later steps that rescaled, [3] the bits of the largest fp32 P the row
 *     formed before its 16-bit conversion (0.0f if none).  A step counts
 *     only when the row sees at least one of its keys.
 * Returns ATTN_E_NULL / ATTN_E_ALIGN for a bad row_stats, else as attn_fwd.
 */
int attn_fwd_stats(const attn_fwd_args* args, uint32_t* row_stats, void* stream);

/*
 * Matrix-core rate calibration; no attention work.  Launches `blocks`
 * workgroups of 256 threads (4 waves); every wave issues `iters` x 16 dense
 * 32x32x16 MFMAs of `dtype` (ATTN_DTYPE_F16 / _BF16) into four independent
 * accumulators, on operands it reads once from `operands`, and each thread
 * writes the sum of its accumulators to `out` (so the work is kept).
 *   operands: device, 16-byte aligned, 8 KiB: 64 lanes x 8 16-byte chunks,
 *     lane-major; chunks 0-3 are a lane's A fragments, 4-7 its B fragments
 *     (16-bit values of `dtype`; random values or zeros, which draw less
 *     power).  Read only.
 *   out: device float [blocks * 256], 4-byte aligned; overwritten.
 * Work per call: blocks * 4 * iters * 16 * 32768 FLOP.  Asynchronous on
 * `stream`.  Returns ATTN_E_NULL, ATTN_E_ALIGN, ATTN_E_SHAPE (blocks or
 * iters < 1), ATTN_E_UNSUPPORTED (unknown dtype), ATTN_E_LAUNCH, else
 * ATTN_OK.  Used for the board's sustained matrix-core rate under its power
 * limit, the context for the published peak the kernels are priced against.
 */
int attn_debug_calib_mfma(int32_t dtype, const void* operands, float* out, int32_t blocks, int32_t iters,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_DEBUG_H */
