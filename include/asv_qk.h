/* asv_qk.h -- C ABI of the qk stage of an attention layer of the
 * shared-round verify step: q and k head norm, half-split RoPE, and the
 * window's K and V appended to every stream's cache, one launch a layer over
 * every row through the table that asv_seg_table_build wrote.
 *
 * Conventions as in asv.h (return codes, ownership, streams, cache layouts).
 */
#ifndef ASV_QK_H
#define ASV_QK_H

#include "asv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ASV_QKV_WIDTH 3072   /* a row's qkv projection: q 32x64 | k 8x64 | v 8x64 */

/* The qk stage of attention layer `layer` over every row of the table.
 *
 * Defines: PR #1377 "LFM2: shared-round decode" (per stream an attention
 * layer is a qk launch, the attention and the merge; the shared round runs
 * each once a layer over every row through the table of cache addresses,
 * row offsets and key counts; the inline-bodies commit names the qk row
 * body); PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)"
 * (the target's RoPE kernel is half-split and the q and k rows carry norm
 * gains; a rope theta that is not finite must be refused).
 *
 * For row r of stream s at window position p, key position
 * pos = keys_s - rows_s + p, and each head x of 64 values:
 *   y = x / sqrt(mean(x^2) + eps) * gain          (q heads: q_gain, k: k_gain)
 *   for i < 32, a_i = pos * theta^(-i/32):
 *     out_i = y_i cos a_i - y_{i+32} sin a_i,  out_{i+32} = y_{i+32} cos a_i + y_i sin a_i
 * rounded to bf16 (nearest even). q goes to q_out[r][h][:]; k goes to the
 * stream's K cache at [kv head][pos][:] and v, copied exactly, to its V cache
 * at key pos (the layouts of asv.h). Nothing else in the caches is written.
 * The angles are formed and reduced in float64; the norm and the rotation
 * run in float32, so an output is within one bf16 step of the float64 value
 * rounded once, away from cancellation.
 *
 *   qkv     device, bf16 [n_rows][ASV_QKV_WIDTH], 16-byte aligned
 *   q_gain, k_gain  device, bf16 [64], 16-byte aligned
 *   q_out   device, bf16 [n_rows][32][64], 16-byte aligned (may not alias qkv)
 * Errors: ASV_E_ARG (null, misaligned or aliasing pointer, a table from
 * another build); ASV_E_SHAPE (layer out of range; theta not a finite
 * number > 0, eps not a finite number >= 0); ASV_E_HIP. */
int asv_shared_qk(const asv_table_info* info, const void* dev_blob, int32_t layer,
                  const uint16_t* qkv, const uint16_t* q_gain, const uint16_t* k_gain,
                  double theta, double eps, uint16_t* q_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ASV_QK_H */
