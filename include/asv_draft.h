/* asv_draft.h -- C ABI of the drafter-side kernels that pair with the
 * shared-round verify step: the device draft-id gather and the Markov-head
 * step (PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)").
 *
 * Conventions as in asv.h (return codes, ownership, streams): every
 * buffer is the caller's, nothing is allocated, and a call enqueues its
 * launches on `stream` (a hipStream_t; NULL is the null stream).
 */
#ifndef ASV_DRAFT_H
#define ASV_DRAFT_H

#include "asv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {      /* one stream's drafts for asv_draft_ids             */
  int32_t src;        /* first pick of the stream                          */
  int32_t dst;        /* id slot the first pick goes to                    */
  int32_t count;      /* picks to copy (0 or less: none)                   */
} asv_draft_span;

#define ASV_MARKOV_MAX_CHAINS 32   /* chains of one Markov call               */
#define ASV_MARKOV_MAX_DEPTH 16    /* rows of one chain (the drafter trains 9) */
#define ASV_MARKOV_MAX_RANK 256    /* W1/W2 rank (the pages admit up to 256)   */

typedef struct {      /* one drafted block for asv_markov_pick             */
  int32_t row0;       /* first row of the block's logits and picks          */
  int32_t depth;      /* rows row0 .. row0 + depth - 1, one after the other */
} asv_markov_chain;

/* Copy each stream's drafts from the picks into the verify ids, with a
 * failure flag per stream.
 *
 * Defines: PR #1391 "lfm2: draft with LiquidAI's DSpark drafter
 * (--drafter)", description: a device kernel moves the drafter's picks for
 * every window into the id array the verify step consumes, an id past the
 * vocabulary becoming 0; its held-draft fix: a per-stream flag, checked
 * before the caches are committed, fails a window whose pick is invalid or
 * came from a row with a NaN or an infinity (DraftNonfinite).
 *
 * For stream s (span = spans[s]) and i < span.count:
 *   p = pick[span.src + i];  ids[span.dst + i] = (0 <= p < vocab) ? p : 0
 *   fail[s] = 1 when some p is outside [0, vocab) or pick_flag[span.src + i]
 *             is set (the argmax saw a NaN or an infinity), else 0.
 * A span with count <= 0 copies nothing and does not fail. An entry whose
 * pick or id index falls outside [0, n_picks) or [0, n_ids) fails its
 * stream and writes nothing. ids outside the spans are untouched. Streams
 * run in parallel: source ranges may overlap, destination ranges must not
 * (where they do, which stream's id remains is unspecified).
 *
 *   spans      device, asv_draft_span [n_streams], 4-byte aligned
 *   pick       device, int32 [n_picks] (asv_row_argmax's picks)
 *   pick_flag  device, uint8 [n_picks] (asv_row_argmax's flags)
 *   ids        device, int32 [n_ids], written inside the spans only
 *   fail       device, uint8 [n_streams], all written
 * Errors: ASV_E_SHAPE for a negative count or size or vocab < 1; ASV_E_ARG
 * for a null or misaligned pointer; ASV_E_HIP. n_streams == 0 launches
 * nothing. */
int asv_draft_ids(const asv_draft_span* spans, int32_t n_streams, const int32_t* pick,
                  const uint8_t* pick_flag, int64_t n_picks, int64_t vocab, int32_t* ids,
                  int64_t n_ids, uint8_t* fail, void* stream);

/* Markov-head step of the drafter: each drafted row's pick and flag.
 *
 * Defines: PR #1391 "lfm2: draft with LiquidAI's DSpark drafter
 * (--drafter)", description and new-kernel list: the drafter's Markov head
 * scores each row of the block as its logits plus the low-rank term
 * W2 . W1[token before the row] and picks that row's argmax before it moves
 * to the next row, whose previous token is that pick (lowest token on a
 * tie, a NaN score flagged); the testing notes give the score as
 * bf16(base + bf16(W2 . W1[prev])) at 1 x 128,000 x 256 (rows x vocabulary
 * x rank); the config admission caps the rank at 256.
 *
 * For chain c (chains[c] = {row0, depth}) and j < depth, row r = row0 + j:
 *   prev = j == 0 ? prev0[c] : pick[r - 1]
 *   dot_v = sum_k W2[v][k] * W1[prev][k]   in float32, k = 0, 1, .. rank-1,
 *           one rounding per term (the bf16 x bf16 product is exact)
 *   score_v = bf16(fl32(base[r][v] + bf16(dot_v)))   (round to nearest even)
 *   pick[r] = the lowest v with the largest score (NaN skipped, -0 == +0;
 *             0 when every score is NaN)
 *   flag[r] = 1 when some score is NaN or an infinity, or prev is outside
 *             [0, vocab) (then dot_v is taken as +0 and W1 is not read)
 * Rows outside the chains are not written.
 *
 *   base       device, bf16 [rows][row_stride] (the block rows' logits)
 *   chains     HOST, asv_markov_chain [n_chains]; rows in range, disjoint
 *   prev0      device, int32 [n_chains] (each chain's first previous token)
 *   w1         device, bf16 [vocab][rank], 16-byte aligned
 *   w2c        device, bf16 W2 in tiles of 64 tokens, each [rank/8][tl][8]
 *              (tl = 64, or vocab % 64 for a shorter last tile): element
 *              (v, k) at (64 * rank * t + (k / 8) * tl + v - 64 t) * 8 + k % 8,
 *              t = v / 64 (asv_markov_pack_w2); vocab * rank elements
 *   pick, flag device, int32 / uint8 [rows]
 *   workspace  device, asv_markov_workspace(vocab) bytes, 16-byte aligned;
 *              one call at a time per workspace (two halves of block
 *              records, depths alternating)
 * Two forms on `stream`, the same bits from either (asv_markov_pick_form
 * chooses; asv_markov_pick takes ASV_MARKOV_AUTO):
 *   resident: a clearing launch and one launch of 512-token blocks that
 *     all run at once, each wave keeping its 64 tokens of W2 in registers
 *     for every depth (W2 read once a pass); the blocks trade depth-tagged
 *     8-byte records through the workspace between depths. Admitted when
 *     ceil(vocab / 512) <= 512 and every block fits on the device at once
 *     (one a CU: vocab <= 131,072 at rank 256 on a 256-CU device). Its
 *     blocks wait for each other, so it needs them all running together:
 *     run one resident pass at a time on a device (order calls made on
 *     different streams), and expect other work on the device to delay
 *     it. A block that waits more than a second for a record abandons the
 *     pass: flag 2 on every row of the depth it waited for and the later
 *     ones (pick then undefined there).
 *   launches: one launch a depth plus one: the launch of depth j + 1 folds
 *     depth j's 4-byte block records (256-token blocks) for its previous
 *     tokens (its block 0 writes depth j's picks and flags), and the last
 *     launch folds the deepest depth; W2 is read once a depth.
 * The host never reads a pick.
 * Errors: ASV_E_SHAPE (n_chains > ASV_MARKOV_MAX_CHAINS, a depth outside
 * 1..ASV_MARKOV_MAX_DEPTH, a chain outside [0, rows) or two chains sharing a
 * row, vocab < 1 or > 2^30, row_stride < vocab); ASV_E_UNSUPPORTED (rank not
 * a multiple of 8 in 8..256); ASV_E_ARG (null or misaligned pointer);
 * ASV_E_CAPACITY (workspace too small); ASV_E_HIP. n_chains == 0 launches
 * nothing. */
size_t asv_markov_workspace(int64_t vocab);
int asv_markov_pick(const uint16_t* base, int64_t rows, int64_t row_stride,
                    const asv_markov_chain* chains, int32_t n_chains, const int32_t* prev0,
                    const uint16_t* w1, const uint16_t* w2c, int64_t vocab, int32_t rank,
                    int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                    void* stream);

/* asv_markov_pick with its form chosen: ASV_MARKOV_AUTO (resident when it
 * is admitted, else launches), ASV_MARKOV_LAUNCHES, or ASV_MARKOV_RESIDENT
 * (ASV_E_UNSUPPORTED when not admitted on this device and rank).
 * Defines: as asv_markov_pick. Errors: as asv_markov_pick, and ASV_E_ARG for
 * an unknown form. */
#define ASV_MARKOV_AUTO 0
#define ASV_MARKOV_LAUNCHES 1
#define ASV_MARKOV_RESIDENT 2
int asv_markov_pick_form(const uint16_t* base, int64_t rows, int64_t row_stride,
                         const asv_markov_chain* chains, int32_t n_chains, const int32_t* prev0,
                         const uint16_t* w1, const uint16_t* w2c, int64_t vocab, int32_t rank,
                         int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                         int32_t form, void* stream);

/* W2 [vocab][rank] (row-major bf16, as the checkpoint holds it) into the
 * tiled layout asv_markov_pick reads; once, when the weights load.
 * Plain data movement, no arithmetic. Errors: ASV_E_SHAPE (vocab),
 * ASV_E_UNSUPPORTED (rank), ASV_E_ARG (null, misaligned or overlapping). */
int asv_markov_pack_w2(const uint16_t* w2, int64_t vocab, int32_t rank, uint16_t* w2c,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ASV_DRAFT_H */
