/*
 * asv.h -- the shared-round verify step of LFM2 speculative decoding on
 * AMD Instinct MI355X (gfx950): a plain C ABI.
 *
 * Where the operations come from (the pages' problem statement):
 *   PR #1377 "LFM2: shared-round decode" -- commit log and "What this
 *   changes": a shared round of several streams runs each layer's short conv
 *   and attention ONCE over all rows of all streams, driven by one table
 *   that says per stream where its caches live, where its rows start and how
 *   many keys it holds, with each stream's attention partials held apart; a GPU argmax picks each head row's first
 *   largest logit and flags rows holding a nonfinite logit, so the host only
 *   draws flagged, sampled or masked rows.
 *
 * The library computes, per layer and over every live stream at once:
 *   asv_shared_conv   gated short conv against each stream's own conv state
 *   asv_shared_attn   GQA attention split over keys, partials per stream
 *   asv_attn_merge    merge of each row's split partials
 *   asv_row_argmax    greedy pick + nonfinite flag per logit row
 * from a table built once per round on the host (asv_seg_table_build) and
 * copied to the device (asv_table_upload).
 *
 * Conventions for every call:
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Every pointer is a DEVICE pointer unless its comment says "host".
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Kernels are enqueued asynchronously on it; faults surface at the
 *     caller's next synchronisation.
 *   - The caller owns every buffer. The library allocates nothing and keeps
 *     no mutable global state; calls are reentrant.
 *   - Return value: ASV_OK (0) or a negative ASV_E_* code; nothing is
 *     launched and nothing is written when a call returns an error.
 *   - Buffers reached only through the table (conv states, K/V caches) are
 *     invisible to any caching allocator of the caller: they must stay alive
 *     until the work enqueued on `stream` has finished.
 */
#ifndef ASV_H
#define ASV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ASV_ABI_VERSION 4

/* Model dimensions compiled into the kernels (LFM2.5-24B-A2B shapes). */
#define ASV_HIDDEN 2048          /* conv channels, attention row width      */
#define ASV_CONV_IN 6144         /* conv input row: B | C | x, 2048 each     */
#define ASV_CONV_WIDTH 3         /* conv taps                                */
#define ASV_Q_HEADS 32
#define ASV_KV_HEADS 8           /* q head h reads kv head h / 4             */
#define ASV_HEAD_DIM 64
#define ASV_TILE_ROWS 16         /* rows of one tile, never across streams   */
#define ASV_KEY_BLOCK 32         /* V cache block; capacities are multiples  */
#define ASV_MAX_ROWS 2048        /* rows of one round (the served scratch)   */
#define ASV_MAX_KEYS 131072      /* keys (and capacity) of one stream        */
#define ASV_PARTIAL_FLOATS 66    /* floats per partial record: o[64], m, l   */

/* Error codes. */
#define ASV_OK 0
#define ASV_E_ARG (-1)           /* null, misaligned or aliasing pointer      */
#define ASV_E_SHAPE (-2)         /* rows / keys / capacity / layer out of range */
#define ASV_E_UNSUPPORTED (-3)   /* a dimension other than the compiled one   */
#define ASV_E_CAPACITY (-4)      /* caller buffer too small (size reported)   */
#define ASV_E_HIP (-5)           /* the HIP runtime refused a copy or launch  */

/* One live stream of the round (host).
 *   rows        window rows this round (draft rows, or a prompt chunk), >= 1
 *   key_count   keys in the stream's cache INCLUDING the window's own rows;
 *               window row i (0-based) sees keys [0, key_count - rows + i + 1)
 *   kv_capacity slots in the stream's K/V cache, a multiple of 32,
 *               key_count <= kv_capacity <= 131072                          */
typedef struct {
  int32_t rows;
  int32_t key_count;
  int32_t kv_capacity;
} asv_stream_desc;

/* Table arrays, as laid out inside the blob (all little-endian). */
typedef struct {      /* one per stream, caller order                     */
  int32_t row0;       /* first row of the stream (exclusive prefix sum)   */
  int32_t rows;
  int32_t keys;
  int32_t cap;
  int32_t split_keys; /* A: keys in each of the first nbig splits        */
  int32_t nsplit;     /* n = ceil(keys / C), C = 768, 1024, 2560, 7168 or
                         5120 by the stream's rows (<= 2, <= 4, <= 8, <= 16,
                         more)                                            */
  int64_t poff;       /* first partial record of the stream               */
  int32_t split_tail; /* B: keys in each later split (the last one ends
                         at keys)                                         */
  int32_t nbig;       /* splits of A keys; split t starts at t*A for
                         t < nbig, else nbig*A + (t - nbig)*B             */
  int32_t reserved[2];
} asv_seg;
/* The split plan depends only on the stream's rows and keys. Windows of up
 * to 8 rows: n equal splits, A = B = ceil(keys / n) rounded up to 32 and
 * nbig = n. Longer windows (16-row tiles) with n >= 2: nbig = ceil(n / 2)
 * splits of A = ceil(5 keys / (5 nbig + 4 (n - nbig))) rounded up to 32,
 * then n - nbig splits of B = ceil((keys - nbig A) / (n - nbig)) rounded up
 * to 32, about 4/5 of A (equal splits if that left a split empty). */

typedef struct {      /* one per row                                       */
  int32_t stream;
  int32_t pos;        /* row index inside its stream's window             */
  int32_t nkeys;      /* keys the row sees: keys - rows + pos + 1 (causal),
                         keys (asv_block_table_build)                      */
  int32_t tile;
} asv_row;

typedef struct {      /* runs of <= 16 rows of one stream                  */
  int32_t stream;
  int32_t row0;
  int32_t nrows;
  int32_t pos0;
} asv_tile;

typedef struct {      /* one attention work item: (tiles, kv head, split) */
  int32_t tile;       /* its first tile                                   */
  int8_t head;
  int8_t ntiles;      /* 1: one tile, its keys striped over the block's
                         waves; 2-4: that many consecutive tiles of one
                         stream, a wave each, every wave walking all of
                         the split's keys (streams of more than one tile
                         are cut into groups of 4 tiles, the last shorter) */
  int16_t stream;     /* the tiles' stream (also in the tile records; here
                         so that a block reads its stream's records and
                         K/V addresses beside its tile record, not after) */
  int32_t split;
  int32_t keys;       /* keys the item visits: the split's keys that the
                         last row of its last tile sees                   */
} asv_work;
/* The work list holds each kind of item by cost, largest first (keys for
 * one-tile items, 4 x keys for groups, whose waves each walk every key), the
 * two kinds in alternating runs of 256 items, groups first. */

/* What asv_seg_table_build reports (host). Offsets are byte offsets of the
 * arrays inside the blob; the same struct is passed back to every call. */
typedef struct {
  int32_t abi_version;
  int32_t n_streams;
  int32_t n_rows;
  int32_t n_tiles;
  int32_t n_work;
  int32_t n_conv_layers;
  int32_t n_attn_layers;
  int32_t max_tile_rows;
  int64_t partial_count;   /* partial records (ASV_PARTIAL_FLOATS floats each) */
  int64_t blob_bytes;
  int64_t off_segs;        /* asv_seg[n_streams]                              */
  int64_t off_rows;        /* asv_row[n_rows]                                 */
  int64_t off_tiles;       /* asv_tile[n_tiles]                               */
  int64_t off_work;        /* asv_work[n_work], in the order described above  */
  int64_t off_conv_state;  /* uint64 device addresses [n_conv_layers][n_streams] */
  int64_t off_k;           /* uint64 device addresses [n_attn_layers][n_streams] */
  int64_t off_v;           /* uint64 device addresses [n_attn_layers][n_streams] */
} asv_table_info;

int asv_abi_version(void);
const char* asv_strerror(int code);

/* Build the round's segment table on the host (no HIP call).
 *
 * Defines: PR #1377 "LFM2: shared-round decode", shared-round commit (one
 * per-stream table of cache addresses, first rows and key counts; a row map and
 * tiles; the partials of each stream kept apart, their count checked at 1,
 * 32 and 2,048 rows).
 *
 *   streams        host, n_streams descriptors in caller order
 *   conv_state     host, [n_conv_layers][n_streams] device addresses of each
 *                  stream's conv state: bf16 [2][2048], 16-byte aligned,
 *                  read AND written by asv_shared_conv (may be NULL when
 *                  n_conv_layers == 0)
 *   k_cache        host, [n_attn_layers][n_streams] device addresses of each
 *                  stream's K cache: bf16 [8][kv_capacity][64]
 *   v_cache        host, [n_attn_layers][n_streams] device addresses of each
 *                  stream's V cache: bf16 [8][kv_capacity/32][64][32], i.e.
 *                  key j, dim d of kv head g at
 *                  ((g*(kv_capacity/32) + j/32)*64 + d)*32 + j%32
 *                  (both may be NULL when n_attn_layers == 0)
 *   blob, blob_bytes  host output buffer; blob == NULL asks for the size only
 *   info           host output: sizes and array offsets (always filled when
 *                  the descriptors are valid)
 *
 * Errors: ASV_E_SHAPE when n_streams < 1, a stream has rows < 1,
 * key_count < rows, key_count > 131072, kv_capacity not a multiple of 32,
 * below key_count or above 131072, more than 2048 rows in total, or a
 * negative layer count; ASV_E_ARG for a null or misaligned address, or when
 * two streams' buffers of one layer overlap (every stream reads and writes
 * only its own state and cache); ASV_E_CAPACITY when blob is non-NULL and
 * blob_bytes < info->blob_bytes. The blob is written only on success. */
int asv_seg_table_build(const asv_stream_desc* streams, int32_t n_streams,
                        const void* const* conv_state, int32_t n_conv_layers,
                        const void* const* k_cache, const void* const* v_cache,
                        int32_t n_attn_layers, void* blob, size_t blob_bytes,
                        asv_table_info* info);

/* The same table for block (non-causal) attention.
 *
 * Defines: PR #1391 "lfm2: draft with LiquidAI's DSpark drafter
 * (--drafter)", its list of new kernels (the target's attention and merge
 * with a FULL flag, every block row seeing the keys [0, len + 1), beside the
 * target's causal instantiations) and the drafter's description (a block of
 * the pending token and mask tokens attends non-causally). Read as: every row
 * of stream s sees all K_s keys of its cache, so the window's rows attend to
 * each other in both directions.
 *
 * Arguments, layout, ownership and errors are those of asv_seg_table_build;
 * the only differences are in the blob: every asv_row has nkeys = key_count,
 * and the work list holds every split of the stream for every tile.
 * asv_shared_attn and asv_attn_merge take either table: they read each row's
 * visible key count from the table. */
int asv_block_table_build(const asv_stream_desc* streams, int32_t n_streams,
                          const void* const* conv_state, int32_t n_conv_layers,
                          const void* const* k_cache, const void* const* v_cache,
                          int32_t n_attn_layers, void* blob, size_t blob_bytes,
                          asv_table_info* info);

/* Copy a built blob (host) to the device, where every launch reads it.
 *
 * Defines: PR #1377 "LFM2: shared-round decode", shared-round commit (the
 * round's table is written once on the host and read by every layer's
 * launches on the GPU).
 *
 *   blob, bytes  host, the blob asv_seg_table_build or asv_block_table_build
 *                wrote, bytes = info->blob_bytes; it must stay unchanged
 *                until the copy has run (pinned host memory makes the copy
 *                asynchronous)
 *   dev_blob     device, >= bytes, 16-byte aligned; owned by the caller
 * bytes == 0 copies nothing and returns ASV_OK.
 * Errors: ASV_E_ARG (null blob or dev_blob, dev_blob not 16-byte aligned),
 * ASV_E_HIP (the runtime refused the copy). */
int asv_table_upload(const void* blob, size_t bytes, void* dev_blob, void* stream);

/* Gated short conv of one layer over every row of the round.
 *
 * Defines: PR #1377 "LFM2: shared-round decode", shared-round commit (one
 * conv launch a layer over every row, each row against its own stream's conv
 * state, checked against a host replay of the conv steps); the dense-twin
 * commit (a 6,144-wide conv input from 2,048-wide rows).
 *
 * For row i of stream s (rows in window order):
 *   B, C, x = X[r][0:2048], X[r][2048:4096], X[r][4096:6144]
 *   bx_i = bf16(B * x)                              (round to nearest even)
 *   h = [state_s[0], state_s[1], bx_0, bx_1, ...]
 *   Y[r][c] = bf16(C[c] * (W[c][0] h_i[c] + W[c][1] h_{i+1}[c] + W[c][2] h_{i+2}[c]))
 * in fp32 (taps accumulated in order 0, 1, 2), and afterwards
 * state_s = [h_w, h_{w+1}] (bit-exact: the rounded bx values).
 *
 *   x  bf16 [n_rows][6144], y bf16 [n_rows][2048], w bf16 [2048][3] (this
 *   layer's weights); all 16-byte aligned. Writes y and this layer's conv
 *   states, nothing else.
 * Errors: ASV_E_ARG (null/misaligned), ASV_E_SHAPE (layer out of range),
 * ASV_E_HIP (launch failed). */
int asv_shared_conv(const asv_table_info* info, const void* dev_blob, int32_t layer,
                    const uint16_t* x, const uint16_t* w, uint16_t* y, void* stream);

/* Split-K GQA attention of one layer over every row of the round.
 *
 * Defines: PR #1377 "LFM2: shared-round decode", shared-round commit (one
 * attention launch a layer over every stream's rows, partials of each stream
 * held apart, checked against float64 attention); with a table from
 * asv_block_table_build, PR #1391's block attention (FULL flag).
 *
 * Row r of stream s, q head h (kv head g = h / 4), split t covering keys
 * [t*S_s, (t+1)*S_s) of the n_r keys the row sees (the table's count: causal
 * from asv_seg_table_build, all K_s from asv_block_table_build), scores
 * s_j = (q . k_j) / 8, writes record p = poff_s + (t*rows_s + pos_r)*32 + h:
 *   o[p][0:64] = sum_j e^(s_j - m) v_j / l,  m = max_j s_j,  l = sum_j e^(s_j - m)
 * (an empty split writes m = -inf, l = 0, o = 0). Keys past a stream's key
 * count are never used: their V slots are read as zero and their scores
 * masked, so they may hold anything (NaN included).
 * Precision: fp32 accumulation; the weights e^(s_j - m) enter the products
 * with ~16 bits (bf16 hi + lo) for streams of at most 16 rows, and rounded
 * to fp16 (11 bits, V scaled exactly into fp16 by a power of 2 per 16-wide
 * d tile) for longer streams (prompt chunks). Within 1e-3 of the record's
 * largest |o| and 1e-3 of l on the tested workloads (largest seen: 5e-4
 * for chunks, 2e-5 otherwise).
 *
 *   q         bf16 [n_rows][32][64], 16-byte aligned
 *   partials  float [info->partial_count * 66], 16-byte aligned: the o
 *             records first ([partial_count][64]) then (m, l) pairs
 *             ([partial_count][2]); m is in score units (natural log).
 * Writes only the records of the round's rows; reads K/V only.
 * Errors: ASV_E_ARG, ASV_E_SHAPE (layer out of range), ASV_E_HIP. */
int asv_shared_attn(const asv_table_info* info, const void* dev_blob, int32_t layer,
                    const uint16_t* q, float* partials, void* stream);

/* Merge each row's split partials into its attention output.
 *
 * Defines: PR #1377 "LFM2: shared-round decode", inline-bodies and
 * shared-round commits (the merge body run once over every row).
 *
 * For row r, q head h over its splits t < ceil(n_r / S_s), in split order:
 *   M = max_t m_t,  O[r][h] = bf16( sum_t e^(m_t - M) l_t o_t / sum_t e^(m_t - M) l_t )
 *   o  bf16 [n_rows][32][64] (= [n_rows][2048]), 16-byte aligned.
 * Errors: ASV_E_ARG, ASV_E_HIP. */
int asv_attn_merge(const asv_table_info* info, const void* dev_blob, const float* partials,
                   uint16_t* o, void* stream);

/* Workspace bytes asv_row_argmax needs for `rows` rows of `vocab` logits. */
size_t asv_row_argmax_workspace(int64_t rows, int64_t vocab);

/* Greedy pick and nonfinite flag of every logit row.
 *
 * Defines: PR #1377 "LFM2: shared-round decode", GPU-pick commit and the
 * kernel contract entry (the host draw's pick: the first largest logit, ties
 * to the lower id; a row holding a nonfinite logit is flagged).
 *
 * pick[r] = the lowest id whose value is the largest non-NaN value of the
 * row (+Inf and -Inf order as usual, -0 equals +0); 0 when every value is
 * NaN. flag[r] = 1 when the row holds a NaN or an infinity, else 0. A flagged
 * row is data, not an error: the caller draws it on the host.
 *
 *   logits     bf16, row r at logits + r*row_stride, 16-byte aligned,
 *              row_stride a multiple of 8 and >= vocab
 *   pick       int32 [rows];  flag  uint8 [rows]
 *   workspace  >= asv_row_argmax_workspace(rows, vocab) bytes, 16-byte
 *              aligned, contents ignored on entry
 * Errors: ASV_E_ARG, ASV_E_SHAPE (rows < 0, vocab < 1 or > 2^30),
 * ASV_E_CAPACITY (workspace too small), ASV_E_HIP. rows == 0 launches
 * nothing and returns ASV_OK. */
int asv_row_argmax(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t row_stride,
                   int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Bytes of the device array asv_row_argmax_noalloc uses as its workspace. */
#define ASV_ARGMAX_SCRATCH_BYTES (4u << 20)

/* asv_row_argmax without a caller workspace and without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same pick,
 * flag, arguments (minus the workspace), layout and results as
 * asv_row_argmax, bit for bit; the two launches are the same kernels.
 *
 * Workspace: a library-owned device array of ASV_ARGMAX_SCRATCH_BYTES
 * (4 MiB) on each GPU the library runs on, held until the process ends;
 * its address is resolved on the first call on a device (no allocation,
 * no copy). So asv_row_argmax_workspace(rows, vocab) must not exceed 4 MiB:
 * rows * ceil(vocab / 8192) <= 262,144 (e.g. 2,048 rows of up to 1,048,576
 * logits, or 16,384 rows of 128,000). Nothing in the array needs clearing:
 * every record is written before it is read.
 *
 * Every call on one GPU shares that GPU's array: calls whose work overlaps
 * in time on one GPU (on two streams, or from two host threads without
 * ordering) race on it and give undefined picks. Calls on one stream, one
 * after the other, are safe.
 *
 * Errors: those of asv_row_argmax; ASV_E_CAPACITY when the workspace the
 * call needs exceeds ASV_ARGMAX_SCRATCH_BYTES; ASV_E_HIP when the array's
 * device address cannot be resolved. rows == 0 launches nothing. */
int asv_row_argmax_noalloc(const uint16_t* logits, int64_t rows, int64_t vocab,
                           int64_t row_stride, int32_t* pick, uint8_t* flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ASV_H */
