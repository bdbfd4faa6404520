/*
 * ds4attn.h -- C ABI of the fused multi-query FlashAttention step for MI355X (gfx950).
 *
 * One attention step of the DeepSeek V4 Flash engine: every query head of a
 * token attends, with one shared K/V head, to the rows of two KV regions under
 * one softmax.  Region 0 holds the raw sliding-window rows, region 1 the pooled
 * compressed rows, either all of them or a per-token index list.  It runs in three
 * stages:
 *
 *   ds4attn_pad       KV rows padded to 32-row blocks
 *   ds4attn_blockmap  one status byte per (query tile, KV block): skip / partial / full
 *   ds4attn_decode    fused Q.K^T, online softmax and P.V (tuned for few tokens)
 *   ds4attn_prefill   the same computation, tuned for long token chunks
 *
 * and three steps around it: ds4attn_quantize_fp8 (K/V rows into the FP8 cache
 * format), ds4attn_topk (an index list from given scores) and ds4attn_compress
 * (raw rows pooled into compressed rows).
 *
 * Pages the operations follow:
 *   [P-Metal] "How DeepSeek V4 Flash Model Inference Works on Apple Silicon with
 *             Metal Backend" (instagit.com, antirez/ds4)
 *   [P-DS4]   "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine"
 *             (wikichat.gnat.co, summary of ds4.md)
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are HIP device addresses; the caller owns every
 *     buffer.  The library allocates nothing, frees nothing, keeps no pointer past
 *     the call and has no mutable global state; calls are thread-safe.  (One
 *     exception: ds4attn_decode_noalloc keeps its scratch in a static per-device
 *     array, see there.)
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = the null stream)
 *     and runs asynchronously; the library never synchronises.
 *   - Arguments are checked before anything is enqueued.  On any nonzero
 *     return nothing was enqueued (except DS4ATTN_E_HIP, which reports a
 *     failed launch).  A fault while the kernels run surfaces at the caller's
 *     next synchronisation.  No C++ exception crosses this boundary.
 *   - Byte strides: every stride is in bytes and must be a multiple of 16;
 *     every device pointer to K, V, Q or O must be 16-byte aligned.  Rows of K,
 *     V, Q and O are contiguous along the head dimension.
 *   - Output O is always float32, [batch][n_tok][n_head][head_dim] by strides.
 */
#ifndef DS4ATTN_H
#define DS4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  DS4ATTN_OK = 0,
  DS4ATTN_E_INVAL = 1,        /* a null pointer, a negative size, a bad stride or alignment */
  DS4ATTN_E_UNSUPPORTED = 2,  /* a valid request this build has no kernel for */
  DS4ATTN_E_WORKSPACE = 3,    /* a workspace smaller than the call needs */
  DS4ATTN_E_HIP = 4           /* the HIP runtime refused a launch */
};

/* Element types.  Q, and K/V stored plainly, are F16 or F32 (the same type);
 * E4M3 is the element type of quantized K/V rows (OCP FP8 E4M3: bias 7, 3
 * mantissa bits, no infinities, 0x7F/0xFF NaN, largest value 448).  O is always
 * float32. */
enum { DS4ATTN_F16 = 0, DS4ATTN_F32 = 1, DS4ATTN_E4M3 = 2 };

/* Storage of K and V rows (ds4attn_args.kv_format).
 *   PLAIN:     elements of ds4attn_args.dtype.
 *   FP8_E4M3:  E4M3 codes with one float32 scale per K row and one per V row
 *              (region.k_scale / v_scale); a row's value is decode(code) * scale.
 *              This is the cache format ds4attn_quantize_fp8 writes ([P-DS4]
 *              "Architecture Deep Dive", Whole-Model Graph Execution: K/V rows are
 *              quantized to FP8 before they are stored; the element format and the
 *              per-row scale are this library's choice, the pages give none).
 *              In the attention a K row's scale multiplies its scores in float32.
 *              The prefill kernel takes its scores from E4M3 x E4M3 matrix-core
 *              products of the K codes and the query carried as two E4M3 terms
 *              under a power-of-two factor per head, which reproduce each query
 *              element to within 2^-8 of itself (or 2^-14 of the factor, if that
 *              is larger); the decode kernels convert K codes to float16.  A V
 *              row's scale is folded into the softmax weight of that row: the
 *              weight P times the scale times a power of two, rounded once to
 *              float16, where the power of two follows the largest V scale seen
 *              so far and comes off the output in float32.  The weights thus keep
 *              float16's relative precision at any V magnitude, and every finite
 *              scale (ds4attn_quantize_fp8 writes amax/448 of finite rows) stays in
 *              range: the factor keeps scale times factor below 2^7 and P <= 2^8.
 *              No output or partial sum exceeds the V rows' magnitude, so the
 *              outputs are finite wherever every visible row's values (code times
 *              scale) are finite float32 values. */
enum { DS4ATTN_KV_PLAIN = 0, DS4ATTN_KV_FP8_E4M3 = 1 };

/* Status byte values of the block map ([P-Metal] "Mask Handling and Block Skipping":
 * a single-byte status per block; fully masked blocks are skipped).  FULL marks a
 * block whose every (token, row) pair is visible, so the mask need not be read. */
enum { DS4ATTN_BLK_SKIP = 0, DS4ATTN_BLK_PARTIAL = 1, DS4ATTN_BLK_FULL = 2 };

/* Flags of ds4attn_args.flags. */
enum {
  /* Run the generic vector-ALU kernel even where the matrix-core kernel applies
   * ([P-Metal] "Vector vs Non-Vector Execution Paths": a path that handles any
   * head size).  Results agree within rounding; it exists for cross-checks. */
  DS4ATTN_FLAG_GENERIC = 1,
  /* Decode on the matrix-core kernel only, with a chosen split of the work over a
   * workgroup's four waves (by default the library picks one from the length a
   * token's block list can reach).  DIMS: the waves share each key block and split
   * the head dimension, while four more waves move the blocks into LDS.  KEYS: the
   * waves take different key rows (16-row halves of float16 blocks, whole FP8
   * blocks) and merge their partial results at the end.
   * WIDE: DIMS over 32 heads per workgroup (two 16-head tiles per wave sharing
   * each operand read, half the workgroups), for n_head a multiple of 32 and no
   * index list; the library picks it when a batch has more groups of 16 heads
   * than the chip has CUs (256).  Setting more than one is DS4ATTN_E_INVAL; with
   * DS4ATTN_FLAG_GENERIC, or where the matrix-core kernel (or, for WIDE, its
   * conditions) does not apply, DS4ATTN_E_UNSUPPORTED, and ds4attn_decode_split
   * refuses WIDE.  Results agree within rounding; they exist for cross-checks and
   * measurement. */
  DS4ATTN_FLAG_DECODE_DIMS = 2,
  DS4ATTN_FLAG_DECODE_KEYS = 4,
  DS4ATTN_FLAG_DECODE_WIDE = 8
};

/* One KV region.  Row r of sequence b starts at  k + b*stride_b + r*stride_row
 * (same for v).  K and V may alias (one "KV" row, [P-DS4] KV Cache Design).
 * Rows [0, n_rows) are live; the attention kernels read whole 32-row blocks, so
 * rows [n_rows, ceil32(n_rows)) must exist (ds4attn_pad provides them).  Rows
 * that are masked are never allowed to reach the result, whatever they hold.
 * valid: device uint8 [batch][valid_stride_b bytes], nonzero = row visible, or
 * NULL = every live row visible.
 * k_scale, v_scale: FP8 rows only (kv_format DS4ATTN_KV_FP8_E4M3), else ignored:
 * device float32, the scale of row r of sequence b at byte offset
 * b*scale_stride_b + 4*r; only rows < n_rows are read.  The scales may alias. */
typedef struct ds4attn_region {
  const void *k;
  const void *v;
  const uint8_t *valid;
  const float *k_scale;
  const float *v_scale;
  int64_t stride_b;
  int64_t stride_row;
  int64_t valid_stride_b;
  int64_t scale_stride_b;
  int32_t n_rows;
  int32_t reserved;
} ds4attn_region;

/* Description of one attention call ([P-DS4] "Architecture Deep Dive":
 * 64 query heads, 1 KV head, head dim 512, 128-token sliding window, raw plus
 * compressed rows; ratio-4 layers attend an indexer's top-512 compressed rows).
 *
 * Visibility of key rows for token t of sequence b (t in [0, n_tok)):
 *   region 0 row j:  j < r0.n_rows, r0.valid[b][j] != 0 (if given), and when
 *                    window > 0:  0 <= (q_pos0 + t) - (k_pos0 + j) < window.
 *   region 1 row c:  r1_index == NULL: c < r1.n_rows and r1.valid[b][c] != 0 (if given);
 *                    r1_index != NULL: c = r1_index[(b*n_tok + t)*r1_k + e] for each
 *                    entry e with 0 <= c < r1.n_rows and r1.valid[b][c] != 0 (if
 *                    given); entries act as a multiset; other entries are unused.
 * O[b][t][h] = sum_a p_a V_a,  p = softmax_a(scale * Q[b][t][h] . K_a) over the
 * visible rows a of both regions; a token with no visible row gets O = 0. */
typedef struct ds4attn_args {
  int32_t batch;        /* B >= 0 independent sequences */
  int32_t n_tok;        /* T >= 0 query tokens per sequence */
  int32_t n_head;       /* H >= 1 query heads (one KV head) */
  int32_t head_dim;     /* D: 64, 128, 256 or 512 */
  int32_t dtype;        /* DS4ATTN_F16 or DS4ATTN_F32, for Q, K and V */
  int32_t flags;        /* DS4ATTN_FLAG_* */
  int64_t q_stride_b, q_stride_t, q_stride_h;   /* bytes */
  int64_t o_stride_b, o_stride_t, o_stride_h;   /* bytes (float32 output) */
  float scale;          /* softmax scale, normally (float)(1/sqrt(head_dim)) */
  int32_t window;       /* 0 = no positional mask on region 0 */
  int64_t q_pos0;       /* position of token 0 */
  int64_t k_pos0;       /* position of region-0 row 0 */
  ds4attn_region r0;    /* raw rows */
  ds4attn_region r1;    /* compressed rows; n_rows = 0 if absent */
  const int32_t *r1_index;  /* device int32 [B][T][r1_k], or NULL */
  int32_t r1_k;             /* entries per token when r1_index != NULL (1..2048) */
  int32_t kv_format;        /* DS4ATTN_KV_PLAIN (0) or DS4ATTN_KV_FP8_E4M3, both regions */
} ds4attn_args;

/*
 * ds4attn_pad -- pad one KV region to whole 32-row blocks
 * ([P-Metal] "KV-Cache Management on Metal Device Buffers": the cache is
 * padded to a multiple of 32 rows so the attention kernel reads full blocks;
 * "FlashAttention Kernel Architecture": the pad kernel aligns accesses to
 * 32-row boundaries).
 *
 *   in       region with in->n_rows live rows; in->k, in->v device [B][n_rows][head_dim]
 *            by in->stride_b / in->stride_row; in->valid optional.
 *   dtype    element type of the rows: DS4ATTN_F16, DS4ATTN_F32 or DS4ATTN_E4M3 (FP8
 *            codes; a zero code is +0.0; the per-row scales are not touched, the
 *            attention never reads the scale of a padding row).
 *   k_pad, v_pad  device outputs [B][ceil32(n_rows)][head_dim] by out_stride_b /
 *            out_stride_row.  Rows < n_rows are copied bit for bit; rows
 *            [n_rows, ceil32(n_rows)) are set to +0.0 (all bits zero).  If
 *            k_pad == in->k with equal strides (in place, the buffer already has
 *            the capacity) the live rows are left as they are; partly
 *            overlapping buffers are rejected.
 *   valid_pad  optional device uint8 [B][valid_pad_stride_b] output: byte r =
 *            in->valid[b][r] (or 1 without in->valid) for r < n_rows, 0 for the tail.
 *            valid_pad == in->valid with equal strides is in place (only the tail
 *            is written); other overlap with in->valid is rejected.
 * When every output is its input and n_rows is a multiple of 32 there is nothing
 * to write and no kernel is launched.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL or DS4ATTN_E_HIP.
 */
int ds4attn_pad(const ds4attn_region *in, int32_t batch, int32_t head_dim, int32_t dtype,
                void *k_pad, void *v_pad, int64_t out_stride_b, int64_t out_stride_row,
                uint8_t *valid_pad, int64_t valid_pad_stride_b, void *stream);

/*
 * ds4attn_blockmap -- the skip map ([P-Metal] "Mask Handling and Block Skipping":
 * the mask is scanned and one status byte is written per block; the attention
 * kernel skips fully masked blocks).
 *
 * Blocks are 32 KV rows of the dense part of the key space: the ceil32(r0.n_rows)/32
 * blocks of region 0, followed, when r1_index == NULL, by the ceil32(r1.n_rows)/32
 * blocks of region 1 (an indexed region has no shared blocks and is not mapped).
 * Query tiles are bq consecutive tokens (the last tile may be shorter).
 *   blk  device uint8 [B][ceil(n_tok/bq)][nb] written here, nb from ds4attn_blockmap_dims;
 *        byte = SKIP if no (token, row) pair of the tile x block is visible,
 *        FULL if every pair is (padding rows are never visible), else PARTIAL.
 * Only the mask fields of *a are read (sizes, window, positions, validity, r1_index
 * presence); q/o strides and dtype are ignored.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL or DS4ATTN_E_HIP.
 */
int ds4attn_blockmap(const ds4attn_args *a, int32_t bq, uint8_t *blk, void *stream);

/* Sizes of the map for *a and bq: *n_tiles = ceil(n_tok/bq), *n_blocks = nb.
 * Host only; returns DS4ATTN_OK or DS4ATTN_E_INVAL. */
int ds4attn_blockmap_dims(const ds4attn_args *a, int32_t bq, int64_t *n_tiles, int32_t *n_blocks);

/*
 * ds4attn_decode / ds4attn_prefill -- fused Q.K^T, online softmax and P.V in one
 * dispatch ([P-Metal] "FlashAttention Kernel Architecture": dot products,
 * softmax and weighted value sum fused into a single GPU dispatch), skipping the
 * blocks the map marks SKIP ([P-Metal] "Mask Handling and Block Skipping").
 *
 *   q    device [B][T][H][D] of a->dtype by a->q_stride_*
 *   blk  device map from ds4attn_blockmap with the same *a and this bq, or NULL
 *        (then no block is skipped and every block is masked pair by pair; the
 *        result is the same).  A bq larger than n_tok means one tile.
 *   o    device float32 [B][T][H][D] by a->o_stride_*; every element is written.
 *   workspace, workspace_bytes
 *        device scratch for the work split the library picks for this call
 *        (ds4attn_workspace_bytes gives its size; 0 bytes when the call runs
 *        unsplit).  decode divides each token's key blocks over several
 *        workgroups when the batch leaves most compute units idle (one sequence
 *        of a long-context layer), and combines the parts with the online-softmax
 *        rescale ([P-DS4] "Architecture Deep Dive", Whole-Model Graph Execution:
 *        the attention path depends on the layer's ratio and the batch size).
 *        NULL: no workspace, the call runs unsplit (same result up to rounding).
 *        Otherwise 16-byte aligned, not overlapping o, and at least the size
 *        ds4attn_workspace_bytes returns (else DS4ATTN_E_WORKSPACE); its contents
 *        on entry do not matter and it is free again once the call's work on
 *        `stream` has run.  prefill currently plans no split (0 bytes).
 * Both compute the same result.  decode splits the heads of a token over
 * several workgroups (for T = 1 and small batches); prefill keeps all heads of a
 * token in one workgroup (for 2048-token chunks,
 * [P-DS4] Whole-Model Graph Execution).  Supported: D in {64,128,256,512},
 * F16 or F32; D = 512 F16 with H % 16 == 0 runs on the matrix cores, the rest
 * on the vector-ALU kernel.  FP8 rows (a->kv_format = DS4ATTN_KV_FP8_E4M3) need
 * the matrix-core case (F16 Q, D = 512, H % 16 == 0, no DS4ATTN_FLAG_GENERIC);
 * the rows are 512 bytes of codes, strides multiples of 16 as above, and both
 * regions with live rows need k_scale and v_scale (4-byte aligned,
 * scale_stride_b a multiple of 4 and >= 4*n_rows when batch > 1); anything else
 * with FP8 rows returns DS4ATTN_E_UNSUPPORTED (shapes) or DS4ATTN_E_INVAL
 * (pointers, strides).
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL, DS4ATTN_E_UNSUPPORTED, DS4ATTN_E_WORKSPACE
 * or DS4ATTN_E_HIP.
 */
int ds4attn_decode(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq,
                   float *o, void *workspace, int64_t workspace_bytes, void *stream);
int ds4attn_prefill(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq,
                    float *o, void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes ds4attn_decode (is_prefill = 0) or ds4attn_prefill (nonzero)
 * uses for *a: B * T * (H / 16) * splits records of 16 * 512 * 4 + 128 bytes for
 * the split the library picks, 0 when it runs the call unsplit.  It depends on the
 * shapes, sizes, window, index length and flags of *a, not on its pointers.
 * Host only; returns the status ds4attn_decode / ds4attn_prefill would return for
 * the same *a before looking at q, blk and o (DS4ATTN_OK, DS4ATTN_E_INVAL or
 * DS4ATTN_E_UNSUPPORTED). */
int ds4attn_workspace_bytes(const ds4attn_args *a, int32_t is_prefill, int64_t *bytes);

/*
 * ds4attn_decode_noalloc -- ds4attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments without the workspace, same result and the same
 * work split: the split's records go to a static scratch array of the library
 * (8,421,376 bytes = 256 records, enough for every split the plan picks), of
 * which each device the library runs on holds its own copy until the process
 * ends.  Nothing is allocated, freed or cleared: every record is written before
 * it is read.
 *   - Calls on one device share that device's array and keep no result in it; two
 *     calls whose work overlaps in time on one device (different streams, or
 *     different host threads without ordering) race on it and may return wrong
 *     outputs.  Calls in order on one stream are safe.
 *   - `stream` must belong to the current device (NULL = its null stream), else
 *     DS4ATTN_E_INVAL.  The first call on a device looks up the array's address
 *     there (DS4ATTN_E_HIP if that fails).
 * Returns what ds4attn_decode returns, and DS4ATTN_E_WORKSPACE if a split needed
 * more than the array holds (the plan never does).
 */
int ds4attn_decode_noalloc(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq,
                           float *o, void *stream);

/* The query-tile size the prefill kernel is tuned for (a map built with any
 * bq >= 1 is accepted). */
int32_t ds4attn_prefill_bq(void);

/*
 * ds4attn_decode_split -- ds4attn_decode with a chosen split: each token's key
 * blocks divided over `splits` workgroups per group of 16 heads, for batches too
 * small to fill the chip (one sequence of a long-context layer: [P-DS4] "Architecture Deep Dive",
 * 32K-1M contexts; the fused step of [P-Metal] "FlashAttention Kernel
 * Architecture" run on parts of the block list).  Each part keeps its own running
 * maximum m_s, sum l_s and output O_s (normalised by l_s) in `workspace`; a second
 * kernel combines them: O = sum_s w_s O_s / sum_s w_s with w_s = 2^(m_s - M) l_s
 * and M = max_s m_s (the online-softmax rescale, applied once across parts; the
 * weights are normalised before the outputs are summed, so that no partial sum
 * exceeds the V rows' magnitude).  The result equals
 * ds4attn_decode's up to rounding.  (ds4attn_decode picks the split itself; this
 * entry point fixes it, for measurement and cross-checks.)
 *   splits     1..64; 1 runs unsplit (no workspace needed)
 *   workspace  device, 16-byte aligned, at least ds4attn_decode_workspace_bytes
 *              bytes (else DS4ATTN_E_WORKSPACE), not overlapping o; its contents
 *              on entry do not matter
 * Needs the matrix-core case (F16 Q, D = 512, H % 16 == 0, no DS4ATTN_FLAG_GENERIC;
 * either KV format), else DS4ATTN_E_UNSUPPORTED.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL, DS4ATTN_E_UNSUPPORTED, DS4ATTN_E_WORKSPACE
 * or DS4ATTN_E_HIP.
 */
int ds4attn_decode_split(const ds4attn_args *a, const void *q, const uint8_t *blk, int32_t bq,
                         float *o, int32_t splits, void *workspace, int64_t workspace_bytes,
                         void *stream);

/* Workspace bytes ds4attn_decode_split needs for *a and `splits` (0 for splits = 1):
 * B * T * (H / 16) * splits records of 16 * 512 * 4 + 128 bytes.  Host only;
 * returns DS4ATTN_OK, DS4ATTN_E_INVAL or DS4ATTN_E_UNSUPPORTED (H % 16 != 0). */
int ds4attn_decode_workspace_bytes(const ds4attn_args *a, int32_t splits, int64_t *bytes);

/*
 * ds4attn_topk -- top-k index selection from given scores: the index list of a
 * ratio-4 layer ([P-DS4] "Architecture Deep Dive", Layer Compression: each token
 * attends the top-512 compressed rows its indexer selects; the scoring itself is
 * learned and not computed here).
 *
 *   scores  device float32, row r (0 <= r < rows) at scores + r*score_stride bytes,
 *           n scores per row
 *   idx     device int32 output, row r at idx + r*idx_stride bytes, k entries: the
 *           indices of the min(k, n) largest scores of the row in ascending order,
 *           then -1 (an unused entry) up to k.  Scores compare by the IEEE total
 *           order of their bit patterns (-0 < +0; a NaN with the sign bit clear
 *           ranks above +inf, one with it set below -inf); equal scores go to the
 *           lower index, so the result is unique.
 *   0 <= rows <= 2^24, 0 <= n < 2^30, 1 <= k <= 2048; pointers and strides are multiples of 4
 *   bytes; score_stride >= 4*n and idx_stride >= 4*k when rows > 1; idx must not
 *   overlap the scores.  The output is a valid ds4attn_args.r1_index with r1_k = k.
 *   rows == 0 launches nothing.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL, DS4ATTN_E_UNSUPPORTED (rows > 2^24 or n >= 2^30) or
 * DS4ATTN_E_HIP.
 */
int ds4attn_topk(const float *scores, int64_t rows, int32_t n, int64_t score_stride, int32_t k,
                 int32_t *idx, int64_t idx_stride, void *stream);

/*
 * ds4attn_quantize_fp8 -- the FP8 KV quantize step ([P-DS4] "Architecture Deep
 * Dive", Whole-Model Graph Execution: K/V rows are quantized to FP8 before they
 * are stored in the cache; the format is this library's choice, see
 * DS4ATTN_KV_FP8_E4M3).
 *
 *   x       device rows [batch][n_rows][head_dim] of dtype (DS4ATTN_F16 or DS4ATTN_F32),
 *           row r of sequence b at x + b*x_stride_b + r*x_stride_row; finite values
 *   codes   device uint8 output, same indexing by code_stride_b / code_stride_row
 *   scales  device float32 output, row r of sequence b at byte b*scale_stride_b + 4*r
 * Per row, in float32: amax = max |x|, scale = amax / 448; each code is the E4M3
 * value nearest to x / scale clamped to [-448, 448], ties to even mantissa, with
 * the sign bit of x / scale; a row with scale 0 gets zero codes.
 * head_dim in {64, 128, 256, 512}; x, codes and their strides 16-byte aligned;
 * scales 4-byte aligned with scale_stride_b a multiple of 4 and >= 4*n_rows when
 * batch > 1; outputs must not overlap x or each other.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL, DS4ATTN_E_UNSUPPORTED or DS4ATTN_E_HIP.
 */
int ds4attn_quantize_fp8(const void *x, int32_t dtype, int32_t batch, int32_t n_rows, int32_t head_dim,
                         int64_t x_stride_b, int64_t x_stride_row, uint8_t *codes,
                         int64_t code_stride_b, int64_t code_stride_row, float *scales,
                         int64_t scale_stride_b, void *stream);

/*
 * ds4attn_compress -- the compressor step of a compressed layer ([P-DS4]
 * "Architecture Deep Dive", Layer Compression and KV Cache Design: the compressor
 * keeps a rolling KV/score state and appends a pooled row at every ratio
 * boundary, every 4 raw rows in ratio-4 layers and every 128 in ratio-128 layers).
 * The pages name the state but not the pooling formula; this library's reading:
 * every raw row carries a score per element, and element d of a compressed row is
 * the softmax over the group's rows i of the scores s_i[d], weighting kv_i[d].
 *
 * The stream of a sequence is its n_state pending rows followed by its n_new new
 * rows.  Rows c*ratio .. c*ratio + ratio - 1 of the stream form group c, for the
 * n_out = (n_state + n_new) / ratio complete groups, and
 *     comp[c][d] = sum_i exp(s_i[d] - M) kv_i[d] / sum_i exp(s_i[d] - M),  M = max_i s_i[d],
 * computed in float32 and rounded once to float16.  The new state is the trailing
 * (n_state + n_new) mod ratio rows of the stream, written to state rows 0, 1, ...
 *
 *   state_kv     device float16 [batch][ratio][head_dim], packed rows (row r of
 *                sequence b at byte b*state_kv_stride_b + r*2*head_dim); rows
 *                [0, n_state) are read, and the new state is written in place
 *   state_score  device float32, the same layout with 4*head_dim bytes per row
 *   kv_new       device float16 [batch][n_new][head_dim], packed rows, batch stride in bytes
 *   score_new    device float32 [batch][n_new][head_dim], packed rows
 *   comp         device float16 output [batch][n_out][head_dim], packed rows (the
 *                caller points it at its next free compressed row); may be NULL
 *                when n_out is 0
 * The caller advances its own counts: n_state' = (n_state + n_new) mod ratio and
 * n_comp' = n_comp + n_out.  Scores must be finite.  head_dim in {64, 128, 256,
 * 512}; 1 <= ratio <= 1024 and 0 <= n_state < ratio (the same for every sequence);
 * pointers and batch strides 16-byte aligned; batch strides large enough for their
 * rows when batch > 1.  The state buffers must not overlap each other or the new
 * rows, and comp must not overlap any input.  Both kernels run on `stream`, the
 * pooling first (it reads the old state), then the state update.
 * Returns DS4ATTN_OK, DS4ATTN_E_INVAL, DS4ATTN_E_UNSUPPORTED or DS4ATTN_E_HIP; on an
 * error nothing is enqueued.
 */
int ds4attn_compress(int32_t batch, int32_t head_dim, int32_t ratio, int32_t n_state, int32_t n_new,
                     void *state_kv, int64_t state_kv_stride_b, float *state_score, int64_t state_score_stride_b,
                     const void *kv_new, int64_t kv_new_stride_b, const float *score_new,
                     int64_t score_new_stride_b, void *comp, int64_t comp_stride_b, void *stream);

/* A static, NUL-terminated description of a status code. */
const char *ds4attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DS4ATTN_H */
