/*
 * pmqa.h - C ABI of the MI355X (gfx950) FP8 paged MQA logits + per-row top-k library.
 *
 * The two operations are the sparse-attention indexer's decode scoring step and
 * the selection that follows it:
 *
 *   paged_mqa_logits : the op the pages call deepgemm_fp8_paged_mqa_logits
 *                      (aiter PR #4244 "fix silent tail-row drop in
 *                      deepgemm_fp8_paged_mqa_logits at large output stride":
 *                      bug description, root cause and fix; the reproducer
 *                      gives its tensors and their shapes).
 *   topk_per_row     : the follow-on top_k_per_row_decode that turns each logits
 *                      row into the sparse-KV index list (same page, first
 *                      paragraph).
 *
 * Score (the DSA indexer score; the pages name the op but print no formula, so
 * this is the reading adopted): for output row r = b*next_n + j and token t,
 *
 *     logit[r, t] = sum_h  w[r, h] * relu( scale_t * sum_d q[r, h, d] * k_t[d] )
 *
 * with q and k in OCP e4m3fn and the product accumulated in fp32 on the fp8
 * matrix cores.  Scales may take either sign: relu acts on scale * dot, so a
 * negative scale selects the heads whose dot is negative.  A NaN scale gives
 * its token a NaN score in every row that sees it (relu passes NaN on) and
 * changes nothing else.  Infinite scales, NaN codes and scores beyond the fp32
 * range are outside the contract, as is the top-k order of NaN scores.  Causal mask (reading adopted for MTP): the next_n rows of a
 * request are its last next_n positions, so row j sees
 * visible = clamp(ctx_b - next_n + j + 1, 0, ctx_b) tokens; columns
 * [visible, ctx_b) receive -inf and columns >= ctx_b are never written.
 *
 * Conventions shared by every entry point:
 *   - every pointer argument is DEVICE memory owned by the caller; the library
 *     allocates nothing and keeps no state between calls;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without synchronising; results are ordered only with
 *     later work on the same stream;
 *   - arguments checkable on the host are checked BEFORE anything is enqueued:
 *     on any error nothing is launched and a non-zero pmqa_status is returned.
 *     Nothing is silently dropped or truncated on the host side;
 *   - integer sizes are element counts unless the name says bytes.
 */
#ifndef PMQA_H_
#define PMQA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define PMQA_API __attribute__((visibility("default")))
#else
#define PMQA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PMQA_OK = 0,
  PMQA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PMQA_ERR_SHAPE = 2,       /* a size or stride is out of range                  */
  PMQA_ERR_UNSUPPORTED = 3, /* a valid but unimplemented shape or dtype           */
  PMQA_ERR_WORKSPACE = 4,   /* a workspace is missing or too small               */
  PMQA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch       */
  PMQA_ERR_ALIGNMENT = 6    /* a pointer lacks the alignment stated below        */
} pmqa_status;

/*
 * paged_mqa_logits - FP8 paged MQA logits over each request's paged K cache.
 *
 * q             [batch*next_n, num_heads, head_dim] e4m3fn bytes, row-major,
 *               16-byte aligned.  Row r = b*next_n + j (the pages' q is
 *               [B, next_n, H, D]).
 * kv_cache      the page pool, [num_pages, page_size, head_dim + 4] bytes,
 *               4-byte aligned.  Token s of page p is the record starting at
 *               byte (p*page_size + s)*(head_dim+4): head_dim e4m3fn codes then
 *               the token's fp32 scale, little endian (the pages' cache is
 *               [num_blocks, block_size, 1, D+4] fp8, the trailing four bytes
 *               of each token reinterpreted as its scale).  Byte offsets are formed in
 *               64-bit, so pools larger than 2^31 / 2^32 bytes are addressed
 *               correctly (ATOM PR #2533 "Address Triton decode KV rows with
 *               int64 ids").
 * weights       [batch*next_n, num_heads] fp32, 16-byte aligned.
 * context_lens  [batch] int32, ctx_b >= 0 (negative values count as 0).
 * block_tables  [batch, block_table_stride] int64 page ids.  Only the first
 *               ceil(ctx_b/page_size) ids of row b are used; entries past them
 *               may hold anything (the kernel may load them alongside the used
 *               ones, never past the row's block_table_stride entries, and never
 *               dereferences them).  Precondition not checked on the host (it
 *               lives in device memory): used ids lie in [0, num_pages).
 * page_size     tokens per page: a power of two from 1 to 256.  Pages smaller
 *               than the 16-token matrix tile are assembled into one tile (aiter
 *               PR #6626 section 1: a tile is built from several 8-token pages);
 *               page_size 1 reads token-level tables (a dense table of cache
 *               row ids, ATOM PR #2533).
 * next_n        MTP query positions per request, >= 1.
 * out           fp32 logits; row r starts at element r*out_row_stride (the row
 *               offset is computed in 64-bit: rows whose byte offset passes
 *               2^31 are written, aiter PR #4244 "Fix").  4-byte aligned.
 *               Columns [0, visible) get scores, [visible, ctx_eff) get -inf,
 *               nothing else is written (ctx_eff defined below).
 * out_row_stride  elements between output rows, >= 1.
 * batch         number of requests, >= 0 (0 enqueues nothing).
 * num_heads     16, 32, 64 or 128.
 * head_dim      128.
 * block_table_stride  entries between block-table rows, >= 1.
 * stream        hipStream_t to enqueue on.
 *
 * ctx_eff = min(ctx_b, block_table_stride*page_size, out_row_stride): the
 * kernel never reads past a table row nor writes past an output row, even
 * when the caller's context length exceeds them (a precondition violation).
 */
PMQA_API pmqa_status paged_mqa_logits(const void* q, const void* kv_cache, const float* weights,
                             const int32_t* context_lens, const int64_t* block_tables,
                             int32_t page_size, int32_t next_n, float* out,
                             int64_t out_row_stride, int32_t batch, int32_t num_heads,
                             int32_t head_dim, int64_t block_table_stride, void* stream);

/*
 * paged_mqa_logits_preshuffled - paged_mqa_logits over a pool in the
 * preshuffled page layout (the pages' kernels read K through a preshuffled
 * layout built by a library call with (min(page, 16), 16) tiles, aiter PR
 * #6626 section 1, whose permutation they do not print; this layout is this
 * library's own, with that tiling).  Same arguments, checks and results as
 * paged_mqa_logits (bit-identical logits for the same tokens), except:
 *
 * kv_cache      the page pool, num_pages pages of page_size * (head_dim + 4)
 *               bytes, 4-byte aligned.  Page p is cut into tiles of
 *               R = min(page_size, 16) tokens; tile t starts at byte
 *               p*page_size*132 + t*R*132.  Inside a tile, for each of the 8
 *               16-byte pieces c of a token's 128 codes (codes [16c, 16c+16)),
 *               the pieces of the R tokens follow in token order (piece c of
 *               the tile's token m at tile byte (c*R + m)*16); then the R
 *               tokens' fp32 scales, little endian (token m at tile byte
 *               128*R + 4*m).  quantize_k_cache_preshuffled writes this layout.
 * page_size     8, 16, 32, 64, 128 or 256 (PMQA_ERR_UNSUPPORTED for 1, 2, 4:
 *               their pages would split the 16-byte pieces).
 *
 * A 64-token step of a request then reads its pages' bytes contiguously and
 * a matrix-core operand (two 16-byte pieces of one token) from contiguous
 * LDS bytes across a wave.
 */
PMQA_API pmqa_status paged_mqa_logits_preshuffled(const void* q, const void* kv_cache,
                                                  const float* weights,
                                                  const int32_t* context_lens,
                                                  const int64_t* block_tables, int32_t page_size,
                                                  int32_t next_n, float* out,
                                                  int64_t out_row_stride, int32_t batch,
                                                  int32_t num_heads, int32_t head_dim,
                                                  int64_t block_table_stride, void* stream);

/*
 * topk_per_row - indices of the k largest logits of each row (the follow-on
 * top_k_per_row_decode of aiter PR #4244, first paragraph, which turns each
 * logits row into the sparse-KV index list the caller keeps).
 *
 * logits        fp32 [batch*next_n, logits_row_stride], row r at element
 *               r*logits_row_stride, 4-byte aligned.  Only [0, visible(r)) of
 *               each row is read, visible as for paged_mqa_logits (clamped to
 *               logits_row_stride).
 * context_lens  [batch] int32, as for paged_mqa_logits.
 * k             1 .. 2048.
 * out_idx       [batch*next_n, k] int32, row-major.  Row r receives the
 *               min(k, visible(r)) token indices of its largest scores, in
 *               unspecified order, and -1 in the remaining slots.  Every row
 *               is written, including rows with nothing visible.  Among equal
 *               scores at the k-th boundary the lowest indices are taken.
 * batch, next_n as for paged_mqa_logits.
 * logits_row_stride  elements between logits rows, >= 1.
 * workspace     DEVICE scratch owned by the caller, 16-byte aligned, or NULL
 *               when workspace_bytes is 0.  Its contents on entry are ignored
 *               and on return unspecified; calls that share it must be ordered
 *               on one stream.  When logits_row_stride exceeds 16384, a row
 *               of more than 8192 visible scores is split into segments of at
 *               most 8192 scores (of at most 16384 when the workspace or the
 *               merge's 16384 candidates allow no more segments), each
 *               selected by its own workgroup into k candidates held here, and
 *               a second launch merges them; the workspace bounds how far rows
 *               are split (the candidates of every row's segments must fit),
 *               never the result: a smaller one (0 included) only gives long
 *               rows fewer, longer segments.
 *               topk_per_row_workspace_size gives the size that splits rows of
 *               up to a given length fully; sized for the longest visible row
 *               (rather than for the stride) it is also what lets the split
 *               launch assume segments of at most 8192 scores and run two
 *               workgroups per CU.
 * workspace_bytes  bytes at workspace.  PMQA_ERR_WORKSPACE when it is nonzero
 *               and workspace is NULL.
 * stream        hipStream_t to enqueue on.
 */
PMQA_API pmqa_status topk_per_row(const float* logits, const int32_t* context_lens, int32_t k,
                                  int32_t* out_idx, int32_t batch, int32_t next_n,
                                  int64_t logits_row_stride, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * topk_per_row_noalloc - topk_per_row for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, checks and results as topk_per_row,
 * without the workspace: the candidates of split rows go to a scratch array
 * the library holds in device memory, PMQA_NOALLOC_SCRATCH_BYTES per GPU
 * (allocated with the library's code on each GPU it runs on, kept until the
 * process ends).  Rows are split exactly as topk_per_row splits them with a
 * workspace of topk_per_row_workspace_size(batch*next_n, k, logits_row_stride)
 * bytes; when that exceeds PMQA_NOALLOC_SCRATCH_BYTES the call returns
 * PMQA_ERR_WORKSPACE and enqueues nothing.  It calls no allocating routine.
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * on a GPU (different streams, different threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.  Nothing in
 * the scratch has to start at zero (each call writes what it reads).  The
 * first call on a device looks up that device's copy (hipGetSymbolAddress);
 * a failure there returns PMQA_ERR_HIP.
 */
#define PMQA_NOALLOC_SCRATCH_BYTES (64u << 20)
PMQA_API pmqa_status topk_per_row_noalloc(const float* logits, const int32_t* context_lens,
                                          int32_t k, int32_t* out_idx, int32_t batch,
                                          int32_t next_n, int64_t logits_row_stride,
                                          void* stream);

/*
 * topk_per_row_workspace_size - workspace bytes with which topk_per_row splits
 * every row of up to max_row_len visible scores as far as it splits rows
 * (segments of at most 8192 scores, at most 16384 / k of them): rows * k * 8
 * bytes per segment of the longest row; 0 when max_row_len <= 16384 (rows that
 * short are never split).
 * Host only.  Returns 0 for invalid arguments (rows < 0, k outside 1..2048,
 * max_row_len < 0).
 */
PMQA_API size_t topk_per_row_workspace_size(int32_t rows, int32_t k, int64_t max_row_len);

/*
 * paged_mqa_logits_timed, topk_per_row_timed - the same operations, for callers
 * that time each launch (benchmarks, serving telemetry).  start_event and
 * stop_event are caller-created hipEvent_t handles (either may be NULL); they
 * are recorded by the kernel dispatch itself when the kernel starts and when it
 * ends (AMD's extended launch), so hipEventElapsedTime between them is the
 * kernel's own duration, without the queue gaps that separate event records
 * around a launch would add.  Arguments, checks and results are otherwise
 * exactly those of the untimed calls.
 */
PMQA_API pmqa_status paged_mqa_logits_timed(const void* q, const void* kv_cache,
                                            const float* weights, const int32_t* context_lens,
                                            const int64_t* block_tables, int32_t page_size,
                                            int32_t next_n, float* out, int64_t out_row_stride,
                                            int32_t batch, int32_t num_heads, int32_t head_dim,
                                            int64_t block_table_stride, void* stream,
                                            void* start_event, void* stop_event);

PMQA_API pmqa_status paged_mqa_logits_preshuffled_timed(
    const void* q, const void* kv_cache, const float* weights, const int32_t* context_lens,
    const int64_t* block_tables, int32_t page_size, int32_t next_n, float* out,
    int64_t out_row_stride, int32_t batch, int32_t num_heads, int32_t head_dim,
    int64_t block_table_stride, void* stream, void* start_event, void* stop_event);

PMQA_API pmqa_status topk_per_row_timed(const float* logits, const int32_t* context_lens,
                                        int32_t k, int32_t* out_idx, int32_t batch,
                                        int32_t next_n, int64_t logits_row_stride,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        void* start_event, void* stop_event);

/*
 * pmqa_check_inputs - debug check of the preconditions that live in device
 * memory, which the calls above cannot check without a synchronisation (the
 * failure classes the pages report: stores silently dropped at large output
 * strides, aiter PR #4244; wrong pages read through wrapped ids, ATOM PR #2533).
 * For every request b it checks
 *     ctx_b <= block_table_stride*page_size  and  ctx_b <= out_row_stride
 * (negative lengths count as 0, as above), and that every page id the context
 * uses (entries i < ceil(ctx_b/page_size) of its table row, never past the row)
 * lies in [0, num_pages).  It reads only context_lens and those table entries
 * and never dereferences an id.
 *
 * context_lens, block_tables  as for paged_mqa_logits.
 * num_pages     pages in the pool, >= 1.
 * result        DEVICE int32[2], 4-byte aligned, written by the enqueued work:
 *               result[0] = number of requests that break a precondition,
 *               result[1] = the lowest such request index (batch when none).
 * The call enqueues on `stream` and returns; the caller synchronises and reads
 * `result`.  Host-checkable argument errors return a status (nothing enqueued).
 */
PMQA_API pmqa_status pmqa_check_inputs(const int32_t* context_lens, const int64_t* block_tables,
                                       int32_t batch, int32_t page_size,
                                       int64_t block_table_stride, int64_t out_row_stride,
                                       int64_t num_pages, int32_t* result, void* stream);

/* Element types of the K rows quantize_k_cache accepts. */
typedef enum {
  PMQA_DTYPE_F32 = 0,  /* IEEE binary32                              */
  PMQA_DTYPE_BF16 = 1  /* bfloat16: the high 16 bits of a binary32   */
} pmqa_dtype;

/*
 * quantize_k_cache - the producer of the records paged_mqa_logits reads:
 * quantises new K rows to e4m3fn and writes them, with their scales, into the
 * paged cache at caller-given slots.  The pages name this step through its
 * addressing only (ATOM PR #2533: the cache kernels compute slots in int64);
 * the quantisation is the per-token one of the cache's K (fp32 scale =
 * amax/448, e4m3fn codes), and the record layout is the one paged_mqa_logits
 * documents (aiter PR #4244 reproducer).
 *
 * For each token i in [0, num_tokens), with s = slot_mapping[i]:
 *     scale = max_d |k[i, d]| / 448  (fp32 division; 1 when the quotient is 0)
 *     code[d] = e4m3fn(clamp(k[i, d] / scale, -448, 448))  (fp32 division, then
 *               round to nearest, ties to the even code)
 * and the record of cache row s, at byte s*(head_dim+4) of kv_cache (formed in
 * 64-bit), receives the head_dim codes followed by scale (little-endian fp32).
 *
 * k             [num_tokens, head_dim] row-major, elements of type k_dtype,
 *               16-byte aligned.
 * k_dtype       PMQA_DTYPE_F32 or PMQA_DTYPE_BF16 (widened exactly to fp32).
 * slot_mapping  [num_tokens] int64 cache rows (page*page_size + offset in the
 *               page), 8-byte aligned.  Tokens whose slot lies outside
 *               [0, num_slots) are skipped (padding tokens carry -1).  Two
 *               tokens must not share a slot (which one lands is unspecified).
 * num_tokens    >= 0 (0 enqueues nothing).
 * head_dim      128.
 * kv_cache      the page pool, num_slots records of head_dim+4 bytes,
 *               4-byte aligned; only the records of the tokens' slots are
 *               written.
 * num_slots     records in the pool (num_pages * page_size), >= 0.
 * stream        hipStream_t to enqueue on.
 * Scores of non-finite k rows are outside the contract (the record is written
 * but its contents are unspecified).
 */
PMQA_API pmqa_status quantize_k_cache(const void* k, int32_t k_dtype,
                                      const int64_t* slot_mapping, int32_t num_tokens,
                                      int32_t head_dim, void* kv_cache, int64_t num_slots,
                                      void* stream);

/*
 * quantize_k_cache_preshuffled - quantize_k_cache writing the preshuffled page
 * layout that paged_mqa_logits_preshuffled reads: token i's codes and scale
 * go to the tile positions of cache row slot_mapping[i] (page = slot /
 * page_size) instead of one 132-byte record.  page_size as for
 * paged_mqa_logits_preshuffled; num_slots must be a whole number of pages
 * (PMQA_ERR_SHAPE otherwise).  Other arguments, checks and the quantisation
 * are those of quantize_k_cache.
 */
PMQA_API pmqa_status quantize_k_cache_preshuffled(const void* k, int32_t k_dtype,
                                                  const int64_t* slot_mapping, int32_t num_tokens,
                                                  int32_t head_dim, void* kv_cache,
                                                  int64_t num_slots, int32_t page_size,
                                                  void* stream);

/* quantize_k_cache with dispatch-recorded start/stop events, as the other _timed calls. */
PMQA_API pmqa_status quantize_k_cache_timed(const void* k, int32_t k_dtype,
                                            const int64_t* slot_mapping, int32_t num_tokens,
                                            int32_t head_dim, void* kv_cache, int64_t num_slots,
                                            void* stream, void* start_event, void* stop_event);

/* Human-readable name of a status code (static storage; never NULL). */
PMQA_API const char* pmqa_status_string(pmqa_status status);

/* Library version, as major*10000 + minor*100 + patch. */
PMQA_API int32_t pmqa_version(void);

/* Name of the logits kernel paged_mqa_logits launches for these sizes (host
 * only: no GPU, no device memory), written NUL-terminated into name[0..name_len):
 * "logits_flat_kernel<H,R>" (one single-wave workgroup per 64-token iteration,
 * taken when every next_n row of a request fits one wave of 64 q rows and the
 * iterations the contexts could hold are at most 8192),
 * "logits_shared_kernel<H,G,D>" (128 heads with 2 or 4 next_n rows: one request
 * run per workgroup of G waves, one row each, around one ring of D K slots) or
 * "logits_kernel<H,R,W,D>" (the persistent grid: R next_n rows per wave, W waves
 * per workgroup, D iterations in flight per wave).  The sizes are those of
 * paged_mqa_logits and are checked the same way.  Returns PMQA_ERR_NULL for a
 * NULL name or name_len < 1, and PMQA_ERR_SHAPE when the name does not fit. */
PMQA_API pmqa_status pmqa_logits_kernel(int32_t batch, int32_t next_n, int32_t page_size,
                                        int64_t out_row_stride, int32_t num_heads,
                                        int32_t head_dim, int64_t block_table_stride,
                                        char* name, int32_t name_len);

#ifdef __cplusplus
}
#endif

#endif /* PMQA_H_ */
