/*
 * vts.h -- exact batched variable-length top-K selection (C ABI).
 *
 * Two operations, both asynchronous on the caller's HIP stream, both exact
 * with ties interchangeable:
 *
 *   vts_topk_varlen                 decode-step top-k with per-request lengths
 *   vts_topk_varlen_ordered         the same in canonical order with a tie-break
 *   vts_topk_page_table_transform   top-k over row windows, fused with a
 *                                   page-table translation of the indices
 *
 * The unprefixed names topk_varlen and topk_page_table_transform are exported
 * as aliases of the two entry points.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device memory (or memory the device can
 *     read/write directly); the caller owns all of it.  The library allocates
 *     nothing during a call and reads no device memory from the host, so a call
 *     may be captured into a HIP graph.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  The
 *     call only enqueues work; results are ready when the stream reaches it.
 *   - Integers in device arrays (lengths, starts, hints) may hold any value: the
 *     kernels clamp them as described and never read out of bounds because of
 *     them.
 *   - Return value: a vts_status.  Argument errors are detected on the host
 *     before any HIP call, so nothing is enqueued when a call fails.
 */
#ifndef VTS_H
#define VTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the score rows. */
typedef enum { VTS_F32 = 0, VTS_BF16 = 1, VTS_F16 = 2 } vts_dtype;

typedef enum {
    VTS_OK = 0,
    /* pre_idx was not usable (misaligned); it was ignored and the call ran
     * without a hint.  Results are unaffected.  (FlashInfer top_k_varlen doc,
     * `pre_idx`: a malformed hint is discarded with a warning.) */
    VTS_WARN_HINT_DISCARDED = 1,
    /* a shape, pointer, alignment or grouping argument breaks the contract
     * (FlashInfer top_k_varlen doc, "raises ValueError"). */
    VTS_ERR_INVALID = -1,
    /* the request is valid but outside what this library implements:
     * top_k above 16384 (above 2048 in the deterministic mode), a row of
     * width columns taking 2^31 bytes or more, or a device other than
     * gfx950. */
    VTS_ERR_UNSUPPORTED = -2,
    /* workspace pointer null or smaller than the matching *_workspace_bytes(). */
    VTS_ERR_WORKSPACE = -3,
    /* a HIP runtime call failed (no device, launch failure). */
    VTS_ERR_HIP = -4,
    /* vts_topk_varlen_noalloc: the shape needs more scratch than its fixed
     * device array holds. */
    VTS_ERR_TOO_LARGE = -5
} vts_status;

/* Workspace: device scratch used by rows that several workgroups share and by
 * candidate overflow.  Query its size with the matching *_workspace_bytes()
 * (a pure host function of the shape and element type), allocate it, fill it with zeros ONCE
 * (vts_workspace_init or any memset), then pass it to every call of that
 * shape.  Each call leaves it as it found it apart from the event counters of
 * vts_workspace_stats, so it never needs clearing again.  One workspace must
 * not be used by two calls that can run at the same time (for example on two
 * streams): give each stream its own.  (FlashInfer top_k_varlen doc,
 * `workspace`: a zero-initialised, self-restoring slab, one per stream.) */
size_t vts_topk_varlen_workspace_bytes(int64_t num_rows, int64_t width, int32_t top_k,
                                       int32_t dtype);
size_t vts_page_transform_workspace_bytes(int64_t num_rows, int64_t width, int32_t top_k,
                                          int32_t dtype);

/* Fills `bytes` bytes of `workspace` with zeros on `stream`. */
int vts_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * vts_topk_varlen -- FlashInfer "flashinfer.top_k_varlen" documentation
 * (signature, `seq_lens`, `compress_ratio`, `next_n`, `pre_idx`,
 * `return_values`, `out_indices`, `out_values`).
 *
 * logits      device, dtype elements, num_rows rows of `width` columns with
 *             consecutive rows `row_stride` elements apart (row_stride >=
 *             width); the base must be aligned to the element size.
 * seq_lens    device int32[num_rows / next_n]: KV-cache length of each request
 *             in KV-token units.  Row r belongs to request i = r / next_n as its
 *             t = r % next_n-th row and ranks its first
 *               n = max(0, (seq_lens[i] - next_n + t + 1) / compress_ratio)
 *             columns (integer division), clamped to `width`.
 * top_k       1 <= top_k <= 16384 (the range of FlashInfer's radix_filter
 *             backend, same page, `backend`).  Above 2048 the candidate
 *             lists live in LDS and the workspace (a larger workspace, see
 *             vts_topk_varlen_workspace_bytes) instead of registers.
 * next_n      >= 1, must divide num_rows.
 * compress_ratio >= 1.
 * pre_idx     device int32[num_rows / next_n, top_k] or NULL: the previous
 *             step's selection for each request, a sampling anchor only
 *             (FlashInfer top_k_varlen doc, `pre_idx`).  It is validated
 *             (16-byte aligned, else ignored with VTS_WARN_HINT_DISCARDED).
 *             The default path does not read it: its threshold comes from a
 *             strided sample of the row, which measured faster than also
 *             bounding it by the hint (the VTS_TUNE_HINT_RUNG switch turns
 *             that on; it reads the row at every hinted column and the next
 *             one).  Results never depend on it.
 * out_indices device int32[num_rows, top_k], 16-byte aligned.  Row r receives
 *             the column indices of its top-k (in no particular order) when
 *             n > top_k; the indices 0..n-1 followed by -1 when n <= top_k (all
 *             -1 when n == 0).
 * out_values  device dtype[num_rows, top_k], 16-byte aligned, or NULL (values
 *             not returned).  Bit copies of the selected elements, aligned
 *             with out_indices; slots holding -1 get the lowest finite value
 *             of the dtype (-FLT_MAX for fp32, 0xFF7F bf16, 0xFBFF fp16).
 * workspace   device, >= vts_topk_varlen_workspace_bytes(num_rows, width,
 *             top_k, dtype) bytes, 16-byte aligned, zeroed once (see above).
 *
 * Ties: all elements that compare equal are interchangeable; -0 and +0 are
 * ties.  +inf, -inf and subnormals rank exactly.  NaN is ordered above +inf
 * (sign clear) or below -inf (sign set).
 */
int vts_topk_varlen(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                    int64_t row_stride, const int32_t* seq_lens, int32_t top_k, int32_t next_n,
                    int32_t compress_ratio, const int32_t* pre_idx, int32_t* out_indices,
                    void* out_values, void* workspace, size_t workspace_bytes, void* stream);

/*
 * vts_topk_varlen_noalloc -- vts_topk_varlen for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): the same arguments, results and errors,
 * without the workspace.  Its scratch is a fixed 32 MiB device array of the
 * library (one per device, held from the library's first use of that device
 * until the process ends); the call allocates nothing and frees nothing.
 *
 * Limit: the shape's workspace must fit the array with at least 3776
 * candidate slots per workgroup; otherwise VTS_ERR_TOO_LARGE and nothing is
 * enqueued.  That admits up to about 1100 row units (rows times workgroups
 * per row; e.g. 1024 rows of 262144 columns, or 64 rows split in four),
 * with fewer spill slots per unit than the workspace entry point when it is
 * near the limit (a spill beyond them takes the slower, still exact,
 * re-filtering path).
 *
 * Each call first clears the array's counters and row tickets on `stream`
 * (a small kernel), then runs the selection.  Every call on one device shares
 * that device's array: calls that can overlap on one device (two streams, two
 * threads) race and must be serialised by the caller.
 */
int vts_topk_varlen_noalloc(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                            int64_t row_stride, const int32_t* seq_lens, int32_t top_k,
                            int32_t next_n, int32_t compress_ratio, const int32_t* pre_idx,
                            int32_t* out_indices, void* out_values, void* stream);

/* Tie-breaks of the deterministic mode (the *_ordered entry points). */
enum vts_tie_break {
    VTS_TIE_SMALL = 1,   /* of the values equal to the k-th, the smallest columns */
    VTS_TIE_LARGE = 2,   /* of the values equal to the k-th, the largest columns */
    /* added to SMALL or LARGE: the same selected set, written in no particular
     * order (no canonical sort); a row with n <= top_k is then the identity
     * 0..n-1 followed by -1, as in the unordered entry points */
    VTS_TIE_UNSORTED = 4
};

/*
 * vts_topk_varlen_ordered -- vts_topk_varlen in deterministic mode (the
 * FlashInfer page-size PR body on the SGLang PR #33237 page, "Description" and
 * "Performance": a deterministic post-sort of each row's outputs and a SMALL /
 * LARGE choice among tied values).  The order itself is not spelled out there;
 * value descending, then column ascending, is the reading taken here.
 *
 * Arguments, windows, errors and workspace are those of vts_topk_varlen,
 * except that top_k is at most 2048 (VTS_ERR_UNSUPPORTED above);
 * tie_break is VTS_TIE_SMALL or VTS_TIE_LARGE, optionally plus
 * VTS_TIE_UNSORTED (anything else: VTS_ERR_INVALID).  The selected set is
 * unique: every value above the k-th largest, then, of the values equal to
 * it, those at the smallest (SMALL) or largest (LARGE) columns.  Values
 * compare as numbers: -0 and +0 are equal (TensorRT-LLM PR #17821, "Test
 * coverage": signed zeros normalised), every NaN with the sign clear is
 * above +inf and equal to every other such NaN, every NaN with the sign set
 * below -inf and equal to every other such NaN.  Each row's outputs are in
 * canonical order: value descending, then column ascending; a row with
 * n <= top_k lists all n columns in that order, then -1.  The output is a
 * function of the inputs alone (bit-identical from run to run); out_values
 * are bit copies of the selected elements, as for vts_topk_varlen.  The sort
 * adds an epilogue per row (about 66 LDS compare-exchange rounds at top_k
 * 2048); VTS_TIE_UNSORTED skips it.
 */
int vts_topk_varlen_ordered(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                            int64_t row_stride, const int32_t* seq_lens, int32_t top_k,
                            int32_t next_n, int32_t compress_ratio, const int32_t* pre_idx,
                            int32_t* out_indices, void* out_values, void* workspace,
                            size_t workspace_bytes, void* stream, int32_t tie_break);

/*
 * vts_topk_page_table_transform -- top-k over row windows with the compact
 * page-table transform (FlashInfer page-size PR body quoted on the SGLang
 * PR #33237 page, "Description"; `lengths` / `row_starts` as in SGLang's
 * fast_topk_v2, TopK_Ops page, I/O contract).
 *
 * scores       device, dtype, num_rows rows, `width` columns, `row_stride`
 *              elements apart (row_stride >= width).
 * lengths      device int32[num_rows]: valid length of each row's window.
 * row_starts   device int32[num_rows] or NULL (all 0): first column of each
 *              row's window, in score elements.  The window is
 *              [row_start, row_start + n) with n = clamp(length, 0,
 *              width - row_start); a start outside [0, width] gives n = 0.
 * src_page_table device int32, num_rows rows of page_table_width entries,
 *              page_table_stride entries apart.
 * page_table_row_starts device int32[num_rows] or NULL: first page-table entry
 *              of each row, in page-table entries.  NULL means the row start
 *              (row_starts, or 0); when page_size > 1 and row_starts is given
 *              it is required.
 * page_size    1 <= page_size <= 2^30.
 * top_k        1 <= top_k <= 16384.
 * out          device int32[num_rows, top_k], 16-byte aligned: for each
 *              selected window-relative index idx,
 *                src_page_table[r, pt_start + idx / page_size] * page_size
 *                  + idx % page_size,
 *              and -1 in unused slots.  A page-table entry outside
 *              [0, page_table_width) also yields -1.
 * out_raw_indices device int32[num_rows, top_k] or NULL: the window-relative
 *              indices themselves, positionally aligned with `out`, -1 in
 *              unused slots.  Must not overlap `out`.
 * workspace    as for vts_topk_varlen, sized by vts_page_transform_workspace_bytes.
 */
int vts_topk_page_table_transform(const void* scores, int32_t dtype, int64_t num_rows,
                                  int64_t width, int64_t row_stride, const int32_t* lengths,
                                  const int32_t* row_starts, const int32_t* src_page_table,
                                  int64_t page_table_stride, int64_t page_table_width,
                                  const int32_t* page_table_row_starts, int32_t page_size,
                                  int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * vts_topk_page_table_transform_ordered -- vts_topk_page_table_transform in
 * the deterministic mode of vts_topk_varlen_ordered (same page, "Description":
 * `out_raw_indices` stays positionally aligned with `out` through the
 * deterministic post-sort).  The selection over each window, its order and
 * tie_break are those of vts_topk_varlen_ordered, on window-relative indices;
 * `out` holds their translations slot by slot.
 */
int vts_topk_page_table_transform_ordered(
    const void* scores, int32_t dtype, int64_t num_rows, int64_t width, int64_t row_stride,
    const int32_t* lengths, const int32_t* row_starts, const int32_t* src_page_table,
    int64_t page_table_stride, int64_t page_table_width, const int32_t* page_table_row_starts,
    int32_t page_size, int32_t top_k, int32_t* out, int32_t* out_raw_indices, void* workspace,
    size_t workspace_bytes, void* stream, int32_t tie_break);

/*
 * vts_topk_transform_ragged -- top-k over row windows with the ragged-KV index
 * transform (SGLang TopK_Ops page, fast_topk_transform_ragged_fused: the
 * offset of each row's top-k indices in a ragged KV buffer).
 *
 * scores, lengths, row_starts, top_k, workspace: as for
 *              vts_topk_page_table_transform (workspace sized by
 *              vts_page_transform_workspace_bytes).
 * topk_indices_offset device int32[num_rows]: added to every selected
 *              window-relative index of the row (int32 arithmetic; keeping
 *              the sums in range is the caller's contract).
 * out          device int32[num_rows, top_k], 16-byte aligned: idx +
 *              topk_indices_offset[r] for each selected window-relative
 *              index idx, -1 in unused slots.
 * out_raw_indices device int32[num_rows, top_k] or NULL: the window-relative
 *              indices, positionally aligned with `out`, -1 in unused slots.
 *              Must not overlap `out`.
 */
int vts_topk_transform_ragged(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                              int64_t row_stride, const int32_t* lengths,
                              const int32_t* row_starts, const int32_t* topk_indices_offset,
                              int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                              void* workspace, size_t workspace_bytes, void* stream);

/* vts_topk_transform_ragged in the deterministic mode (see
 * vts_topk_page_table_transform_ordered). */
int vts_topk_transform_ragged_ordered(const void* scores, int32_t dtype, int64_t num_rows,
                                      int64_t width, int64_t row_stride, const int32_t* lengths,
                                      const int32_t* row_starts,
                                      const int32_t* topk_indices_offset, int32_t top_k,
                                      int32_t* out, int32_t* out_raw_indices, void* workspace,
                                      size_t workspace_bytes, void* stream, int32_t tie_break);

/*
 * vts_topk_transform_page1 -- top-k over row windows with the page-size-1
 * transform of SGLang's fast_topk_transform_fused (TopK_Ops page): each row
 * is a query of one request, found through `cu_seqlens_q`, and each selected
 * window-relative index (a KV position of that request) is replaced by the
 * request's page-table entry for it.
 *
 * scores, lengths, row_starts, top_k: as for vts_topk_page_table_transform.
 * page_table   device int32, num_batches rows of page_table_width entries,
 *              page_table_stride entries apart: row b maps KV positions of
 *              request b to physical KV slots.
 * cu_seqlens_q device int32[num_batches + 1], non-decreasing: rows
 *              [cu_seqlens_q[b], cu_seqlens_q[b + 1]) belong to request b.
 * out          device int32[num_rows, top_k], 16-byte aligned:
 *              page_table[b(r), idx] for each selected index idx, -1 in
 *              unused slots, where idx >= page_table_width, and in every slot
 *              of a row outside [cu_seqlens_q[0], cu_seqlens_q[num_batches]).
 * out_raw_indices device int32[num_rows, top_k] or NULL: the window-relative
 *              indices, positionally aligned with `out`; must not overlap it.
 * workspace    as for vts_topk_varlen, sized by vts_page_transform_workspace_bytes;
 *              the call also writes a row-to-request map into it (a small
 *              kernel on `stream` before the selection).
 */
int vts_topk_transform_page1(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                             int64_t row_stride, const int32_t* lengths, const int32_t* row_starts,
                             const int32_t* page_table, int64_t page_table_stride,
                             int64_t page_table_width, const int32_t* cu_seqlens_q,
                             int64_t num_batches, int32_t top_k, int32_t* out,
                             int32_t* out_raw_indices, void* workspace, size_t workspace_bytes,
                             void* stream);

/* vts_topk_transform_page1 in the deterministic mode (see
 * vts_topk_page_table_transform_ordered). */
int vts_topk_transform_page1_ordered(const void* scores, int32_t dtype, int64_t num_rows,
                                     int64_t width, int64_t row_stride, const int32_t* lengths,
                                     const int32_t* row_starts, const int32_t* page_table,
                                     int64_t page_table_stride, int64_t page_table_width,
                                     const int32_t* cu_seqlens_q, int64_t num_batches,
                                     int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     int32_t tie_break);

/* Aliases with the operation names of the pages. */
int topk_varlen(const void* logits, int32_t dtype, int64_t num_rows, int64_t width,
                int64_t row_stride, const int32_t* seq_lens, int32_t top_k, int32_t next_n,
                int32_t compress_ratio, const int32_t* pre_idx, int32_t* out_indices,
                void* out_values, void* workspace, size_t workspace_bytes, void* stream);
int topk_page_table_transform(const void* scores, int32_t dtype, int64_t num_rows, int64_t width,
                              int64_t row_stride, const int32_t* lengths,
                              const int32_t* row_starts, const int32_t* src_page_table,
                              int64_t page_table_stride, int64_t page_table_width,
                              const int32_t* page_table_row_starts, int32_t page_size,
                              int32_t top_k, int32_t* out, int32_t* out_raw_indices,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text of a vts_status. */
const char* vts_status_string(int status);

/* Event counters kept in a workspace, copied to `out` (host, `count` <= 4
 * entries)
 * with a synchronous copy on `stream`, then cleared:
 *   out[0]  workgroups whose candidates overflowed and were re-filtered
 *   out[1]  rows whose sampled threshold kept fewer than top_k candidates
 *           and that were re-selected over the whole row
 *   out[2]  rows whose candidates outgrew on-chip memory (selected over the
 *           spilled workspace slots too)
 *   out[3]  rows with fewer than top_k keys at or above the likely threshold,
 *           so that the whole candidate list (keys at or above the safe
 *           threshold) was ranked */
int vts_workspace_stats(void* workspace, uint32_t* out, int32_t count, void* stream);

/* Plan log: with VTS_LOG=1 in the environment (read once per process), every
 * call prints one line to stderr naming the entry point, the shape, the
 * kernels (any-order, ordered, wide or hinted), the units per row, the row
 * placement and the device's compute units.  Results never depend on it. */

/* Diagnostic and test switches.  Each applies to the calls (and workspace-size
 * queries) of the thread that set it, nowhere else.  None of them changes
 * results, only which internal path computes them.
 *   VTS_TUNE_NSPLIT       workgroups per long row (0 = automatic, 1..32)
 *   VTS_TUNE_FORCE_PATH   0 normal, 1 every chunk uses the compaction filter,
 *                         2 every row is re-selected over the whole row
 *   VTS_TUNE_LDS_SLOTS    on-chip candidate slots before spilling to the
 *                         workspace (0 = default; 64..3776)
 *   VTS_TUNE_SPILL_SLOTS  candidate slots per workgroup, on chip and in the
 *                         workspace, before a chunk is re-filtered
 *                         (0 = default; 64..8192)
 *   VTS_TUNE_SAMPLE_SIGMA margin of the safe threshold rung in tenths of a
 *                         standard deviation of the sample count (0 = 50)
 *   VTS_TUNE_LIKELY_SIGMA margin of the likely rung, same unit (0 = 20; a
 *                         value >= the safe margin merges the two rungs)
 *   VTS_TUNE_MIN_CHUNK    valid columns per workgroup below which a row is not
 *                         split further (0 = default: 32768, and 128 KB of
 *                         columns for the length-balanced units of 512-row
 *                         batches; 256..2^20)
 *   VTS_TUNE_NO_BALANCE   1 turns off the length-balanced placement of rows on
 *                         compute units (0 = on where it applies)
 *   VTS_TUNE_HINT_RUNG    1: vts_topk_varlen calls with a pre_idx and top_k
 *                         <= 2048 also bound the safe threshold from below by the
 *                         k-th largest value read at the hinted columns
 *                         (0 = hint not read)
 * The workspace size follows the split count in force when it is queried.
 * Returns VTS_OK or VTS_ERR_INVALID for an unknown key or value. */
enum {
    VTS_TUNE_NSPLIT = 1,
    VTS_TUNE_FORCE_PATH = 2,
    VTS_TUNE_LDS_SLOTS = 3,
    VTS_TUNE_SPILL_SLOTS = 4,
    VTS_TUNE_SAMPLE_SIGMA = 5,
    VTS_TUNE_MIN_CHUNK = 6,
    VTS_TUNE_LIKELY_SIGMA = 7,
    VTS_TUNE_NO_BALANCE = 8,
    VTS_TUNE_HINT_RUNG = 9
};
int vts_set_tuning(int32_t key, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* VTS_H */
