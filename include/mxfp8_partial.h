/*
 * mxfp8_partial.h -- C ABI of libmxfp8partial.so: MXFP8 partial amax, amax MAX-combine,
 * E8M0 scale update and partial E4M3 cast for a contiguous fragment of a flattened 2-D
 * master weight, on AMD Instinct MI355X (gfx950).
 *
 * The operation is the distributed master-weight writeback of "Support row-only MXFP8
 * distributed master-weight casts" (TransformerEngine PR 3488): each rank holds a contiguous
 * fragment [start, start + len) of the row-major flattening of a rows x cols weight
 * (section Changes; the kernel documentation in the review threads describes the input as a
 * contiguous piece of the flattened tensor), computes per-block amax for the directions that
 * exist, the amax of all fragments is MAX-combined in a single packed reduction, scales are
 * updated for the present directions, and the fragment is cast in place to E4M3 row-wise
 * data and, only when that output is present, column-wise data (flow diagram of the Greptile
 * summary).  The block shape (1x32 row-wise, 32x1 column-wise) and
 * the numeric rules below follow the OCP Microscaling (MX) v1.0 and OFP8 specifications.
 *
 * Conventions shared by every entry point
 *  - All buffer pointers are DEVICE pointers unless stated otherwise.  The caller owns every
 *    buffer; the library allocates nothing, keeps no pointer after a call returns, and never
 *    synchronizes: work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream).
 *  - An absent direction or output is an empty handle: ptr == NULL.  There is no shape
 *    sentinel (the pages drop the empty-shape convention in favour of empty handles).
 *  - Element (r, c) of the weight is flat index i = r * cols + c.  Fragment element k is
 *    input[k] = x[start + k].  Row-wise block (r, j) covers columns [32 j, min(32 j + 32, cols))
 *    of row r; column-wise block (b, c) covers rows [32 b, min(32 b + 32, rows)) of column c.
 *  - amax arrays hold the input dtype (FP32 or BF16 bit patterns; the review threads show a
 *    check that the amax dtype equals the input dtype): amax_row is [rows][ld >= ceil(cols/32)], amax_col is
 *    [ceil(rows/32)][ld >= cols].  Scale arrays are uint8 E8M0 with the same shapes.
 *    Entries beyond the logical width (padding) are never read or written.
 *  - data_row / data_col are uint8 E4M3 and FRAGMENT-RELATIVE: byte k belongs to element
 *    start + k, in the weight's row-major order for both directions (column-wise data is not
 *    transposed).  In-place writes into a full-size MXFP8 tensor pass base + start; a
 *    fragment-sized output buffer passes its own pointer.
 *  - Errors: every check runs on the host before anything is enqueued; a call returns a
 *    status code and never aborts or throws.  mxfp8_last_error() gives a message for the
 *    calling thread's last non-OK status.  A HIP launch failure returns MXFP8_ERR_HIP: the
 *    launches issued before the failing one stay enqueued, and no launch follows it.
 *  - Across the pieces of one call, a buffer that one piece writes must not overlap any
 *    buffer of another piece (MXFP8_ERR_LAYOUT), except that pieces may share an amax or
 *    scale array: the same pointer, leading dimension and shape in the same role, which is
 *    how the pieces of one weight merge the blocks their fragments cut.
 *  - len == 0 (an empty master shard on a participating rank) is a valid no-op; input and
 *    outputs may then be NULL.
 *  - Precondition, not checked (device data): inputs are finite, and pre-rounding (below)
 *    does not overflow BF16; amax entries are non-negative; scale bytes are at most 254.
 */
#ifndef MXFP8_PARTIAL_H
#define MXFP8_PARTIAL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP8_OK = 0,
  MXFP8_ERR_ARG = 1,     /* n < 0, pieces == NULL with n > 0, rows/cols < 1, k < 1, NULL input */
  MXFP8_ERR_RANGE = 2,   /* [start, start + len) not inside [0, rows * cols]                     */
  MXFP8_ERR_DTYPE = 3,   /* unknown dtype, or pre-rounding requested for a BF16 input            */
  MXFP8_ERR_LAYOUT = 4,  /* leading dimension below the logical width, misaligned element
                            pointer, or an input overlapping an output                            */
  MXFP8_ERR_MISSING = 5, /* a required buffer is absent (row-wise outputs are always required;
                            column-wise scales are required when column-wise work is requested) */
  MXFP8_ERR_HIP = 6      /* a kernel launch failed                                                */
} mxfp8_status;

typedef enum { MXFP8_FP32 = 0, MXFP8_BF16 = 1 } mxfp8_dtype;

/* A device buffer and its leading dimension in elements; ptr == NULL means absent. */
typedef struct {
  void* ptr;
  int64_t ld;
} mxfp8_buf;

/* One fragment of one weight.  Which fields an entry point reads is stated at that entry
 * point; the others are ignored. */
typedef struct {
  int64_t rows, cols;       /* logical shape of the whole 2-D weight                          */
  int64_t start, len;       /* fragment [start, start + len) of its row-major flattening      */
  int32_t in_dtype;         /* MXFP8_FP32 or MXFP8_BF16                                       */
  int32_t preround_bf16;    /* 1: round FP32 master values to BF16 (nearest, ties to even)
                               before amax and cast (the rounding through the model dtype
                               of section Changes); FP32 input only                           */
  const void* input;        /* len elements of in_dtype, aligned to the element size          */
  mxfp8_buf amax_row;       /* in_dtype entries, [rows][ld]                                   */
  mxfp8_buf amax_col;       /* in_dtype entries, [ceil(rows/32)][ld]; NULL = row-only         */
  mxfp8_buf scale_row;      /* uint8 E8M0, [rows][ld]                                         */
  mxfp8_buf scale_col;      /* uint8 E8M0, [ceil(rows/32)][ld]                                */
  void* data_row;           /* uint8 E4M3, len bytes, fragment-relative                       */
  void* data_col;           /* uint8 E4M3, len bytes, fragment-relative; NULL = row-only      */
} mxfp8_piece;

/* Step 1 -- partial amax (first step of the flow diagram; the kernel documentation in the
 * review threads marks both amax outputs as in/out).
 * For each of the n pieces (a host array) and every block the fragment touches in a present
 * direction, with m = max |w| over the fragment's elements in the block, w being the input
 * value (pre-rounded to BF16 if requested):
 *  - a block the fragment holds whole: amax[block] = m (no other fragment touches it; the
 *    old entry is not read);
 *  - a block a fragment boundary cuts: amax[block] = max(amax[block], m);
 *  - blocks the fragment does not touch keep their entry.
 * So pieces of one weight whose fragments do not overlap may share amax buffers within a
 * call or across calls, and a zero-filled buffer accumulates the amax of all pieces (on it
 * the result is max(entry, m) for every touched block).  Calls that share an amax buffer must
 * be ordered (one stream, or streams synchronized with each other): a piece that no other
 * piece of its call shares amax buffers with may merge by a read and a write rather than an
 * atomic.  The column-wise direction is
 * computed iff amax_col.ptr != NULL.  Reads: rows, cols, start, len, in_dtype,
 * preround_bf16, input, amax_row (required), amax_col. */
int mxfp8_partial_amax(const mxfp8_piece* pieces, int n, void* hip_stream);

/* Step 2 -- MAX-combine (section Changes keeps a single MAX all-reduce over the packed amax;
 * on one GPU the partials of several fragments are combined on the device instead).
 * dst[e] = max over j < k of srcs[j][e], for e < count entries of amax_dtype.  srcs is a HOST
 * array of k device pointers; dst may equal srcs[0] (in place) but must not partly overlap
 * any source.  Pack the amax of every present direction of a batch into one buffer and call
 * this once per batch. */
int mxfp8_combine_amax(void* dst, const void* const* srcs, int k, int64_t count,
                       int32_t amax_dtype, void* hip_stream);

/* Step 3 -- E8M0 scales for the present directions (flow diagram; section Changes skips the
 * update of absent column-wise scales).  For every block the piece's
 * fragment touches: scale = clamp(floor(log2 amax) - 8 + 127, 0, 254), and 0 for amax == 0
 * (OCP MX, emax of E4M3 = 8).  Other scale bytes are left as they are.  The column-wise
 * direction is computed iff amax_col.ptr != NULL, and then scale_col is required.  Reads:
 * rows, cols, start, len, in_dtype (the amax dtype), amax_row, amax_col, scale_row
 * (required), scale_col.  Pieces whose fragments share a cut block write the same byte. */
int mxfp8_compute_scales(const mxfp8_piece* pieces, int n, void* hip_stream);

/* Step 4 -- partial cast, in place (last steps of the flow diagram: row-wise output always;
 * column-wise output only when present, in which case its scales are required, otherwise its
 * reads and writes are skipped).
 * data_row[k] = E4M3(w * 2^(127 - s)) with s the row-wise block's scale byte, rounded to
 * nearest even and saturated to +-448 (the sign of zero is kept); data_col[k] likewise with
 * the column-wise block's scale, only when data_col != NULL, which then requires scale_col.
 * When data_col is NULL, scale_col is ignored even if set.  Row-wise outputs (data_row,
 * scale_row) are always required.  Reads: rows, cols, start, len, in_dtype, preround_bf16,
 * input, scale_row, scale_col, data_row, data_col. */
int mxfp8_partial_cast(const mxfp8_piece* pieces, int n, void* hip_stream);

/* Steps 3 and 4 in one pass (the scale update and the output writes of the flow diagram,
 * fused by this library; the pages run them as separate steps).
 * Same results as mxfp8_compute_scales followed by mxfp8_partial_cast on the same pieces:
 * the scale of each block the fragment touches is derived from its amax entry, written to
 * scale_row / scale_col, and used directly for that block's E4M3 bytes; the scale arrays
 * are written, never read.  The column-wise work (amax_col read, scale_col and data_col
 * written) happens iff data_col != NULL, which then requires amax_col and scale_col; when
 * data_col is NULL both are ignored even if set.  Required: input, amax_row, scale_row,
 * data_row.  Scale and data outputs must not overlap the input, the amax arrays or each
 * other.  Reads: rows, cols, start, len, in_dtype (also the amax dtype), preround_bf16,
 * input, amax_row, amax_col, scale_row, scale_col, data_row, data_col.  Pieces whose
 * fragments share a cut block write the same scale byte. */
int mxfp8_scales_and_cast(const mxfp8_piece* pieces, int n, void* hip_stream);

/* Steps 1, 3 and 4 in one pass over a fragment that needs no combine (the steps of the flow
 * diagram around the all-reduce, fused by this library for fragments that own all their
 * blocks).  The fragment must consist of whole 32-row bands: start a multiple of 32 * cols
 * and start + len a multiple of 32 * cols or equal to rows * cols (the whole weight is one
 * such fragment); otherwise MXFP8_ERR_RANGE.  Every block it touches then lies wholly
 * inside it, so its amax are final: the call computes them, writes them to amax_row /
 * amax_col when those are given (overwriting, not merging), and writes the E8M0 scales and
 * the E4M3 data exactly as mxfp8_partial_amax into zero-filled amax, mxfp8_compute_scales
 * and mxfp8_partial_cast would.  The input is read once.  The column-wise work (amax_col,
 * scale_col, data_col) happens iff data_col != NULL, which then requires scale_col; when
 * data_col is NULL, amax_col and scale_col are ignored.  Required: input, scale_row,
 * data_row; amax_row and amax_col are optional outputs.  Outputs must not overlap the input
 * or each other.  Reads: rows, cols, start, len, in_dtype, preround_bf16, input, amax_row,
 * amax_col, scale_row, scale_col, data_row, data_col. */
int mxfp8_quantize(const mxfp8_piece* pieces, int n, void* hip_stream);

/* Message for the calling thread's last non-OK status (static storage, thread-local). */
const char* mxfp8_last_error(void);

/* The kernel source this library was built from: 16 hex digits of SHA-256 over the kernel
 * source with its comments and blank space removed, as the build computed it, or "unknown"
 * for a build that did not set it.  Static storage; host-only.  For tying a measurement to
 * the source it ran. */
const char* mxfp8_build_id(void);

/* Times the kernels of the calling thread's next call of a launching entry point
 * (mxfp8_partial_amax, mxfp8_combine_amax, mxfp8_compute_scales, mxfp8_partial_cast,
 * mxfp8_scales_and_cast, mxfp8_quantize): start_event and stop_event are hipEvent_t handles
 * the caller created (host pointers, caller-owned).  That call launches through
 * hipExtLaunchKernel, and the runtime stamps start_event when the call's first kernel starts
 * and stop_event when its last kernel ends, so hipEventElapsedTime gives the kernels' time
 * without the dispatch around them.  The next such call consumes the events whether it
 * launches, launches nothing (an empty call: the events stay unrecorded) or fails; both
 * NULL cancels.  Not for a stream being captured into a graph.  Returns MXFP8_OK, or
 * MXFP8_ERR_ARG if exactly one event is NULL.  Host-only; launches nothing. */
int mxfp8_time_next_call(void* start_event, void* stop_event);

/* Validates a whole call of entry point kernel = 0 (mxfp8_partial_amax), 1
 * (mxfp8_partial_cast), 2 (mxfp8_scales_and_cast), 3 (mxfp8_quantize) or 4
 * (mxfp8_compute_scales) exactly as that entry point does, every piece and the pieces
 * against each other, and returns the status it would return before launching anything
 * (MXFP8_OK if it would launch).  Host-only; launches nothing.  For callers that validate a
 * fixed plan once and replay it. */
int mxfp8_check_call(const mxfp8_piece* pieces, int n, int kernel);

/* Which kernel variant a piece would use for kernel 0 = partial amax, 1 = partial cast,
 * 2 = scales and cast, 3 = quantize (each validated as for its entry point):
 * 1 = the vectorized path (16-byte loads of row segments, for rows of whole 16-byte chunks:
 * cols % 8 == 0 for BF16, cols % 4 == 0 for FP32, whatever the alignment of input and
 * outputs), 2 (partial cast only) = the vectorized path in tiles that own whole 128-byte
 * lines of the outputs, taken when the outputs' rows do not start on a 128-byte line (such
 * as fragment-sized outputs) while cols is a multiple of 128 and both outputs share their
 * offset within a line, 0 = the element-wise path (other cols), negative = the piece fails
 * validation (the status code, negated).
 * Host-only; launches nothing.  For a BF16 input the vectorized path may read, never writes,
 * the other 2 bytes of the 4-byte word that holds the fragment's first element and of the one
 * that holds its last element, and ignores them; no kernel reads anything else outside the
 * fragment. */
int mxfp8_query_path(const mxfp8_piece* piece, int kernel);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_PARTIAL_H */
