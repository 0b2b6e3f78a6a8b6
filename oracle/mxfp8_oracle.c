/*
 * mxfp8_oracle.c -- plain CPU oracle for the MXFP8 partial amax / combine / scale / cast path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path never calls it and shares
 * no code, header, table or helper with it.
 *
 * What it computes, and where that is defined:
 *  - The path itself (partial per-block amax over a contiguous fragment of the flattened
 *    weight, MAX-combine of the amax for the directions that exist, scale update for the
 *    present directions, in-place cast of the fragment to E4M3 row-wise data and optionally
 *    column-wise data): "Support row-only MXFP8 distributed master-weight casts"
 *    (TransformerEngine PR 3488), sections "Description" and "Changes", the flow diagram in
 *    the Greptile summary, and the kernel documentation quoted in the review threads
 *    (input = contiguous segment of the flattened tensor; amax buffers are [in,out];
 *    amax dtype equals the input dtype).
 *  - The numeric rules the pages leave open are taken from the OCP Microscaling (MX) v1.0
 *    and OCP 8-bit floating point (OFP8) specifications: 32-value blocks (1x32 row-wise,
 *    32x1 column-wise), shared scale X = 2^(floor(log2 amax) - emax_elem) with
 *    emax_elem = 8 for E4M3, stored as E8M0 (biased by 127, clamped to [0, 254]; a zero
 *    block takes the smallest scale), and elements rounded to E4M3 (bias 7, max 448,
 *    no infinities) with round-to-nearest-even and saturation.
 *
 * Every value is carried in IEEE binary64, where all steps below are exact except the
 * two explicit roundings (to BF16 and to E4M3), which are done with nearbyint() in the
 * default round-to-nearest-even mode.  Build without -ffast-math.
 *
 * Parity: pinned by tests/test_oracle_pins.py (hand-worked blocks, exhaustive nearest-code
 * search, torch's float8_e4m3fn and bfloat16 conversions, numpy block maxima, and the
 * fragment / transpose / power-of-two / row-only invariants).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

enum { MXO_FP32 = 0, MXO_BF16 = 1 };
enum { MXO_OK = 0, MXO_EARG = 1, MXO_ERANGE = 2, MXO_EDTYPE = 3, MXO_ELAYOUT = 4,
       MXO_ENONFINITE = 5, MXO_ESCALE = 6 };

#define BLOCK 32
#define E4M3_MAX 448.0
#define E8M0_MAX 254

/* ---------------------------------------------------------------- element access */

static double bf16_bits_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Value v is exactly representable in BF16 (caller guarantees); return its bit pattern. */
static uint16_t bf16_bits_of(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static double load_value(const void* buf, int64_t idx, int dtype) {
  if (dtype == MXO_BF16) return bf16_bits_value(((const uint16_t*)buf)[idx]);
  return (double)((const float*)buf)[idx];
}

static void store_value(void* buf, int64_t idx, int dtype, double v) {
  if (dtype == MXO_BF16)
    ((uint16_t*)buf)[idx] = bf16_bits_of(v);
  else
    ((float*)buf)[idx] = (float)v;
}

/* ---------------------------------------------------------------- roundings */

/* Round a finite value to the nearest BF16 value, ties to even (the "rounding through the
 * model dtype" of the Changes section).  BF16 has 8 significant bits and FP32's exponent
 * range, so the grid spacing at exponent q is 2^(q-7), with q floored at -126 for the
 * subnormal range.  Returns +-INFINITY when the rounded magnitude exceeds BF16's largest
 * finite value (2 - 2^-7) * 2^127. */
double mxo_round_to_bf16(double x) {
  if (x == 0.0) return x;
  double ax = fabs(x);
  int e;
  frexp(ax, &e);            /* ax = m * 2^e, m in [0.5, 1): floor(log2 ax) = e - 1 */
  int q = e - 1;
  if (q < -126) q = -126;
  double step = ldexp(1.0, q - 7);
  double r = nearbyint(ax / step) * step;
  if (r > ldexp(255.0, 120)) r = INFINITY; /* (2 - 2^-7) * 2^127 = 255 * 2^120 */
  return copysign(r, x);
}

/* E8M0 scale byte for a block whose max |value| is amax (OCP MX: X = 2^(floor(log2 amax) - 8)
 * for E4M3, biased by 127 and clamped to [0, 254]; amax == 0 gives the smallest scale). */
int mxo_e8m0_scale(double amax) {
  if (amax == 0.0) return 0;
  int e;
  frexp(amax, &e);
  long b = (long)(e - 1) - 8 + 127;
  if (b < 0) b = 0;
  if (b > E8M0_MAX) b = E8M0_MAX;
  return (int)b;
}

/* Nearest E4M3 code to v, ties to even, magnitude saturated to 448 (OFP8 E4M3: bias 7,
 * 3 mantissa bits, subnormal spacing 2^-9, no infinities).  The sign bit is kept, so
 * -0 and negative values that round to zero give 0x80. */
int mxo_e4m3_code(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a > E4M3_MAX) a = E4M3_MAX;
  int q;
  if (a < ldexp(1.0, -6)) {
    q = -6;                 /* subnormals share the spacing of the smallest binade */
  } else {
    int e;
    frexp(a, &e);
    q = e - 1;
  }
  double step = ldexp(1.0, q - 3);
  double r = nearbyint(a / step) * step; /* may carry into the next binade; still <= 448 */
  int code;
  if (r == 0.0) {
    code = 0;
  } else if (r < ldexp(1.0, -6)) {
    code = (int)(r / ldexp(1.0, -9)); /* exponent field 0, mantissa = r / 2^-9 */
  } else {
    int e;
    frexp(r, &e);
    int rq = e - 1;
    int mant = (int)(r / ldexp(1.0, rq - 3)) - 8;
    code = ((rq + 7) << 3) | mant;
  }
  return (neg << 7) | code;
}

/* ---------------------------------------------------------------- shared checks */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int check_piece(int64_t rows, int64_t cols, int64_t start, int64_t len, int dtype,
                       int preround) {
  if (rows < 1 || cols < 1) return MXO_EARG;
  if (dtype != MXO_FP32 && dtype != MXO_BF16) return MXO_EDTYPE;
  if (preround && dtype != MXO_FP32) return MXO_EDTYPE;
  if (start < 0 || len < 0 || start > rows * cols || len > rows * cols - start) return MXO_ERANGE;
  return MXO_OK;
}

/* Working value of fragment element k: the master value, optionally rounded to BF16. */
static int working_value(const void* input, int64_t k, int dtype, int preround, double* w) {
  double x = load_value(input, k, dtype);
  if (!isfinite(x)) return MXO_ENONFINITE;
  if (preround) x = mxo_round_to_bf16(x);
  if (!isfinite(x)) return MXO_ENONFINITE;
  *w = x;
  return MXO_OK;
}

/* ---------------------------------------------------------------- the four steps */

/* Is the whole block, from flat index `first` to flat index `last`, inside the fragment? */
static int block_inside(int64_t first, int64_t last, int64_t start, int64_t len) {
  return first >= start && last < start + len;
}

/* Step 1, partial amax.  Element k of the fragment is element i = start + k of the
 * row-major flattening, at row i / cols and column i % cols.  Its row-wise block is
 * (row, col / 32) and its column-wise block is (row / 32, col).  The amax buffers are
 * in/out (kernel documentation in the review threads):
 *  - a block the fragment holds whole gets the max |w| over its elements: this fragment is
 *    the only one that touches it, and its old entry is not part of the result;
 *  - a block a fragment boundary cuts becomes max(entry, |w|) over the fragment's elements
 *    in it, so the pieces of several fragments that share one buffer merge;
 *  - entries the fragment does not touch keep their value.
 * On a zero-filled buffer, which every update starts from, both kinds of block come out as
 * max(entry, |w|).  amax_col == NULL means the column-wise direction is absent. */
int mxo_partial_amax(int64_t rows, int64_t cols, int64_t start, int64_t len, int dtype,
                     int preround, const void* input, void* amax_row, int64_t ld_row,
                     void* amax_col, int64_t ld_col) {
  int st = check_piece(rows, cols, start, len, dtype, preround);
  if (st) return st;
  if (ld_row < ceil_div(cols, BLOCK) || (amax_col && ld_col < cols)) return MXO_ELAYOUT;
  /* first pass: the entry of every block the fragment holds whole starts again from 0 */
  for (int64_t k = 0; k < len; ++k) {
    int64_t i = start + k, r = i / cols, c = i % cols;
    int64_t j = c / BLOCK, b = r / BLOCK;
    int64_t row_first = r * cols + j * BLOCK;
    int64_t row_last = r * cols + (j * BLOCK + BLOCK < cols ? j * BLOCK + BLOCK : cols) - 1;
    if (block_inside(row_first, row_last, start, len))
      store_value(amax_row, r * ld_row + j, dtype, 0.0);
    if (amax_col) {
      int64_t col_first = b * BLOCK * cols + c;
      int64_t col_last = ((b * BLOCK + BLOCK < rows ? b * BLOCK + BLOCK : rows) - 1) * cols + c;
      if (block_inside(col_first, col_last, start, len))
        store_value(amax_col, b * ld_col + c, dtype, 0.0);
    }
  }
  /* second pass: every touched entry takes the max with |w| of each fragment element */
  for (int64_t k = 0; k < len; ++k) {
    int64_t i = start + k, r = i / cols, c = i % cols;
    double w;
    st = working_value(input, k, dtype, preround, &w);
    if (st) return st;
    double a = fabs(w);
    int64_t er = r * ld_row + c / BLOCK;
    if (a > load_value(amax_row, er, dtype)) store_value(amax_row, er, dtype, a);
    if (amax_col) {
      int64_t ec = (r / BLOCK) * ld_col + c;
      if (a > load_value(amax_col, ec, dtype)) store_value(amax_col, ec, dtype, a);
    }
  }
  return MXO_OK;
}

/* Step 2, MAX-combine: dst[e] = max over the k source buffers of src[j][e].  On several
 * ranks this is the one packed-amax MAX all-reduce; dst may be one of the sources. */
int mxo_combine_amax(void* dst, const void* const* srcs, int k, int64_t count, int dtype) {
  if (k < 1 || count < 0) return MXO_EARG;
  if (dtype != MXO_FP32 && dtype != MXO_BF16) return MXO_EDTYPE;
  for (int64_t e = 0; e < count; ++e) {
    double m = load_value(srcs[0], e, dtype);
    for (int j = 1; j < k; ++j) {
      double v = load_value(srcs[j], e, dtype);
      if (v > m) m = v;
    }
    store_value(dst, e, dtype, m);
  }
  return MXO_OK;
}

/* Step 3, scale update for the present directions: every block the fragment touches gets
 * the E8M0 byte of its (combined) amax.  Other scale bytes are left as they are. */
int mxo_compute_scales(int64_t rows, int64_t cols, int64_t start, int64_t len, int dtype,
                       const void* amax_row, int64_t ld_arow, const void* amax_col,
                       int64_t ld_acol, uint8_t* scale_row, int64_t ld_srow,
                       uint8_t* scale_col, int64_t ld_scol) {
  int st = check_piece(rows, cols, start, len, dtype, 0);
  if (st) return st;
  int64_t nb = ceil_div(cols, BLOCK);
  if (ld_arow < nb || ld_srow < nb) return MXO_ELAYOUT;
  if (amax_col && (!scale_col || ld_acol < cols || ld_scol < cols)) return MXO_ELAYOUT;
  for (int64_t k = 0; k < len; ++k) {
    int64_t i = start + k, r = i / cols, c = i % cols;
    scale_row[r * ld_srow + c / BLOCK] =
        (uint8_t)mxo_e8m0_scale(load_value(amax_row, r * ld_arow + c / BLOCK, dtype));
    if (amax_col)
      scale_col[(r / BLOCK) * ld_scol + c] =
          (uint8_t)mxo_e8m0_scale(load_value(amax_col, (r / BLOCK) * ld_acol + c, dtype));
  }
  return MXO_OK;
}

/* Step 4, partial cast: data_row[k] = E4M3(w * 2^(127 - s_row)) with s_row the scale byte of
 * the element's row-wise block, and, only when data_col is present, data_col[k] likewise with
 * the column-wise block's scale.  Outputs are fragment-relative: byte k belongs to element
 * start + k.  When data_col is absent, scale_col is not read. */
int mxo_partial_cast(int64_t rows, int64_t cols, int64_t start, int64_t len, int dtype,
                     int preround, const void* input, const uint8_t* scale_row, int64_t ld_srow,
                     const uint8_t* scale_col, int64_t ld_scol, uint8_t* data_row,
                     uint8_t* data_col) {
  int st = check_piece(rows, cols, start, len, dtype, preround);
  if (st) return st;
  if (ld_srow < ceil_div(cols, BLOCK)) return MXO_ELAYOUT;
  if (data_col && (!scale_col || ld_scol < cols)) return MXO_ELAYOUT;
  for (int64_t k = 0; k < len; ++k) {
    int64_t i = start + k, r = i / cols, c = i % cols;
    double w;
    st = working_value(input, k, dtype, preround, &w);
    if (st) return st;
    int sr = scale_row[r * ld_srow + c / BLOCK];
    if (sr > E8M0_MAX) return MXO_ESCALE;
    data_row[k] = (uint8_t)mxo_e4m3_code(ldexp(w, 127 - sr));
    if (data_col) {
      int sc = scale_col[(r / BLOCK) * ld_scol + c];
      if (sc > E8M0_MAX) return MXO_ESCALE;
      data_col[k] = (uint8_t)mxo_e4m3_code(ldexp(w, 127 - sc));
    }
  }
  return MXO_OK;
}
