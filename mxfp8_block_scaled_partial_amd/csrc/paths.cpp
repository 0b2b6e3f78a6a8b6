// Kernel-path selection of libmxfp8partial.so: which kernels take a validated piece.  Host
// code only (no HIP kernels), shared by the launchers in kernels.hip and the path query of the
// C ABI in abi.cpp.
#include "mxfp8_internal.h"

namespace mxfp8 {

// Rows of whole 16-byte chunks (cols a multiple of 8 for BF16, of 4 for FP32): a chunk then
// never crosses a block boundary or a row end, every row has the same alignment, and a row's
// short last block (cols % 32 != 0) is a whole number of chunks.  The input needs only its
// element alignment (dword loads, plus a 2-byte shift for BF16 at 2 mod 4), and outputs at any
// byte offset are written through aligned windows or the line-owned cast tiles.
bool vec_common_ok(const Piece& p) { return p.cols % (16 / elem_size(p.dtype)) == 0; }

// Offset (in elements, 1 .. kLineBytes - 1) that puts the line-owned cast tiles' row segments
// on 128-byte lines of the outputs, or 0 when the standard tiles apply.  It needs rows of
// whole chunks and of whole lines (cols % 128 == 0), a row-wise output whose rows do not start
// on a line, and a column-wise output (if any) at the same offset within its lines.
int64_t line_shift(const Piece& p) {
  if (p.cols % kLineBytes != 0 || !vec_common_ok(p)) return 0;
  // the tiles address a row's scale bytes by 32-bit lane offsets up to one row further
  if (p.ld_sr >= (int64_t(1) << 30)) return 0;
  const uintptr_t dr = (reinterpret_cast<uintptr_t>(p.data_row) - (uintptr_t)p.start) % kLineBytes;
  if (dr == 0) return 0;
  if (p.data_col &&
      (reinterpret_cast<uintptr_t>(p.data_col) - (uintptr_t)p.start) % kLineBytes != dr)
    return 0;
  return (int64_t)(kLineBytes - dr);
}

bool amax_fast_ok(const Piece& p) { return vec_common_ok(p); }

bool cast_fast_ok(const Piece& p) { return vec_common_ok(p); }

bool cast_lines_ok(const Piece& p) { return line_shift(p) != 0; }

}  // namespace mxfp8
