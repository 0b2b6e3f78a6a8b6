// Internal interface between the C-ABI host layer (abi.cpp) and the HIP kernels
// (kernels.hip).  Not installed; the public interface is include/mxfp8_partial.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mxfp8 {

enum Dtype : int { kFP32 = 0, kBF16 = 1 };

// A validated piece.  Absent directions / outputs are nullptr.
struct Piece {
  int64_t rows, cols, start, len;
  int dtype;
  bool preround;
  const void* input;
  void* amax_row;
  int64_t ld_ar;
  void* amax_col;
  int64_t ld_ac;
  uint8_t* scale_row;
  int64_t ld_sr;
  uint8_t* scale_col;
  int64_t ld_sc;
  uint8_t* data_row;
  uint8_t* data_col;
};

inline int64_t elem_size(int dtype) { return dtype == kBF16 ? 2 : 4; }

// Kernel-path selection (host only; paths.cpp).
constexpr int kLineBytes = 128;  // the output lines the cast's line-owned tiles start on
// The vector kernels take any fragment of a weight whose rows are whole 16-byte chunks.
bool vec_common_ok(const Piece& p);
// Offset of the line-owned cast tiles (1 .. kLineBytes - 1 elements), or 0 for the standard
// tiles.
int64_t line_shift(const Piece& p);
// Whether the vectorized kernels apply (see mxfp8_query_path in the public header).
bool amax_fast_ok(const Piece& p);
bool cast_fast_ok(const Piece& p);
// Whether the plain cast takes the line-owned tiles.
bool cast_lines_ok(const Piece& p);

// Kernel timing of one call (mxfp8_time_next_call), this thread's: while `stop` is set, every
// launch records it when its kernel ends, and the first one records `start` when its kernel
// starts (then `start` is cleared).  The entry point that consumes them clears both.
struct CallEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
CallEvents& call_events();

// Pieces sharing a kernel specialization go out in as few launches as possible.
hipError_t launch_partial_amax(const Piece* ps, int n, hipStream_t s);
hipError_t launch_partial_cast(const Piece* ps, int n, hipStream_t s);
// The cast with the scales computed from the amax on the fly (and written for touched blocks).
hipError_t launch_scales_and_cast(const Piece* ps, int n, hipStream_t s);
// amax, scales and cast in one pass, for fragments of whole 32-row bands.
hipError_t launch_quantize(const Piece* ps, int n, hipStream_t s);
hipError_t launch_compute_scales(const Piece* ps, int n, hipStream_t s);
hipError_t launch_combine(void* dst, const void* const* srcs, int k, int64_t count, int dtype,
                          hipStream_t s);

}  // namespace mxfp8
