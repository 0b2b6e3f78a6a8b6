// C ABI of libmxfp8partial.so (declared in include/mxfp8_partial.h): argument validation,
// direction selection from empty handles, and dispatch to the compile-time specialized HIP
// kernels.  Every check happens on the host before anything is enqueued; errors come back as
// status codes with a thread-local message, never as aborts or exceptions.
//
// Direction selection follows "Support row-only MXFP8 distributed master-weight casts"
// (section Changes and the follow-up commit): omission is an empty handle, the presence of
// the column-wise output selects the cast's column-wise work, its scales are required when
// it is requested and ignored when it is omitted, and row-wise outputs are always required.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <limits>
#include <vector>

#include "../../include/mxfp8_partial.h"
#include "mxfp8_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local mxfp8::CallEvents g_events;

// Clears the timing events when an entry point returns: they time one call, launched or not.
struct EventsOnce {
  ~EventsOnce() { g_events = mxfp8::CallEvents{}; }
};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Bytes spanned by a [nrows][ld] array whose rows hold `width` elements of `esz` bytes.
Span span2d(const void* p, int64_t nrows, int64_t ld, int64_t width, int64_t esz) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)(((nrows - 1) * ld + width) * esz)};
}

Span span1d(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)bytes};
}

int64_t nblk(int64_t n) { return (n + 31) / 32; }

enum Kind { kAmax, kScales, kCast, kFused, kQuant };
const char* kKindName[] = {"mxfp8_partial_amax", "mxfp8_compute_scales", "mxfp8_partial_cast",
                           "mxfp8_scales_and_cast", "mxfp8_quantize"};

bool aligned(const void* p, int64_t a) { return reinterpret_cast<uintptr_t>(p) % (uintptr_t)a == 0; }

// Checks one piece for entry point `kind`; fills `out`.  *skip is set for an empty fragment.
int check_piece(const mxfp8_piece& q, Kind kind, int idx, mxfp8::Piece* out, bool* skip) {
  const char* fn = kKindName[kind];
  *skip = false;
  if (q.rows < 1 || q.cols < 1)
    return fail(MXFP8_ERR_ARG, "%s: piece %d: rows and cols must be >= 1 (got %lld x %lld)", fn,
                idx, (long long)q.rows, (long long)q.cols);
  if (q.rows > std::numeric_limits<int64_t>::max() / q.cols)
    return fail(MXFP8_ERR_ARG, "%s: piece %d: rows * cols overflows", fn, idx);
  const int64_t n = q.rows * q.cols;
  if (q.start < 0 || q.len < 0 || q.start > n || q.len > n - q.start)
    return fail(MXFP8_ERR_RANGE, "%s: piece %d: fragment [%lld, %lld + %lld) outside [0, %lld]",
                fn, idx, (long long)q.start, (long long)q.start, (long long)q.len, (long long)n);
  if (q.in_dtype != MXFP8_FP32 && q.in_dtype != MXFP8_BF16)
    return fail(MXFP8_ERR_DTYPE, "%s: piece %d: unknown in_dtype %d", fn, idx, q.in_dtype);
  if (q.preround_bf16 != 0 && q.preround_bf16 != 1)
    return fail(MXFP8_ERR_ARG, "%s: piece %d: preround_bf16 must be 0 or 1", fn, idx);
  if (kind != kScales && q.preround_bf16 && q.in_dtype != MXFP8_FP32)
    return fail(MXFP8_ERR_DTYPE, "%s: piece %d: BF16 pre-rounding needs an FP32 input", fn, idx);
  if (q.len == 0) {  // empty master shard: a no-op
    *skip = true;
    return MXFP8_OK;
  }
  if (kind == kQuant) {  // every touched block must lie wholly inside the fragment
    const int64_t band = 32 * q.cols;
    const int64_t end = q.start + q.len;
    if (q.start % band != 0 || (end != n && end % band != 0))
      return fail(MXFP8_ERR_RANGE,
                  "%s: piece %d: fragment [%lld, %lld) does not cover whole 32-row bands", fn,
                  idx, (long long)q.start, (long long)end);
  }
  const int64_t esz = mxfp8::elem_size(q.in_dtype);
  const int64_t nb = nblk(q.cols), nbands = nblk(q.rows);
  mxfp8::Piece p{};
  p.rows = q.rows;
  p.cols = q.cols;
  p.start = q.start;
  p.len = q.len;
  p.dtype = q.in_dtype;
  p.preround = kind != kScales && q.preround_bf16;

  auto need_amax = [&](const mxfp8_buf& b, int64_t width, const char* what, bool required,
                       void** dst, int64_t* ld) -> int {
    if (!b.ptr) {
      if (required) return fail(MXFP8_ERR_MISSING, "%s: piece %d: %s is required", fn, idx, what);
      *dst = nullptr;
      *ld = 0;
      return MXFP8_OK;
    }
    if (b.ld < width)
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d: %s leading dimension %lld < %lld", fn, idx,
                  what, (long long)b.ld, (long long)width);
    if (!aligned(b.ptr, esz))
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d: %s is not aligned to its element size", fn,
                  idx, what);
    *dst = b.ptr;
    *ld = b.ld;
    return MXFP8_OK;
  };
  auto need_scale = [&](const mxfp8_buf& b, int64_t width, const char* what, bool required,
                        uint8_t** dst, int64_t* ld) -> int {
    if (!b.ptr) {
      if (required) return fail(MXFP8_ERR_MISSING, "%s: piece %d: %s is required", fn, idx, what);
      *dst = nullptr;
      *ld = 0;
      return MXFP8_OK;
    }
    if (b.ld < width)
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d: %s leading dimension %lld < %lld", fn, idx,
                  what, (long long)b.ld, (long long)width);
    *dst = static_cast<uint8_t*>(b.ptr);
    *ld = b.ld;
    return MXFP8_OK;
  };
  int st;
  if (kind != kScales) {
    if (!q.input) return fail(MXFP8_ERR_ARG, "%s: piece %d: input is NULL with len > 0", fn, idx);
    if (!aligned(q.input, esz))
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d: input is not aligned to its element size", fn,
                  idx);
    p.input = q.input;
  }
  if (kind == kAmax || kind == kScales) {
    if ((st = need_amax(q.amax_row, nb, "amax_row", true, &p.amax_row, &p.ld_ar))) return st;
    if ((st = need_amax(q.amax_col, q.cols, "amax_col", false, &p.amax_col, &p.ld_ac))) return st;
  }
  if (kind == kScales) {
    if ((st = need_scale(q.scale_row, nb, "scale_row", true, &p.scale_row, &p.ld_sr))) return st;
    if ((st = need_scale(q.scale_col, q.cols, "scale_col", p.amax_col != nullptr, &p.scale_col,
                         &p.ld_sc)))
      return st;
    if (!p.amax_col) p.scale_col = nullptr;  // column-wise scales not updated when absent
  }
  if (kind == kFused) {  // the column-wise work, amax included, follows data_col
    if ((st = need_amax(q.amax_row, nb, "amax_row", true, &p.amax_row, &p.ld_ar))) return st;
    if (q.data_col &&
        (st = need_amax(q.amax_col, q.cols, "amax_col", true, &p.amax_col, &p.ld_ac)))
      return st;
  }
  if (kind == kQuant) {  // amax are optional outputs; the column-wise ones follow data_col
    if ((st = need_amax(q.amax_row, nb, "amax_row", false, &p.amax_row, &p.ld_ar))) return st;
    if (q.data_col &&
        (st = need_amax(q.amax_col, q.cols, "amax_col", false, &p.amax_col, &p.ld_ac)))
      return st;
  }
  if (kind == kCast || kind == kFused || kind == kQuant) {
    if (!q.data_row) return fail(MXFP8_ERR_MISSING, "%s: piece %d: data_row is required", fn, idx);
    if ((st = need_scale(q.scale_row, nb, "scale_row", true, &p.scale_row, &p.ld_sr))) return st;
    p.data_row = static_cast<uint8_t*>(q.data_row);
    p.data_col = static_cast<uint8_t*>(q.data_col);
    if (p.data_col) {
      if ((st = need_scale(q.scale_col, q.cols, "scale_col", true, &p.scale_col, &p.ld_sc)))
        return st;
    } else {
      p.scale_col = nullptr;  // omitted column-wise output: its scales are ignored
      p.ld_sc = 0;
    }
  }

  // Buffers written by the call must not overlap anything else the call touches.
  const Span in = span1d(p.input, p.len * esz);
  const Span ar = p.amax_row ? span2d(p.amax_row, p.rows, p.ld_ar, nb, esz) : Span{0, 0};
  const Span ac = p.amax_col ? span2d(p.amax_col, nbands, p.ld_ac, p.cols, esz) : Span{0, 0};
  const Span sr = p.scale_row ? span2d(p.scale_row, p.rows, p.ld_sr, nb, 1) : Span{0, 0};
  const Span sc = p.scale_col ? span2d(p.scale_col, nbands, p.ld_sc, p.cols, 1) : Span{0, 0};
  const Span dr = p.data_row ? span1d(p.data_row, p.len) : Span{0, 0};
  const Span dc = p.data_col ? span1d(p.data_col, p.len) : Span{0, 0};
  auto clash = [&](Span a, Span b, const char* wa, const char* wb) -> int {
    if (a.hi > a.lo && b.hi > b.lo && overlaps(a, b))
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d: %s overlaps %s", fn, idx, wa, wb);
    return MXFP8_OK;
  };
  if (kind == kAmax) {
    if ((st = clash(ar, in, "amax_row", "input")) || (st = clash(ac, in, "amax_col", "input")) ||
        (st = clash(ar, ac, "amax_row", "amax_col")))
      return st;
  } else if (kind == kScales) {
    if ((st = clash(sr, ar, "scale_row", "amax_row")) || (st = clash(sr, ac, "scale_row", "amax_col")) ||
        (st = clash(sc, ar, "scale_col", "amax_row")) || (st = clash(sc, ac, "scale_col", "amax_col")) ||
        (st = clash(sr, sc, "scale_row", "scale_col")))
      return st;
  } else {
    if (kind == kQuant &&  // the amax are outputs here
        ((st = clash(ar, in, "amax_row", "input")) || (st = clash(ac, in, "amax_col", "input")) ||
         (st = clash(ar, ac, "amax_row", "amax_col"))))
      return st;
    if ((kind == kFused || kind == kQuant) &&
        ((st = clash(sr, in, "scale_row", "input")) || (st = clash(sc, in, "scale_col", "input")) ||
         (st = clash(sr, sc, "scale_row", "scale_col")) ||
         (st = clash(sr, ar, "scale_row", "amax_row")) || (st = clash(sr, ac, "scale_row", "amax_col")) ||
         (st = clash(sc, ar, "scale_col", "amax_row")) || (st = clash(sc, ac, "scale_col", "amax_col")) ||
         (st = clash(dr, ar, "data_row", "amax_row")) || (st = clash(dr, ac, "data_row", "amax_col")) ||
         (st = clash(dc, ar, "data_col", "amax_row")) || (st = clash(dc, ac, "data_col", "amax_col"))))
      return st;
    if ((st = clash(dr, in, "data_row", "input")) || (st = clash(dc, in, "data_col", "input")) ||
        (st = clash(dr, dc, "data_row", "data_col")) || (st = clash(dr, sr, "data_row", "scale_row")) ||
        (st = clash(dr, sc, "data_row", "scale_col")) || (st = clash(dc, sr, "data_col", "scale_row")) ||
        (st = clash(dc, sc, "data_col", "scale_col")))
      return st;
  }
  *out = p;
  return MXFP8_OK;
}

// A buffer one piece of a call uses: its bytes, what it is, and whether the call writes it.
struct Use {
  uintptr_t lo, hi;
  int64_t ld;
  int role;      // index into kRoleName
  bool write;
  int piece;     // first piece using it
  bool shared;   // more than one piece uses this very array
};
const char* kRoleName[] = {"input", "amax_row", "amax_col", "scale_row", "scale_col", "data_row",
                           "data_col"};

// The buffers of validated piece p for entry point `kind` (absent ones are left out).
void uses_of(const mxfp8::Piece& p, Kind kind, int idx, std::vector<Use>& out) {
  const int64_t esz = mxfp8::elem_size(p.dtype);
  const int64_t nb = nblk(p.cols), nbands = nblk(p.rows);
  const bool amax_w = kind == kAmax || kind == kQuant;
  const bool scale_w = kind == kScales || kind == kFused || kind == kQuant;
  auto add = [&](const void* ptr, Span sp, int64_t ld, int role, bool w) {
    if (ptr && sp.hi > sp.lo) out.push_back({sp.lo, sp.hi, ld, role, w, idx, false});
  };
  add(p.input, span1d(p.input, p.len * esz), 0, 0, false);
  add(p.amax_row, span2d(p.amax_row, p.rows, p.ld_ar, nb, esz), p.ld_ar, 1, amax_w);
  add(p.amax_col, span2d(p.amax_col, nbands, p.ld_ac, p.cols, esz), p.ld_ac, 2, amax_w);
  add(p.scale_row, span2d(p.scale_row, p.rows, p.ld_sr, nb, 1), p.ld_sr, 3, scale_w);
  add(p.scale_col, span2d(p.scale_col, nbands, p.ld_sc, p.cols, 1), p.ld_sc, 4, scale_w);
  add(p.data_row, span1d(p.data_row, p.len), 0, 5, true);
  add(p.data_col, span1d(p.data_col, p.len), 0, 6, true);
}

// Across the pieces of one call, a buffer that one piece writes must not overlap a buffer of
// another piece, except that pieces may share an amax or scale array (the same pointer,
// leading dimension and extent in the same role): that is how the pieces of one weight merge
// their blocks.  Within a piece, check_piece has already ruled out overlaps.
int check_across(const std::vector<mxfp8::Piece>& ps, const std::vector<int>& idx, Kind kind) {
  const char* fn = kKindName[kind];
  std::vector<Use> u;
  for (size_t i = 0; i < ps.size(); ++i) uses_of(ps[i], kind, idx[i], u);
  // one entry per shared array
  std::sort(u.begin(), u.end(), [](const Use& a, const Use& b) {
    if (a.lo != b.lo) return a.lo < b.lo;
    if (a.hi != b.hi) return a.hi < b.hi;
    if (a.role != b.role) return a.role < b.role;
    if (a.ld != b.ld) return a.ld < b.ld;
    return a.piece < b.piece;
  });
  std::vector<Use> v;
  for (const Use& x : u) {
    if (!v.empty() && x.role >= 1 && x.role <= 4 && v.back().role == x.role &&
        v.back().lo == x.lo && v.back().hi == x.hi && v.back().ld == x.ld) {
      if (v.back().piece != x.piece) v.back().shared = true;
      continue;
    }
    v.push_back(x);
  }
  // sweep in address order; `active` holds the buffers that reach past the current start
  std::vector<const Use*> active;
  for (const Use& x : v) {
    size_t keep = 0;
    for (const Use* a : active)
      if (a->hi > x.lo) active[keep++] = a;
    active.resize(keep);
    for (const Use* a : active) {
      if (!(a->write || x.write)) continue;
      if (!a->shared && !x.shared && a->piece == x.piece) continue;  // one piece: checked
      return fail(MXFP8_ERR_LAYOUT, "%s: piece %d's %s overlaps piece %d's %s", fn, x.piece,
                  kRoleName[x.role], a->piece, kRoleName[a->role]);
    }
    active.push_back(&x);
  }
  return MXFP8_OK;
}

// Validates a whole call (every piece, then the pieces against each other); fills `todo` with
// the pieces that have work.
int validate_call(const mxfp8_piece* pieces, int n, Kind kind, std::vector<mxfp8::Piece>& todo) {
  const char* fn = kKindName[kind];
  if (n < 0) return fail(MXFP8_ERR_ARG, "%s: n = %d < 0", fn, n);
  if (n > 0 && !pieces) return fail(MXFP8_ERR_ARG, "%s: pieces is NULL", fn);
  // validate everything first, so a bad piece enqueues nothing
  for (int i = 0; i < n; ++i) {
    mxfp8::Piece p;
    bool skip;
    const int st = check_piece(pieces[i], kind, i, &p, &skip);
    if (st) return st;
  }
  todo.clear();
  std::vector<int> idx;  // each one's index in the caller's array
  todo.reserve(n);
  idx.reserve(n);
  for (int i = 0; i < n; ++i) {
    mxfp8::Piece p;
    bool skip;
    check_piece(pieces[i], kind, i, &p, &skip);
    if (!skip) {
      todo.push_back(p);
      idx.push_back(i);
    }
  }
  if (todo.size() > 1) return check_across(todo, idx, kind);
  return MXFP8_OK;
}

template <typename Launch>
int run_pieces(const mxfp8_piece* pieces, int n, void* stream, Kind kind, Launch launch) {
  const EventsOnce once;
  const char* fn = kKindName[kind];
  std::vector<mxfp8::Piece> todo;
  const int st = validate_call(pieces, n, kind, todo);
  if (st) return st;
  if (todo.empty()) return MXFP8_OK;
  const hipError_t e = launch(todo.data(), (int)todo.size(), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MXFP8_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MXFP8_OK;
}

}  // namespace

namespace mxfp8 {
CallEvents& call_events() { return g_events; }
}  // namespace mxfp8

extern "C" {

int mxfp8_partial_amax(const mxfp8_piece* pieces, int n, void* hip_stream) {
  return run_pieces(pieces, n, hip_stream, kAmax, mxfp8::launch_partial_amax);
}

int mxfp8_compute_scales(const mxfp8_piece* pieces, int n, void* hip_stream) {
  return run_pieces(pieces, n, hip_stream, kScales, mxfp8::launch_compute_scales);
}

int mxfp8_partial_cast(const mxfp8_piece* pieces, int n, void* hip_stream) {
  return run_pieces(pieces, n, hip_stream, kCast, mxfp8::launch_partial_cast);
}

int mxfp8_scales_and_cast(const mxfp8_piece* pieces, int n, void* hip_stream) {
  return run_pieces(pieces, n, hip_stream, kFused, mxfp8::launch_scales_and_cast);
}

int mxfp8_quantize(const mxfp8_piece* pieces, int n, void* hip_stream) {
  return run_pieces(pieces, n, hip_stream, kQuant, mxfp8::launch_quantize);
}

int mxfp8_combine_amax(void* dst, const void* const* srcs, int k, int64_t count,
                       int32_t amax_dtype, void* hip_stream) {
  const EventsOnce once;
  const char* fn = "mxfp8_combine_amax";
  if (amax_dtype != MXFP8_FP32 && amax_dtype != MXFP8_BF16)
    return fail(MXFP8_ERR_DTYPE, "%s: unknown amax_dtype %d", fn, amax_dtype);
  if (k < 1) return fail(MXFP8_ERR_ARG, "%s: k = %d < 1", fn, k);
  if (count < 0) return fail(MXFP8_ERR_ARG, "%s: count = %lld < 0", fn, (long long)count);
  if (!srcs) return fail(MXFP8_ERR_ARG, "%s: srcs is NULL", fn);
  if (count == 0) return MXFP8_OK;
  const int64_t esz = mxfp8::elem_size(amax_dtype);
  if (!dst) return fail(MXFP8_ERR_MISSING, "%s: dst is NULL", fn);
  if (!aligned(dst, esz)) return fail(MXFP8_ERR_LAYOUT, "%s: dst is misaligned", fn);
  const Span d = span1d(dst, count * esz);
  for (int j = 0; j < k; ++j) {
    if (!srcs[j]) return fail(MXFP8_ERR_MISSING, "%s: srcs[%d] is NULL", fn, j);
    if (!aligned(srcs[j], esz)) return fail(MXFP8_ERR_LAYOUT, "%s: srcs[%d] is misaligned", fn, j);
    if (j == 0 && srcs[j] == dst) continue;  // in place on the first source
    if (overlaps(d, span1d(srcs[j], count * esz)))
      return fail(MXFP8_ERR_LAYOUT, "%s: dst overlaps srcs[%d] (only dst == srcs[0] is allowed)",
                  fn, j);
  }
  const hipError_t e = mxfp8::launch_combine(dst, srcs, k, count, amax_dtype,
                                             static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess)
    return fail(MXFP8_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MXFP8_OK;
}

const char* mxfp8_last_error(void) { return g_err; }

// Set by the build (build.py) to the hash of the kernel source it compiled.
#ifndef MXFP8_KERNEL_SOURCE_HASH
#define MXFP8_KERNEL_SOURCE_HASH "unknown"
#endif

const char* mxfp8_build_id(void) { return MXFP8_KERNEL_SOURCE_HASH; }

int mxfp8_time_next_call(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(MXFP8_ERR_ARG, "mxfp8_time_next_call: give both events or neither");
  g_events.start = static_cast<hipEvent_t>(start_event);
  g_events.stop = static_cast<hipEvent_t>(stop_event);
  return MXFP8_OK;
}

int mxfp8_check_call(const mxfp8_piece* pieces, int n, int kernel) {
  if (kernel < 0 || kernel > 4)
    return fail(MXFP8_ERR_ARG, "mxfp8_check_call: kernel must be 0 (amax), 1 (cast), 2 "
                               "(scales and cast), 3 (quantize) or 4 (scales)");
  const Kind kinds[5] = {kAmax, kCast, kFused, kQuant, kScales};
  std::vector<mxfp8::Piece> todo;
  return validate_call(pieces, n, kinds[kernel], todo);
}

int mxfp8_query_path(const mxfp8_piece* piece, int kernel) {
  if (!piece) return -fail(MXFP8_ERR_ARG, "mxfp8_query_path: piece is NULL");
  if (kernel < 0 || kernel > 3)
    return -fail(MXFP8_ERR_ARG, "mxfp8_query_path: kernel must be 0 (amax), 1 (cast), 2 "
                                "(scales and cast) or 3 (quantize)");
  mxfp8::Piece p;
  bool skip;
  const Kind kinds[4] = {kAmax, kCast, kFused, kQuant};
  const int st = check_piece(*piece, kinds[kernel], 0, &p, &skip);
  if (st) return -st;
  if (skip) return 0;
  if (kernel == 0) return (int)mxfp8::amax_fast_ok(p);
  if (kernel == 1 && mxfp8::cast_lines_ok(p)) return 2;
  return (int)mxfp8::cast_fast_ok(p);
}

}  // extern "C"
