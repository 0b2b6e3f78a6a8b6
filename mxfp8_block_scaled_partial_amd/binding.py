"""Python binding of libmxfp8partial.so: the C ABI of include/mxfp8_partial.h under the same
names, for torch tensors.

Marshalling only: tensors become device pointers and leading dimensions, zero-element tensors
(including views that still have storage) become empty handles, and the call runs on torch's
current stream.  Every step of the path runs in the library's HIP kernels; there is no CPU
fallback, and a missing or unloadable library raises :class:`LibraryNotBuilt`.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MXFP8_PARTIAL_LIB names another build of the same sources (the host-code
# sanitizer build of the CPU tests loads this way)
LIB_PATH = os.environ.get("MXFP8_PARTIAL_LIB") or os.path.join(HERE, "libmxfp8partial.so")

FP32 = 0
BF16 = 1

OK, ERR_ARG, ERR_RANGE, ERR_DTYPE, ERR_LAYOUT, ERR_MISSING, ERR_HIP = range(7)
STATUS_NAMES = {OK: "OK", ERR_ARG: "ERR_ARG", ERR_RANGE: "ERR_RANGE", ERR_DTYPE: "ERR_DTYPE",
                ERR_LAYOUT: "ERR_LAYOUT", ERR_MISSING: "ERR_MISSING", ERR_HIP: "ERR_HIP"}

# every entry point declared in include/mxfp8_partial.h
EXPORTS = ("mxfp8_partial_amax", "mxfp8_combine_amax", "mxfp8_compute_scales",
           "mxfp8_partial_cast", "mxfp8_scales_and_cast", "mxfp8_quantize", "mxfp8_last_error",
           "mxfp8_check_call", "mxfp8_query_path", "mxfp8_time_next_call", "mxfp8_build_id")

# kernel numbers of mxfp8_check_call / mxfp8_query_path
K_AMAX, K_CAST, K_SCALES_CAST, K_QUANTIZE, K_SCALES = range(5)


class LibraryNotBuilt(RuntimeError):
    pass


class Mxfp8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Buf(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class Piece(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("start", ctypes.c_int64), ("len", ctypes.c_int64),
                ("in_dtype", ctypes.c_int32), ("preround_bf16", ctypes.c_int32),
                ("input", ctypes.c_void_p),
                ("amax_row", Buf), ("amax_col", Buf), ("scale_row", Buf), ("scale_col", Buf),
                ("data_row", ctypes.c_void_p), ("data_col", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libmxfp8partial.so (built in-tree by ``mxfp8_block_scaled_partial_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str):
    """A build of the library at ``path`` with the C ABI's argument and result types set."""
    if not os.path.exists(path):
        raise LibraryNotBuilt(f"{path} is not built; run "
                              "`python -m mxfp8_block_scaled_partial_amd.build`")
    try:
        L = ctypes.CDLL(path)
    except OSError as e:
        raise LibraryNotBuilt(f"cannot load {path}: {e}") from e
    PP = ctypes.POINTER(Piece)
    for name in ("mxfp8_partial_amax", "mxfp8_compute_scales", "mxfp8_partial_cast",
                 "mxfp8_scales_and_cast", "mxfp8_quantize"):
        f = getattr(L, name)
        f.argtypes = [PP, ctypes.c_int, ctypes.c_void_p]
        f.restype = ctypes.c_int
    L.mxfp8_combine_amax.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p),
                                     ctypes.c_int, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_void_p]
    L.mxfp8_combine_amax.restype = ctypes.c_int
    L.mxfp8_last_error.argtypes = []
    L.mxfp8_last_error.restype = ctypes.c_char_p
    L.mxfp8_check_call.argtypes = [PP, ctypes.c_int, ctypes.c_int]
    L.mxfp8_check_call.restype = ctypes.c_int
    L.mxfp8_query_path.argtypes = [PP, ctypes.c_int]
    L.mxfp8_query_path.restype = ctypes.c_int
    L.mxfp8_time_next_call.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.mxfp8_time_next_call.restype = ctypes.c_int
    L.mxfp8_build_id.argtypes = []
    L.mxfp8_build_id.restype = ctypes.c_char_p
    return L


def _check(status: int) -> None:
    if status != OK:
        raise Mxfp8Error(status, lib().mxfp8_last_error().decode(errors="replace"))


# ------------------------------------------------------------------ tensor marshalling


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return FP32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError(f"master values must be float32 or bfloat16, got {dt}")


def _present(t) -> bool:
    return t is not None and t.numel() > 0


def _dev_ptr(t, what: str):
    """Device pointer of a tensor, or None for an absent (None or zero-element) tensor."""
    if not _present(t):
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    return t.data_ptr()


def _bytes_per_elem(t) -> int:
    return t.element_size()


def _buf2d(t, nrows: int, width: int, what: str, esize: int) -> Buf:
    """[nrows][ld] view with unit column stride; ld = the row stride in elements."""
    if not _present(t):
        return Buf(None, 0)
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    if t.element_size() != esize:
        raise ValueError(f"{what} has element size {t.element_size()}, expected {esize}")
    if t.shape[0] < nrows or t.shape[1] < width:
        raise ValueError(f"{what} shape {tuple(t.shape)} is smaller than [{nrows}, {width}]")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{what} must have unit stride along its last dimension")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return Buf(_dev_ptr(t, what), ld)


def _data1d(t, length: int, what: str):
    if not _present(t):
        return None
    if t.element_size() != 1:
        raise ValueError(f"{what} must hold 1-byte elements")
    if not t.is_contiguous() or t.numel() < length:
        raise ValueError(f"{what} must be contiguous with at least {length} elements")
    return _dev_ptr(t, what)


def nblocks(n: int) -> int:
    return (n + 31) // 32


def make_piece(rows: int, cols: int, start: int, input=None, *, length: int | None = None,
               in_dtype: torch.dtype | None = None, amax_row=None, amax_col=None,
               scale_row=None, scale_col=None, data_row=None, data_col=None,
               preround: bool = False) -> Piece:
    """Describe fragment [start, start + length) of a rows x cols weight.

    ``input`` is the fragment's values (contiguous, float32 or bfloat16); ``length`` defaults
    to ``input.numel()``.  amax/scale arguments are 2-D tensors (row stride = leading
    dimension); data arguments are fragment-relative byte tensors.  Zero-element tensors and
    None are empty handles.  The piece holds raw device pointers: the tensors must stay alive
    until the call that uses the piece has been enqueued."""
    if length is None:
        length = 0 if input is None else input.numel()
    if in_dtype is None:
        if input is None:
            raise ValueError("in_dtype is needed when input is None")
        in_dtype = input.dtype
    code = dtype_code(in_dtype)
    esize = 4 if code == FP32 else 2
    if _present(input):
        if input.dtype != in_dtype or not input.is_contiguous():
            raise ValueError("input must be contiguous and of in_dtype")
        if input.numel() < length:
            raise ValueError("input holds fewer than length elements")
    for t, what in ((amax_row, "amax_row"), (amax_col, "amax_col")):
        if _present(t) and t.dtype != in_dtype:
            raise ValueError(f"{what} must have the input dtype {in_dtype}, got {t.dtype}")
    nb, nbands = nblocks(cols), nblocks(rows)
    return Piece(rows, cols, start, length, code, int(bool(preround)),
                 _dev_ptr(input, "input"),
                 _buf2d(amax_row, rows, nb, "amax_row", esize),
                 _buf2d(amax_col, nbands, cols, "amax_col", esize),
                 _buf2d(scale_row, rows, nb, "scale_row", 1),
                 _buf2d(scale_col, nbands, cols, "scale_col", 1),
                 _data1d(data_row, length, "data_row"), _data1d(data_col, length, "data_col"))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _array(pieces):
    if isinstance(pieces, Piece):
        pieces = [pieces]
    arr = (Piece * len(pieces))(*pieces)
    return arr, len(pieces)


# ------------------------------------------------------------------ the entry points


def mxfp8_partial_amax(pieces, stream=None) -> None:
    arr, n = _array(pieces)
    _check(lib().mxfp8_partial_amax(arr, n, _stream(stream)))


def mxfp8_combine_amax(dst, srcs, stream=None) -> None:
    """dst[e] = max_j srcs[j][e] over equally sized float32 / bfloat16 amax tensors."""
    srcs = list(srcs)
    if not srcs:
        raise ValueError("need at least one source")
    code = dtype_code(dst.dtype)
    count = dst.numel()
    for s in srcs:
        if s.dtype != dst.dtype or s.numel() != count or not s.is_contiguous():
            raise ValueError("sources must be contiguous, of dst's dtype and size")
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    ptrs = (ctypes.c_void_p * len(srcs))(*[_dev_ptr(s, "src") for s in srcs])
    _check(lib().mxfp8_combine_amax(_dev_ptr(dst, "dst"), ptrs, len(srcs), count, code,
                                    _stream(stream)))


def mxfp8_compute_scales(pieces, stream=None) -> None:
    arr, n = _array(pieces)
    _check(lib().mxfp8_compute_scales(arr, n, _stream(stream)))


def mxfp8_partial_cast(pieces, stream=None) -> None:
    arr, n = _array(pieces)
    _check(lib().mxfp8_partial_cast(arr, n, _stream(stream)))


def mxfp8_scales_and_cast(pieces, stream=None) -> None:
    """mxfp8_compute_scales then mxfp8_partial_cast, in one pass over the fragment."""
    arr, n = _array(pieces)
    _check(lib().mxfp8_scales_and_cast(arr, n, _stream(stream)))


def mxfp8_quantize(pieces, stream=None) -> None:
    """amax, scales and cast in one pass, for fragments made of whole 32-row bands."""
    arr, n = _array(pieces)
    _check(lib().mxfp8_quantize(arr, n, _stream(stream)))


def mxfp8_check_call(pieces, kernel: int) -> int:
    """The status the entry point numbered ``kernel`` would return for these pieces before
    launching (host-only validation; launches nothing)."""
    arr, n = _array(pieces)
    return lib().mxfp8_check_call(arr, n, kernel)


def mxfp8_query_path(piece: Piece, kernel: int) -> int:
    return lib().mxfp8_query_path(ctypes.byref(piece), kernel)


def mxfp8_time_next_call(start_event: int, stop_event: int) -> None:
    """Times the kernels of this thread's next launching call with two hipEvent_t handles
    (raw handles, e.g. from hipEventCreateWithFlags; 0, 0 cancels)."""
    _check(lib().mxfp8_time_next_call(start_event or None, stop_event or None))


def mxfp8_build_id(library=None) -> str:
    """The kernel source hash the library (default: the loaded one) was built from."""
    return (library or lib()).mxfp8_build_id().decode()


def mxfp8_last_error() -> str:
    return lib().mxfp8_last_error().decode(errors="replace")
