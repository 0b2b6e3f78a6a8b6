"""CPU oracle for the MXFP8 partial amax / combine / scale / cast path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product package never imports it, and the
two share no code: this wrapper talks to ``mxfp8_oracle.c`` (plain C, binary64 arithmetic,
built with gcc) through ctypes and numpy only.

Buffers are numpy arrays on the host:
  * BF16 values are carried as ``uint16`` bit patterns, FP32 values as ``float32``;
  * amax arrays have the input's dtype (the amax-dtype check quoted in the review threads of
    "Support row-only MXFP8 distributed master-weight casts"); 2-D with leading dimension
    ``shape[1]``;
  * scale arrays are ``uint8`` E8M0 bytes, data arrays ``uint8`` E4M3 bytes, fragment-relative.

Error codes from the C side raise :class:`OracleError`.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP32 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp8_oracle.c")
# MXFP8_ORACLE_LIB names another build of mxfp8_oracle.c (the sanitizer build of the CPU
# tests loads this way)
_LIB = os.environ.get("MXFP8_ORACLE_LIB") or os.path.join(_HERE, "libmxfp8_oracle.so")

_ERRORS = {1: "bad argument", 2: "fragment out of range", 3: "bad dtype", 4: "bad layout",
           5: "non-finite working value", 6: "scale byte 255"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.mxo_round_to_bf16.argtypes = [ctypes.c_double]
        L.mxo_round_to_bf16.restype = ctypes.c_double
        L.mxo_e8m0_scale.argtypes = [ctypes.c_double]
        L.mxo_e8m0_scale.restype = i32
        L.mxo_e4m3_code.argtypes = [ctypes.c_double]
        L.mxo_e4m3_code.restype = i32
        L.mxo_partial_amax.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, i64, vp, i64]
        L.mxo_combine_amax.argtypes = [vp, ctypes.POINTER(vp), i32, i64, i32]
        L.mxo_compute_scales.argtypes = [i64, i64, i64, i64, i32, vp, i64, vp, i64, vp, i64,
                                         vp, i64]
        L.mxo_partial_cast.argtypes = [i64, i64, i64, i64, i32, i32, vp, vp, i64, vp, i64, vp,
                                       vp]
        for f in (L.mxo_partial_amax, L.mxo_combine_amax, L.mxo_compute_scales,
                  L.mxo_partial_cast):
            f.restype = i32
        _lib = L
    return _lib


def _check(st: int) -> None:
    if st != 0:
        raise OracleError(f"oracle status {st}: {_ERRORS.get(st, '?')}")


def _ptr(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle buffers must be C-contiguous")
    return a.ctypes.data_as(ctypes.c_void_p)


def _ld(a, default=0):
    return default if a is None else (a.shape[1] if a.ndim == 2 else a.shape[0])


def dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return FP32
    raise ValueError(f"unsupported element array dtype {x.dtype}")


def amax_np_dtype(dtype: int):
    return np.uint16 if dtype == BF16 else np.float32


# ------------------------------------------------------------------ scalar helpers


def round_to_bf16(x: float) -> float:
    return lib().mxo_round_to_bf16(float(x))


def e8m0_scale(amax: float) -> int:
    return lib().mxo_e8m0_scale(float(amax))


def e4m3_code(v: float) -> int:
    return lib().mxo_e4m3_code(float(v))


# ------------------------------------------------------------------ the four steps


def partial_amax(x_frag, rows, cols, start, amax_row, amax_col=None, preround=False):
    """Per-block max |value| of the fragment into amax_row (and amax_col): blocks the fragment
    holds whole are set, blocks a fragment boundary cuts are MAX-merged with their entry,
    untouched entries keep their value."""
    dt = dtype_of(x_frag)
    for a in (amax_row, amax_col):
        if a is not None and a.dtype != amax_np_dtype(dt):
            raise ValueError("amax dtype must equal the input dtype")
    _check(lib().mxo_partial_amax(rows, cols, start, x_frag.size, dt, int(preround),
                                  _ptr(x_frag), _ptr(amax_row), _ld(amax_row), _ptr(amax_col),
                                  _ld(amax_col)))


def combine_amax(srcs, out=None):
    """Element-wise max over equally shaped amax buffers; returns ``out`` (new if None)."""
    srcs = [np.ascontiguousarray(s) for s in srcs]
    dt = dtype_of(srcs[0])
    out = np.empty_like(srcs[0]) if out is None else out
    arr = (ctypes.c_void_p * len(srcs))(*[s.ctypes.data for s in srcs])
    _check(lib().mxo_combine_amax(_ptr(out), arr, len(srcs), srcs[0].size, dt))
    return out


def compute_scales(rows, cols, start, length, amax_row, scale_row, amax_col=None,
                   scale_col=None):
    dt = BF16 if amax_row.dtype == np.uint16 else FP32
    _check(lib().mxo_compute_scales(rows, cols, start, length, dt, _ptr(amax_row),
                                    _ld(amax_row), _ptr(amax_col), _ld(amax_col),
                                    _ptr(scale_row), _ld(scale_row), _ptr(scale_col),
                                    _ld(scale_col)))


def partial_cast(x_frag, rows, cols, start, scale_row, data_row, scale_col=None, data_col=None,
                 preround=False):
    dt = dtype_of(x_frag)
    _check(lib().mxo_partial_cast(rows, cols, start, x_frag.size, dt, int(preround),
                                  _ptr(x_frag), _ptr(scale_row), _ld(scale_row),
                                  _ptr(scale_col), _ld(scale_col), _ptr(data_row),
                                  _ptr(data_col)))


# ------------------------------------------------------------------ whole-path convenience


def nblocks(n: int) -> int:
    return (n + 31) // 32


def new_buffers(rows, cols, dtype, colwise):
    """Zeroed amax and scale arrays with leading dimension equal to the logical width."""
    adt = amax_np_dtype(dtype)
    b = {"amax_row": np.zeros((rows, nblocks(cols)), adt),
         "scale_row": np.zeros((rows, nblocks(cols)), np.uint8),
         "amax_col": None, "scale_col": None}
    if colwise:
        b["amax_col"] = np.zeros((nblocks(rows), cols), adt)
        b["scale_col"] = np.zeros((nblocks(rows), cols), np.uint8)
    return b


def writeback(x_full, rows, cols, fragments, colwise=True, preround=False):
    """Run the whole path over a list of (start, length) fragments of ``x_full`` (flat).

    Each fragment gets its own zeroed amax buffers (one per rank), the buffers are
    MAX-combined, scales are computed for every touched block, and every fragment is cast.
    Returns a dict with the combined amax, the scales and full-size data arrays (bytes
    outside every fragment stay 0)."""
    dt = dtype_of(x_full)
    n = rows * cols
    parts = []
    for (s, l) in fragments:
        b = new_buffers(rows, cols, dt, colwise)
        partial_amax(x_full[s:s + l], rows, cols, s, b["amax_row"], b["amax_col"], preround)
        parts.append(b)
    out = new_buffers(rows, cols, dt, colwise)
    combine_amax([p["amax_row"] for p in parts], out["amax_row"])
    if colwise:
        combine_amax([p["amax_col"] for p in parts], out["amax_col"])
    data_row = np.zeros(n, np.uint8)
    data_col = np.zeros(n, np.uint8) if colwise else None
    for (s, l) in fragments:
        compute_scales(rows, cols, s, l, out["amax_row"], out["scale_row"], out["amax_col"],
                       out["scale_col"])
    for (s, l) in fragments:
        partial_cast(x_full[s:s + l], rows, cols, s, out["scale_row"], data_row[s:s + l],
                     out["scale_col"], None if data_col is None else data_col[s:s + l],
                     preround)
    out["data_row"] = data_row
    out["data_col"] = data_col
    return out
