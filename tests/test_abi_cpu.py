"""CPU tests of the C ABI boundary: the library loads and exports every function that
include/mxfp8_partial.h declares, the ctypes layout matches the header, and host-side
validation returns the documented status codes.  Nothing here launches a kernel: every call
either fails validation, is an empty fragment (a no-op), or is the host-only path query."""
import ctypes
import glob
import os
import re
import subprocess

import pytest
import torch

from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import writeback as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

# fake device addresses: validation compares them but never dereferences them
BASE = 0x7F0000000000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(mxfp8_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == set(B.EXPORTS)
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_piece_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "mxfp8_partial.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(mxfp8_piece),"
        " offsetof(mxfp8_piece,input), offsetof(mxfp8_piece,amax_row),"
        " offsetof(mxfp8_piece,amax_col), offsetof(mxfp8_piece,scale_row),"
        " offsetof(mxfp8_piece,scale_col), offsetof(mxfp8_piece,data_row),"
        " offsetof(mxfp8_piece,data_col), sizeof(mxfp8_buf));return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", f"-I{ROOT}/include", str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    P = B.Piece
    want = [ctypes.sizeof(P), P.input.offset, P.amax_row.offset, P.amax_col.offset,
            P.scale_row.offset, P.scale_col.offset, P.data_row.offset, P.data_col.offset,
            ctypes.sizeof(B.Buf)]
    assert got == want


def raw_piece(rows=64, cols=64, start=0, length=None, dtype=B.BF16, pre=0, **bufs):
    n = rows * cols if length is None else length
    esz = 2 if dtype == B.BF16 else 4
    nb, nbands = (cols + 31) // 32, (rows + 31) // 32
    default = {
        "input": BASE,
        "amax_row": B.Buf(BASE + 0x10000000, nb), "amax_col": B.Buf(BASE + 0x20000000, cols),
        "scale_row": B.Buf(BASE + 0x30000000, nb), "scale_col": B.Buf(BASE + 0x40000000, cols),
        "data_row": BASE + 0x50000000, "data_col": BASE + 0x60000000}
    default.update(bufs)
    del esz, nbands
    return B.Piece(rows, cols, start, n, dtype, pre, default["input"], default["amax_row"],
                   default["amax_col"], default["scale_row"], default["scale_col"],
                   default["data_row"], default["data_col"])


def call(fn, *pieces):
    arr = (B.Piece * len(pieces))(*pieces)
    return getattr(B.lib(), fn)(arr, len(pieces), None)


AMAX, SCALES, CAST = "mxfp8_partial_amax", "mxfp8_compute_scales", "mxfp8_partial_cast"
FUSED = "mxfp8_scales_and_cast"
QUANT = "mxfp8_quantize"


@pytest.mark.parametrize("fn", [AMAX, SCALES, CAST, FUSED, QUANT])
def test_shape_range_dtype_errors(fn):
    assert call(fn, raw_piece(rows=0)) == B.ERR_ARG
    assert call(fn, raw_piece(cols=-3)) == B.ERR_ARG
    assert call(fn, raw_piece(start=1)) == B.ERR_RANGE           # runs one past the end
    assert call(fn, raw_piece(start=-1, length=4)) == B.ERR_RANGE
    assert call(fn, raw_piece(start=4096, length=1)) == B.ERR_RANGE
    assert call(fn, raw_piece(dtype=7)) == B.ERR_DTYPE
    assert "piece 0" in B.mxfp8_last_error()
    assert B.lib()[fn](None, -1, None) == B.ERR_ARG
    assert B.lib()[fn](None, 1, None) == B.ERR_ARG


def test_preround_needs_fp32():
    assert call(AMAX, raw_piece(dtype=B.BF16, pre=1)) == B.ERR_DTYPE
    assert call(CAST, raw_piece(dtype=B.BF16, pre=1)) == B.ERR_DTYPE
    assert call(FUSED, raw_piece(dtype=B.BF16, pre=1)) == B.ERR_DTYPE
    assert call(QUANT, raw_piece(dtype=B.BF16, pre=1)) == B.ERR_DTYPE
    assert call(AMAX, raw_piece(dtype=B.BF16, pre=2)) == B.ERR_ARG


@pytest.mark.parametrize("fn", [AMAX, SCALES, CAST, FUSED, QUANT])
def test_empty_fragment_is_a_no_op_even_with_null_buffers(fn):
    p = B.Piece(64, 64, 17, 0, B.BF16, 0, None, B.Buf(None, 0), B.Buf(None, 0), B.Buf(None, 0),
                B.Buf(None, 0), None, None)
    assert call(fn, p) == B.OK
    assert call(fn) == B.OK  # n == 0


def test_required_buffers():
    assert call(AMAX, raw_piece(amax_row=B.Buf(None, 0))) == B.ERR_MISSING
    assert call(AMAX, raw_piece(input=None)) == B.ERR_ARG
    assert call(SCALES, raw_piece(scale_row=B.Buf(None, 0))) == B.ERR_MISSING
    # column-wise amax present -> column-wise scales required
    assert call(SCALES, raw_piece(scale_col=B.Buf(None, 0))) == B.ERR_MISSING
    assert call(CAST, raw_piece(data_row=None)) == B.ERR_MISSING
    assert call(CAST, raw_piece(scale_row=B.Buf(None, 0))) == B.ERR_MISSING
    # requested column-wise output needs its scales
    assert call(CAST, raw_piece(scale_col=B.Buf(None, 0))) == B.ERR_MISSING
    assert "scale_col" in B.mxfp8_last_error()


def test_scales_and_cast_required_buffers():
    assert call(FUSED, raw_piece(input=None)) == B.ERR_ARG
    for name in ("amax_row", "scale_row"):
        assert call(FUSED, raw_piece(**{name: B.Buf(None, 0)})) == B.ERR_MISSING
        assert name in B.mxfp8_last_error()
    assert call(FUSED, raw_piece(data_row=None)) == B.ERR_MISSING
    # column-wise output present: its amax and scales are required
    for name in ("amax_col", "scale_col"):
        assert call(FUSED, raw_piece(**{name: B.Buf(None, 0)})) == B.ERR_MISSING
        assert name in B.mxfp8_last_error()
    # column-wise output absent: amax_col and scale_col are ignored, even when invalid
    p = raw_piece(data_col=None, amax_col=B.Buf(BASE + 0x20000001, 1),
                  scale_col=B.Buf(BASE + 0x40000000, 1))
    assert B.mxfp8_query_path(p, 2) == 1
    assert B.mxfp8_query_path(raw_piece(data_col=None, amax_col=B.Buf(None, 0),
                                        scale_col=B.Buf(None, 0)), 2) == 1
    # the cast alone needs no amax at all
    assert B.mxfp8_query_path(raw_piece(amax_row=B.Buf(None, 0), amax_col=B.Buf(None, 0)), 1) == 1
    assert B.mxfp8_query_path(raw_piece(amax_row=B.Buf(None, 0)), 2) == -B.ERR_MISSING


def test_scales_and_cast_layout_and_overlap_errors():
    q = B.mxfp8_query_path
    assert q(raw_piece(amax_row=B.Buf(BASE + 0x10000000, 1)), 2) == -B.ERR_LAYOUT  # ld < 2
    assert q(raw_piece(amax_col=B.Buf(BASE + 0x20000002 - 1, 64)), 2) == -B.ERR_LAYOUT
    assert q(raw_piece(scale_col=B.Buf(BASE + 0x40000000, 63)), 2) == -B.ERR_LAYOUT
    # written scales or data overlapping what the call reads, or each other
    cases = [dict(scale_row=B.Buf(BASE + 0x10000000, 2)),            # scale_row on amax_row
             dict(scale_col=B.Buf(BASE + 0x20000000 + 64, 64)),     # scale_col on amax_col
             dict(scale_row=B.Buf(BASE + 8, 2)),                    # scale_row on input
             dict(data_row=BASE + 0x10000000),                      # data_row on amax_row
             dict(data_col=BASE + 0x20000000 + 2),                  # data_col on amax_col
             dict(scale_col=B.Buf(BASE + 0x30000000 + 64, 64)),     # scale_col on scale_row
             dict(data_row=BASE + 0x40000000)]                      # data_row on scale_col
    for c in cases:
        assert q(raw_piece(**c), 2) == -B.ERR_LAYOUT, c
        assert "overlaps" in B.mxfp8_last_error()


def test_quantize_needs_whole_bands():
    q = B.mxfp8_query_path
    # 100 x 64: bands of 32 rows = 2048 elements; the last band is short (4 rows)
    assert q(raw_piece(rows=100, cols=64), 3) == 1                      # the whole weight
    assert q(raw_piece(rows=100, cols=64, start=2048, length=4096), 3) == 1
    assert q(raw_piece(rows=100, cols=64, start=6144, length=256), 3) == 1  # short last band
    assert q(raw_piece(rows=100, cols=64, start=2048, length=2048), 3) == 1
    for s, l in ((1, 2047), (0, 2047), (2048, 100), (32, 2016), (0, 6399)):
        assert q(raw_piece(rows=100, cols=64, start=s, length=l), 3) == -B.ERR_RANGE, (s, l)
        assert "32-row bands" in B.mxfp8_last_error()
    assert call(QUANT, raw_piece(rows=100, cols=64, start=64, length=64)) == B.ERR_RANGE
    # element-wise layout for rows that are not whole 16-byte chunks
    assert q(raw_piece(rows=40, cols=45), 3) == 0 and q(raw_piece(rows=40, cols=40), 3) == 1


def test_quantize_buffers():
    q = B.mxfp8_query_path
    # amax are optional outputs
    assert q(raw_piece(amax_row=B.Buf(None, 0), amax_col=B.Buf(None, 0)), 3) == 1
    assert call(QUANT, raw_piece(data_row=None)) == B.ERR_MISSING
    assert call(QUANT, raw_piece(scale_row=B.Buf(None, 0))) == B.ERR_MISSING
    assert call(QUANT, raw_piece(scale_col=B.Buf(None, 0))) == B.ERR_MISSING
    assert call(QUANT, raw_piece(input=None)) == B.ERR_ARG
    # row-only: column-wise buffers ignored, even when invalid
    assert q(raw_piece(data_col=None, amax_col=B.Buf(BASE + 1, 1), scale_col=B.Buf(None, 0)),
             3) == 1
    # a given amax must be laid out correctly and must not overlap anything
    assert q(raw_piece(amax_row=B.Buf(BASE + 0x10000000, 1)), 3) == -B.ERR_LAYOUT
    for c in (dict(amax_row=B.Buf(BASE + 64, 2)),                     # amax_row on input
              dict(amax_col=B.Buf(BASE + 0x10000000, 64)),            # amax_col on amax_row
              dict(amax_col=B.Buf(BASE + 0x30000000 + 16, 64)),       # amax_col on scale_row
              dict(data_col=BASE + 0x20000000 + 4)):                  # data_col on amax_col
        assert q(raw_piece(**c), 3) == -B.ERR_LAYOUT, c
        assert "overlaps" in B.mxfp8_last_error()


def test_omitted_columnwise_output_ignores_its_scales():
    # data_col absent: a scale_col with an invalid leading dimension is ignored
    p = raw_piece(data_col=None, scale_col=B.Buf(BASE + 0x40000000, 1))
    assert B.mxfp8_query_path(p, 1) >= 0
    # with data_col present the same scale_col is rejected
    p = raw_piece(scale_col=B.Buf(BASE + 0x40000000, 1))
    assert B.mxfp8_query_path(p, 1) == -B.ERR_LAYOUT
    # amax without the column direction ignores nothing it needs: row-only is valid
    p = raw_piece(amax_col=B.Buf(None, 0))
    assert B.mxfp8_query_path(p, 0) >= 0


def test_layout_errors():
    assert call(AMAX, raw_piece(amax_row=B.Buf(BASE + 0x10000000, 1))) == B.ERR_LAYOUT  # ld < 2
    assert call(AMAX, raw_piece(amax_col=B.Buf(BASE + 0x20000000, 63))) == B.ERR_LAYOUT
    assert call(AMAX, raw_piece(input=BASE + 1)) == B.ERR_LAYOUT          # misaligned BF16
    assert call(AMAX, raw_piece(dtype=B.FP32, input=BASE + 2)) == B.ERR_LAYOUT
    assert call(AMAX, raw_piece(amax_row=B.Buf(BASE + 1, 2))) == B.ERR_LAYOUT
    assert call(SCALES, raw_piece(scale_row=B.Buf(BASE + 0x30000000, 1))) == B.ERR_LAYOUT


def test_overlap_errors():
    # input overlapping the row-wise data it is cast into
    assert call(CAST, raw_piece(data_row=BASE + 100)) == B.ERR_LAYOUT
    assert "overlaps" in B.mxfp8_last_error()
    assert call(CAST, raw_piece(data_col=BASE + 0x50000000 + 10)) == B.ERR_LAYOUT
    assert call(AMAX, raw_piece(amax_col=B.Buf(BASE + 0x10000000 + 8, 64))) == B.ERR_LAYOUT
    assert call(SCALES, raw_piece(scale_row=B.Buf(BASE + 0x10000000, 2))) == B.ERR_LAYOUT


def test_combine_validation():
    L = B.lib()
    srcs = (ctypes.c_void_p * 3)(BASE, BASE + 0x1000000, BASE + 0x2000000)
    assert L.mxfp8_combine_amax(BASE + 0x3000000, srcs, 0, 16, B.FP32, None) == B.ERR_ARG
    assert L.mxfp8_combine_amax(BASE + 0x3000000, srcs, 3, -1, B.FP32, None) == B.ERR_ARG
    assert L.mxfp8_combine_amax(BASE + 0x3000000, srcs, 3, 16, 9, None) == B.ERR_DTYPE
    assert L.mxfp8_combine_amax(BASE + 0x3000000, srcs, 3, 0, B.FP32, None) == B.OK
    assert L.mxfp8_combine_amax(None, srcs, 3, 16, B.FP32, None) == B.ERR_MISSING
    assert L.mxfp8_combine_amax(BASE + 0x3000002, srcs, 3, 16, B.FP32, None) == B.ERR_LAYOUT
    # dst may alias srcs[0] only; partial overlap of a later source is rejected
    assert L.mxfp8_combine_amax(BASE + 0x1000000 + 4, srcs, 3, 16, B.FP32, None) == B.ERR_LAYOUT
    nul = (ctypes.c_void_p * 2)(BASE, None)
    assert L.mxfp8_combine_amax(BASE + 0x3000000, nul, 2, 16, B.BF16, None) == B.ERR_MISSING


def test_query_path_selects_vector_kernel_for_whole_chunk_rows():
    q = B.mxfp8_query_path
    assert q(raw_piece(), 0) == 1 and q(raw_piece(), 1) == 1
    # any alignment of input and outputs stays on the vector path
    assert q(raw_piece(start=17, length=100, input=BASE + 34,
                       data_row=BASE + 0x50000000 + 17, data_col=BASE + 0x60000000 + 17), 1) == 1
    assert q(raw_piece(start=17, length=100), 0) == 1
    p = raw_piece(start=32, length=64, input=BASE + 64, data_row=BASE + 0x50000000 + 3)
    assert q(p, 0) == 1 and q(p, 1) == 1
    # rows of whole 16-byte chunks (8 BF16 / 4 FP32 values) but not whole 32-value blocks:
    # still the vector path; other widths: the element-wise path
    assert q(raw_piece(rows=40, cols=40), 0) == 1 and q(raw_piece(rows=40, cols=40), 1) == 1
    assert q(raw_piece(rows=40, cols=44), 0) == 0                   # BF16: 44 % 8 != 0
    assert q(raw_piece(rows=40, cols=44, dtype=B.FP32), 0) == 1     # FP32: 44 % 4 == 0
    assert q(raw_piece(rows=40, cols=45, dtype=B.FP32), 1) == 0
    assert q(raw_piece(rows=40, cols=45), 1) == 0
    assert q(raw_piece(rows=0), 0) == -B.ERR_ARG
    assert q(raw_piece(), 5) == -B.ERR_ARG
    assert q(raw_piece(), 2) == 1 and q(raw_piece(rows=40, cols=45), 2) == 0
    assert q(raw_piece(), 4) == -B.ERR_ARG


# ------------------------------------------------------------------ binding marshalling


def test_binding_maps_zero_element_tensors_to_empty_handles():
    # zero-element views that still have storage become NULL, before any device check
    storage = torch.zeros(64, dtype=torch.uint8)
    empty_view = storage[10:10]
    assert empty_view.numel() == 0 and empty_view.untyped_storage().nbytes() == 64
    p = B.make_piece(4, 32, 0, None, length=0, in_dtype=torch.float32, data_row=empty_view,
                     scale_col=torch.zeros(0, 0, dtype=torch.uint8))
    assert p.data_row is None and p.scale_col.ptr is None and p.input is None


def test_binding_rejects_host_tensors_and_bad_dtypes():
    x = torch.zeros(64, dtype=torch.float32)
    with pytest.raises(ValueError):
        B.make_piece(2, 32, 0, x)
    with pytest.raises(ValueError):
        B.make_piece(2, 32, 0, torch.zeros(64, dtype=torch.float16))
    with pytest.raises(ValueError):
        B.make_piece(2, 32, 0, None, length=64, in_dtype=torch.float32,
                     amax_row=torch.zeros(2, 1, dtype=torch.bfloat16))


# ------------------------------------------------------------------ batch helper host logic


def test_split_fragment_pieces():
    specs = [W.WeightSpec(4, 32, True), W.WeightSpec(2, 32, False), W.WeightSpec(3, 64, True)]
    # sizes 128, 64, 192 -> offsets 0, 128, 192
    assert W.split_fragment(specs, 100, 200) == [(0, 100, 28, 0), (1, 0, 64, 28),
                                                 (2, 0, 108, 92)]
    assert W.split_fragment(specs, 128, 0) == []
    assert W.split_fragment(specs, 0, 384) == [(0, 0, 128, 0), (1, 0, 64, 128), (2, 0, 192, 192)]


def test_packed_amax_layout():
    specs = [W.WeightSpec(40, 96, True), W.WeightSpec(33, 64, False)]
    p = W.PackedAmax(specs, torch.bfloat16, "cpu")
    assert p.numel == 40 * 3 + 2 * 96 + 33 * 2
    r0, c0 = p.views(0)
    r1, c1 = p.views(1)
    assert r0.shape == (40, 3) and c0.shape == (2, 96) and r1.shape == (33, 2) and c1 is None
    assert c0.data_ptr() - r0.data_ptr() == 40 * 3 * 2
    assert r1.data_ptr() - r0.data_ptr() == (40 * 3 + 2 * 96) * 2


def test_whole_bands_of_a_piece():
    spec = W.WeightSpec(100, 64, True)    # bands of 2048 elements, the last one 256
    band, n = 2048, 6400
    assert W.whole_bands(spec, 0, n) == (0, n)
    assert W.whole_bands(spec, 5, n) == (band, n)          # short last band counts as whole
    assert W.whole_bands(spec, 5, 4100) == (band, 2 * band)
    lo, hi = W.whole_bands(spec, 5, 2100)                  # no whole band inside
    assert lo >= hi
    assert W.whole_bands(spec, band, 3 * band) == (band, 3 * band)
    assert W.whole_bands(spec, 3 * band + 1, n) == (4 * band, n)
    lo, hi = W.whole_bands(spec, 3 * band + 1, n - 1)
    assert lo >= hi


def test_boundary_spans_cover_exactly_the_shared_entries():
    """The single-pass combine covers the packed entries of every block that a partial piece
    touches (brute force over the elements), and only whole bands of them."""
    import numpy as np
    specs = [W.WeightSpec(100, 64, True), W.WeightSpec(70, 96, False), W.WeightSpec(64, 32, True)]
    total = sum(s.numel for s in specs)
    g = np.random.Generator(np.random.PCG64(5))
    for trial in range(20):
        cuts = np.sort(g.integers(0, total + 1, 3))
        frags = [(int(a), int(b - a)) for a, b in zip(np.r_[0, cuts], np.r_[cuts, total])]
        spans = W.boundary_spans(specs, frags)
        covered = set()
        for lo, hi in spans:
            covered |= set(range(lo, hi))
        offs = W.PackedAmax(specs, torch.float32, "meta").offsets
        need = set()
        for fs, fl in frags:
            for (i, s, n, _) in W.split_fragment(specs, fs, fl):
                sp = specs[i]
                lo, hi = W.whole_bands(sp, s, s + n)
                parts = [(s, s + n)] if lo >= hi else [(s, lo), (hi, s + n)]
                nb = (sp.cols + 31) // 32
                for a, b in parts:
                    for e in range(a, b):
                        r, c = divmod(e, sp.cols)
                        need.add(offs[i] + r * nb + c // 32)
                        if sp.colwise:
                            need.add(offs[i] + sp.amax_row_entries + (r // 32) * sp.cols + c)
        assert need <= covered, trial
        # nothing outside the bands of the partial pieces
        bands = set()
        for fs, fl in frags:
            for (i, s, n, _) in W.split_fragment(specs, fs, fl):
                sp = specs[i]
                lo, hi = W.whole_bands(sp, s, s + n)
                parts = [(s, s + n)] if lo >= hi else [(s, lo), (hi, s + n)]
                for a, b in parts:
                    for e in range(a, b):
                        bands.add((i, e // sp.cols // 32))
        allowed = set()
        for i, bd in bands:
            sp = specs[i]
            nb = (sp.cols + 31) // 32
            r0, r1 = 32 * bd, min(32 * bd + 32, sp.rows)
            allowed |= set(range(offs[i] + r0 * nb, offs[i] + r1 * nb))
            if sp.colwise:
                oc = offs[i] + sp.amax_row_entries + bd * sp.cols
                allowed |= set(range(oc, oc + sp.cols))
        assert covered <= allowed, trial


# ------------------------------------------------------------------ whole-call validation

def piece_at(start, length, rows=64, cols=64, dtype=B.BF16, k=0, **bufs):
    """A piece whose input and fragment-relative outputs live in slot k of their own regions,
    sharing the weight's amax and scale arrays (as the pieces of one weight do)."""
    esz = 2 if dtype == B.BF16 else 4
    d = {"input": BASE + 0x08000000 * k + start * esz,
         "data_row": BASE + 0x50000000 + start, "data_col": BASE + 0x60000000 + start}
    d.update(bufs)
    return raw_piece(rows=rows, cols=cols, start=start, length=length, dtype=dtype, **d)


@pytest.mark.parametrize("kernel", [B.K_AMAX, B.K_CAST, B.K_SCALES_CAST, B.K_SCALES])
def test_pieces_of_one_weight_may_share_amax_and_scale_arrays(kernel):
    ps = [piece_at(0, 1000, k=0), piece_at(1000, 2000, k=1), piece_at(3000, 1096, k=2)]
    assert B.mxfp8_check_call(ps, kernel) == B.OK, B.mxfp8_last_error()


def test_whole_call_validation_matches_the_entry_points():
    bad = [piece_at(0, 1000), piece_at(1000, 100, rows=0)]
    assert B.mxfp8_check_call(bad, B.K_CAST) == B.ERR_ARG
    assert "piece 1" in B.mxfp8_last_error()
    assert call(CAST, *bad) == B.ERR_ARG
    assert B.mxfp8_check_call(bad[:1], 9) == B.ERR_ARG
    # empty pieces are skipped, as by the entry points
    empty = B.Piece(64, 64, 17, 0, B.BF16, 0, None, B.Buf(None, 0), B.Buf(None, 0),
                    B.Buf(None, 0), B.Buf(None, 0), None, None)
    assert B.mxfp8_check_call([empty, empty], B.K_QUANTIZE) == B.OK


@pytest.mark.parametrize("kernel", [B.K_CAST, B.K_SCALES_CAST])
def test_overlap_across_pieces_is_rejected(kernel):
    good = [piece_at(0, 1000, k=0), piece_at(1000, 2000, k=1)]
    assert B.mxfp8_check_call(good, kernel) == B.OK
    # piece 1's row-wise output overlaps piece 0's
    p1 = piece_at(1000, 2000, k=1, data_row=BASE + 0x50000000 + 900)
    assert B.mxfp8_check_call([good[0], p1], kernel) == B.ERR_LAYOUT
    assert "piece 1's data_row overlaps piece 0's data_row" in B.mxfp8_last_error() or \
        "piece 0's data_row overlaps piece 1's data_row" in B.mxfp8_last_error()
    # piece 1's column-wise output written over piece 0's input
    p1 = piece_at(1000, 2000, k=1, data_col=BASE + 10)
    assert B.mxfp8_check_call([good[0], p1], kernel) == B.ERR_LAYOUT
    assert "overlaps" in B.mxfp8_last_error()
    # the same through the entry point: nothing is launched
    assert call(CAST, good[0], p1) == B.ERR_LAYOUT


def test_overlap_of_a_written_array_with_another_pieces_array_is_rejected():
    # two weights: the second's amax_row partly over the first's (not the same array)
    a = piece_at(0, 4096, k=0)
    b = piece_at(0, 4096, k=1, amax_row=B.Buf(BASE + 0x10000000 + 64, 2),
                 amax_col=B.Buf(BASE + 0x28000000, 64), data_row=BASE + 0x58000000,
                 data_col=BASE + 0x68000000)
    assert B.mxfp8_check_call([a, b], B.K_AMAX) == B.ERR_LAYOUT
    assert "amax_row" in B.mxfp8_last_error()
    # the same array with another leading dimension is not shared either
    b = piece_at(0, 4096, k=1, amax_row=B.Buf(BASE + 0x10000000, 3),
                 amax_col=B.Buf(BASE + 0x28000000, 64))
    assert B.mxfp8_check_call([a, b], B.K_AMAX) == B.ERR_LAYOUT
    # a read-only array shared by the cast pieces may overlap another piece's read-only one
    c = piece_at(0, 4096, k=1, scale_row=B.Buf(BASE + 0x30000000 + 5, 2),
                 data_row=BASE + 0x58000000, data_col=BASE + 0x68000000)
    assert B.mxfp8_check_call([a, c], B.K_CAST) == B.OK
    # ... but not one the call writes
    assert B.mxfp8_check_call([a, c], B.K_SCALES) == B.ERR_LAYOUT


def test_query_path_reports_line_owned_cast_tiles():
    q = B.mxfp8_query_path
    # rows of whole 128-byte lines, outputs off a line: line-owned tiles for the cast only
    p = raw_piece(rows=64, cols=256, start=17, length=1000, input=BASE + 34,
                  data_row=BASE + 0x50000000, data_col=BASE + 0x60000000)
    assert q(p, 1) == 2 and q(p, 0) == 1 and q(p, 2) == 1
    # outputs on a line, or the two outputs at different offsets: the standard tiles
    assert q(raw_piece(rows=64, cols=256, start=17, length=1000, data_row=BASE + 0x50000000 + 17,
                       data_col=BASE + 0x60000000 + 17), 1) == 1
    assert q(raw_piece(rows=64, cols=256, start=17, length=1000, data_row=BASE + 0x50000000,
                       data_col=BASE + 0x60000000 + 1), 1) == 1
    # row-only: only the row-wise output counts
    assert q(raw_piece(rows=64, cols=256, start=17, length=1000, data_row=BASE + 0x50000000,
                       data_col=None), 1) == 2
    # rows that are not whole lines
    assert q(raw_piece(rows=64, cols=192, start=17, length=1000, data_row=BASE + 0x50000000,
                       data_col=BASE + 0x60000000), 1) == 1


def test_call_timing_needs_both_events_or_neither():
    """mxfp8_time_next_call arms the next launching call with a start and a stop event; one
    without the other is an argument error, and both NULL cancels.  An empty call consumes
    the events without launching anything."""
    L = B.lib()
    fake = ctypes.c_void_p(BASE)
    assert L.mxfp8_time_next_call(fake, None) == B.ERR_ARG
    assert "both events" in B.mxfp8_last_error()
    assert L.mxfp8_time_next_call(None, fake) == B.ERR_ARG
    assert L.mxfp8_time_next_call(None, None) == B.OK
    # armed, then consumed by an empty call (nothing launched, no event touched)
    assert L.mxfp8_time_next_call(fake, fake) == B.OK
    assert L.mxfp8_partial_amax(None, 0, None) == B.OK
    assert L.mxfp8_time_next_call(None, None) == B.OK


def test_library_reports_the_kernel_source_it_was_built_from():
    """mxfp8_build_id is the build's hash of the kernel source (comments and blank space
    removed); the in-tree library must be built from the current source."""
    from mxfp8_block_scaled_partial_amd import build as hip_build

    bid = B.mxfp8_build_id(B.load_library(B.LIB_PATH))
    assert re.fullmatch(r"[0-9a-f]{16}", bid), bid
    assert bid == hip_build.kernel_source_hash(), (
        "libmxfp8partial.so was built from another kernel source; rebuild it")
