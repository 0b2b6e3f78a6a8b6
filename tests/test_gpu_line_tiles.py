"""The partial cast's line-owned tiles: fragment-sized outputs whose rows start off a 128-byte
line (an FSDP rank's E4M3 buffers; data - start at any byte offset), on weights whose rows are
whole lines (cols % 128 == 0).  The tiles are shifted in the flat index so that every row
segment starts on an output line; a lane's chunk may then hold two row-wise blocks or run into
the next row.  Compared byte for byte with the oracle, with sentinel bytes around each output
to show nothing outside the fragment is written: random fragments and output offsets, the
fragment at the very start (whose first elements sit in virtual band -1) and at the very end,
single elements, short last bands, padded scale leading dimensions, row-only and
bidirectional, BF16, FP32 and FP32 pre-rounded."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl

from gpu_util import DEV, first_mismatch, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

SENT = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def to_dev_u8(a, ld=None):
    """A scale array on the device, optionally with a padded leading dimension."""
    a = np.asarray(a, dtype=np.uint8)
    if ld is not None and ld > a.shape[1]:
        p = np.full((a.shape[0], ld), 0x7F, dtype=np.uint8)
        p[:, :a.shape[1]] = a
        t = torch.from_numpy(p).to(DEV)
        return t, t[:, :a.shape[1]]
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t, t


def cast_fragment(x, rows, cols, start, length, o, pad, colwise, preround=False, ld_pad=0):
    """Casts [start, start + length) into fragment-sized outputs at byte offset pad from an
    aligned allocation; returns the output bytes and whether the line-owned tiles ran."""
    xs = to_dev(x)[start:start + length].clone()
    nb = (cols + 31) // 32
    srb, sr = to_dev_u8(o["scale_row"], nb + ld_pad if ld_pad else None)
    scb, sc = to_dev_u8(o["scale_col"], cols + ld_pad if ld_pad else None)
    drb = torch.full((length + pad + 16,), SENT, dtype=torch.uint8, device=DEV)
    dcb = torch.full((length + pad + 16,), SENT, dtype=torch.uint8, device=DEV)
    dr, dc = drb[pad:pad + length], dcb[pad:pad + length]
    p = B.make_piece(rows, cols, start, xs, scale_row=sr, scale_col=sc if colwise else None,
                     data_row=dr, data_col=dc if colwise else None, preround=preround)
    path = B.mxfp8_query_path(p, 1)
    B.mxfp8_partial_cast(p)
    torch.cuda.synchronize()
    gr, gc = to_np(drb), to_np(dcb)
    for g in ((gr, gc) if colwise else (gr,)):
        assert (g[:pad] == SENT).all() and (g[pad + length:] == SENT).all(), "wrote outside"
    if not colwise:
        assert (gc == SENT).all(), "row-only cast wrote the column-wise output"
    return gr[pad:pad + length], gc[pad:pad + length], path


def expected_path(cols, start, pad, esize):
    """2 when the line-owned tiles apply (fresh allocations are 128-byte aligned)."""
    return 2 if cols % 128 == 0 and cols % (16 // esize) == 0 and (pad - start) % 128 != 0 else 1


@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp32_pre"])
@pytest.mark.parametrize("shape", [(96, 128), (70, 384), (33, 640), (64, 1024), (1, 256),
                                   (100, 512)])
def test_random_fragments_and_offsets(dtype, shape):
    rows, cols = shape
    n = rows * cols
    pre = dtype == "fp32_pre"
    x = wl.random_matrix(rows, cols, "fp32" if pre else dtype, seed=rows * 7 + cols, kind="mixed")
    g = np.random.Generator(np.random.PCG64(rows * 1000 + cols))
    cases = [(0, n), (1, n - 1), (n - 1, 1), (17, n // 4), (min(127, n - 1), n - min(127, n - 1)),
             (n // 2 + 5, n - n // 2 - 5)]
    cases += [(int(s), int(g.integers(1, n - s + 1))) for s in g.integers(0, n, 10)]
    for s, l in cases:
        o = oracle.writeback(x, rows, cols, [(s, l)], colwise=True, preround=pre)
        for colwise in (True, False):
            pad = int(g.integers(0, 128))
            gr, gc, path = cast_fragment(x, rows, cols, s, l, o, pad, colwise, preround=pre)
            assert path == expected_path(cols, s, pad, 4 if dtype != "bf16" else 2), (s, l, pad)
            label = f"{shape} {dtype} [{s}, +{l}) pad {pad} colwise {colwise}: "
            assert not first_mismatch(gr, o["data_row"][s:s + l]), label + "data_row " + \
                first_mismatch(gr, o["data_row"][s:s + l])
            if colwise:
                assert not first_mismatch(gc, o["data_col"][s:s + l]), label + "data_col " + \
                    first_mismatch(gc, o["data_col"][s:s + l])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_every_line_offset_with_padded_scales(dtype):
    """All 128 output offsets (offset 0 takes the standard tiles) for one fragment cut inside
    blocks at both ends, with scale arrays whose leading dimensions are padded."""
    rows, cols = 72, 256
    x = wl.random_matrix(rows, cols, dtype, seed=99, kind="mixed")
    s, l = 300 + 7, rows * cols - 300 - 7 - 45
    o = oracle.writeback(x, rows, cols, [(s, l)], colwise=True)
    for off in range(128):
        pad = (off + s) % 128  # data - start = allocation + pad - s = allocation + off (mod 128)
        gr, gc, path = cast_fragment(x, rows, cols, s, l, o, pad, True, ld_pad=3 + off % 5)
        assert path == (1 if off == 0 else 2), off
        assert not first_mismatch(gr, o["data_row"][s:s + l]), (off, first_mismatch(gr, o["data_row"][s:s + l]))
        assert not first_mismatch(gc, o["data_col"][s:s + l]), (off, first_mismatch(gc, o["data_col"][s:s + l]))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_output_offsets_that_differ_take_the_standard_tiles(dtype):
    """A column-wise output at another line offset than the row-wise one keeps the standard
    tiles (window stores), with the same bytes."""
    rows, cols = 64, 256
    x = wl.random_matrix(rows, cols, dtype, seed=5, kind="mixed")
    s, l = 17, rows * cols - 17 - 9
    o = oracle.writeback(x, rows, cols, [(s, l)], colwise=True)
    xs = to_dev(x)[s:s + l].clone()
    _, sr = to_dev_u8(o["scale_row"])
    _, sc = to_dev_u8(o["scale_col"])
    drb = torch.zeros(l + 64, dtype=torch.uint8, device=DEV)
    dcb = torch.zeros(l + 64, dtype=torch.uint8, device=DEV)
    p = B.make_piece(rows, cols, s, xs, scale_row=sr, scale_col=sc, data_row=drb[3:3 + l],
                     data_col=dcb[10:10 + l])
    assert B.mxfp8_query_path(p, 1) == 1
    B.mxfp8_partial_cast(p)
    torch.cuda.synchronize()
    assert not first_mismatch(to_np(drb)[3:3 + l], o["data_row"][s:s + l])
    assert not first_mismatch(to_np(dcb)[10:10 + l], o["data_col"][s:s + l])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_several_pieces_in_one_launch(dtype):
    """Pieces of several weights, each with fragment-sized outputs at its own offset, go out
    as one grouped launch of the line-owned tiles."""
    shapes = [(40, 128), (64, 384), (33, 256), (96, 128)]
    pieces, keep, want = [], [], []
    for i, (rows, cols) in enumerate(shapes):
        x = wl.random_matrix(rows, cols, dtype, seed=40 + i, kind="mixed")
        s = 13 * i + 3
        l = rows * cols - s - 5 * i
        o = oracle.writeback(x, rows, cols, [(s, l)], colwise=i % 2 == 0)
        xs = to_dev(x)[s:s + l].clone()
        _, sr = to_dev_u8(o["scale_row"])
        sc = to_dev_u8(o["scale_col"])[1] if i % 2 == 0 else None
        drb = torch.full((l + 64,), SENT, dtype=torch.uint8, device=DEV)
        dcb = torch.full((l + 64,), SENT, dtype=torch.uint8, device=DEV)
        pad = 1 + 11 * i
        p = B.make_piece(rows, cols, s, xs, scale_row=sr, scale_col=sc, data_row=drb[pad:pad + l],
                         data_col=dcb[pad:pad + l] if i % 2 == 0 else None)
        assert B.mxfp8_query_path(p, 1) == 2
        pieces.append(p)
        keep.append((xs, sr, sc, drb, dcb))
        want.append((o, s, l, pad, i % 2 == 0))
    B.mxfp8_partial_cast(pieces)
    torch.cuda.synchronize()
    for (xs, sr, sc, drb, dcb), (o, s, l, pad, colwise) in zip(keep, want):
        gr, gc = to_np(drb), to_np(dcb)
        assert not first_mismatch(gr[pad:pad + l], o["data_row"][s:s + l])
        assert (gr[:pad] == SENT).all() and (gr[pad + l:] == SENT).all()
        if colwise:
            assert not first_mismatch(gc[pad:pad + l], o["data_col"][s:s + l])
        else:
            assert (gc == SENT).all()
