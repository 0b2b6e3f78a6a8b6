"""GPU parity of the single-pass quantize (mxfp8_quantize) for fragments made of whole 32-row
bands, byte for byte against the oracle's path for the same fragment: partial amax into
zero-filled amax, scales, cast.  Amax and scale entries of blocks outside the fragment keep
their previous values.  Covers both kernels (vector and element-wise), short last bands,
partial last tiles, several pieces in one call, the optional amax outputs, row-only calls,
BF16 pre-rounding, inputs 2 bytes off a dword boundary, fragment-sized outputs at every byte
offset, padded leading dimensions, and the full-size weights of the workloads; and the
writeback that sends the whole bands inside each fragment through it (``single_pass``)."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import (DEV, assert_same, bits, first_mismatch, require_gpu, run_matrix, to_dev,
                      to_np)

pytestmark = pytest.mark.gpu

SENT_AMAX_BF16 = 0x1234          # a positive BF16 pattern the call must leave alone
SENT_AMAX_FP32 = 0x12345678
SENT_SCALE = 0xEE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def band_fragments(rows, cols, cuts):
    """Fragments [cuts[i] * 32 * cols, cuts[i + 1] * 32 * cols), the last clipped to the
    weight."""
    n, band = rows * cols, 32 * cols
    out = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        s, e = a * band, min(b * band, n)
        if s < e:
            out.append((s, e - s))
    return out


def sentinel_amax(shape, x):
    if x.dtype == np.uint16:
        return np.full(shape, SENT_AMAX_BF16, np.uint16)
    return np.full(shape, SENT_AMAX_FP32, np.uint32).view(np.float32)


def expected(x, rows, cols, frags, colwise, pre):
    """Per fragment: the oracle's path on zero-filled amax; its touched rows / bands are
    copied over sentinel-filled arrays."""
    n = rows * cols
    nb, nbands = oracle.nblocks(cols), oracle.nblocks(rows)
    out = {"amax_row": sentinel_amax((rows, nb), x),
           "scale_row": np.full((rows, nb), SENT_SCALE, np.uint8),
           "data_row": np.zeros(n, np.uint8),
           "amax_col": sentinel_amax((nbands, cols), x) if colwise else None,
           "scale_col": np.full((nbands, cols), SENT_SCALE, np.uint8) if colwise else None,
           "data_col": np.zeros(n, np.uint8) if colwise else None}
    for s, l in frags:
        o = oracle.writeback(x, rows, cols, [(s, l)], colwise, pre)
        r0, r1 = s // cols, (s + l) // cols
        out["amax_row"][r0:r1] = o["amax_row"][r0:r1]
        out["scale_row"][r0:r1] = o["scale_row"][r0:r1]
        out["data_row"][s:s + l] = o["data_row"][s:s + l]
        if colwise:
            b0, b1 = r0 // 32, (r1 + 31) // 32
            for k in ("amax_col", "scale_col"):
                out[k][b0:b1] = o[k][b0:b1]
            out["data_col"][s:s + l] = o["data_col"][s:s + l]
    return out


def amax_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_quantize(x, rows, cols, frags, colwise, pre, inputs="views", with_amax=True):
    n = rows * cols
    nb, nbands = oracle.nblocks(cols), oracle.nblocks(rows)
    xd = to_dev(x)
    ar = amax_dev(sentinel_amax((rows, nb), x))
    ac = amax_dev(sentinel_amax((nbands, cols), x)) if colwise else None
    sr = torch.full((rows, nb), SENT_SCALE, dtype=torch.uint8, device=DEV)
    sc = (torch.full((nbands, cols), SENT_SCALE, dtype=torch.uint8, device=DEV)
          if colwise else None)
    dr = torch.zeros(n, dtype=torch.uint8, device=DEV)
    dc = torch.zeros(n, dtype=torch.uint8, device=DEV) if colwise else None
    keep, pieces = [], []
    for s, l in frags:
        if inputs == "views":
            xs = xd[s:s + l]
        else:  # own buffer, one element past an aligned allocation (BF16: 2 bytes off)
            buf = torch.empty(l + 1, dtype=xd.dtype, device=DEV)
            buf[1:] = xd[s:s + l]
            keep.append(buf)
            xs = buf[1:]
        keep.append(xs)
        pieces.append(B.make_piece(rows, cols, s, xs, amax_row=ar if with_amax else None,
                                   amax_col=ac if with_amax else None, scale_row=sr,
                                   scale_col=sc, data_row=dr[s:s + l],
                                   data_col=None if dc is None else dc[s:s + l], preround=pre))
    for p in pieces:
        assert B.mxfp8_query_path(p, 3) == (1 if cols % (16 // xd.element_size()) == 0 else 0)
    B.mxfp8_quantize(pieces)
    torch.cuda.synchronize()
    return {"amax_row": to_np(ar), "scale_row": to_np(sr), "data_row": to_np(dr),
            "amax_col": to_np(ac) if colwise else None,
            "scale_col": to_np(sc) if colwise else None,
            "data_col": to_np(dc) if colwise else None}


def check(got, want, rows, cols, label, with_amax=True):
    for k in ("amax_row", "amax_col", "scale_row", "scale_col", "data_row", "data_col"):
        w = want[k]
        if w is None:
            assert got[k] is None
            continue
        g = got[k]
        if k.startswith("amax") and not with_amax:
            w = sentinel_amax(w.shape, w)  # not requested: left exactly as it was
        msg = first_mismatch(bits(g), bits(w), (rows, cols) if k.startswith("data") else None)
        assert not msg, f"{label}{k}: {msg}"


SHAPES = [(32, 32), (37, 45), (33, 40), (1, 70), (70, 1), (96, 33), (65, 96), (100, 64),
          (31, 4128), (64, 1056), (97, 2048), (40, 1024), (128, 96), (50, 1000), (70, 1028)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_matches_oracle(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=rows * 13 + cols, kind="mixed")
    nbands = oracle.nblocks(rows)
    fragsets = [[(0, rows * cols)]]
    if nbands >= 2:
        fragsets.append(band_fragments(rows, cols, [0, 1, nbands]))
    if nbands >= 3:
        fragsets.append(band_fragments(rows, cols, [1, 2, nbands]))  # band 0 untouched
    for frags in fragsets:
        for colwise in (True, False):
            for pre in ((False, True) if dtype == "fp32" else (False,)):
                want = expected(x, rows, cols, frags, colwise, pre)
                for inputs in ("views", "own"):
                    got = run_quantize(x, rows, cols, frags, colwise, pre, inputs)
                    check(got, want, rows, cols, f"{frags} colwise={colwise} pre={pre} {inputs}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_without_amax_outputs(dtype):
    rows, cols = 100, 192
    x = wl.random_matrix(rows, cols, dtype, seed=3, kind="mixed")
    frags = band_fragments(rows, cols, [0, 2, 4])
    want = expected(x, rows, cols, frags, True, False)
    got = run_quantize(x, rows, cols, frags, True, False, "own", with_amax=False)
    check(got, want, rows, cols, "no amax: ", with_amax=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("cols", [128, 1088])
def test_quantize_fragment_sized_outputs(dtype, cols):
    """Output buffers holding only the fragment, at every byte offset (window stores)."""
    rows = 96
    x = wl.random_matrix(rows, cols, dtype, seed=cols, kind="mixed")
    s, l = 32 * cols, 64 * cols
    want = expected(x, rows, cols, [(s, l)], True, False)
    nb = cols // 32
    xs = to_dev(x)[s:s + l].clone()
    for pad in (0, 1, 2, 3):
        sr = torch.full((rows, nb), SENT_SCALE, dtype=torch.uint8, device=DEV)
        sc = torch.full((3, cols), SENT_SCALE, dtype=torch.uint8, device=DEV)
        drb = torch.full((l + 8,), 0xA5, dtype=torch.uint8, device=DEV)
        dcb = torch.full((l + 8,), 0xA5, dtype=torch.uint8, device=DEV)
        p = B.make_piece(rows, cols, s, xs, scale_row=sr, scale_col=sc,
                         data_row=drb[pad:pad + l], data_col=dcb[pad:pad + l])
        assert B.mxfp8_query_path(p, 3) == 1
        B.mxfp8_quantize(p)
        torch.cuda.synchronize()
        gr, gc = to_np(drb), to_np(dcb)
        assert not first_mismatch(to_np(sr), want["scale_row"]), pad
        assert not first_mismatch(to_np(sc), want["scale_col"]), pad
        assert not first_mismatch(gr[pad:pad + l], want["data_row"][s:s + l]), pad
        assert not first_mismatch(gc[pad:pad + l], want["data_col"][s:s + l]), pad
        assert (gr[:pad] == 0xA5).all() and (gr[pad + l:] == 0xA5).all()
        assert (gc[:pad] == 0xA5).all() and (gc[pad + l:] == 0xA5).all()


def test_quantize_padded_leading_dimensions():
    """Padded amax / scale rows (amax_col rows off 16-byte alignment); padding untouched."""
    rows, cols = 100, 192
    x = wl.random_matrix(rows, cols, "bf16", seed=7, kind="mixed")
    nb, nbands = cols // 32, 4
    want = expected(x, rows, cols, [(0, rows * cols)], True, False)
    ard = torch.zeros(rows, nb + 5, dtype=torch.bfloat16, device=DEV)
    acd = torch.zeros(nbands, cols + 3, dtype=torch.bfloat16, device=DEV)
    srb = torch.full((rows, nb + 3), SENT_SCALE, dtype=torch.uint8, device=DEV)
    scb = torch.full((nbands, cols + 1), SENT_SCALE, dtype=torch.uint8, device=DEV)
    dr = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    dc = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    B.mxfp8_quantize(B.make_piece(rows, cols, 0, to_dev(x), amax_row=ard[:, :nb],
                                  amax_col=acd[:, :cols], scale_row=srb[:, :nb],
                                  scale_col=scb[:, :cols], data_row=dr, data_col=dc))
    torch.cuda.synchronize()
    assert not first_mismatch(to_np(ard)[:, :nb], want["amax_row"])
    assert not first_mismatch(to_np(acd)[:, :cols], want["amax_col"])
    assert (to_np(ard)[:, nb:] == 0).all() and (to_np(acd)[:, cols:] == 0).all()
    assert not first_mismatch(to_np(srb)[:, :nb], want["scale_row"])
    assert not first_mismatch(to_np(scb)[:, :cols], want["scale_col"])
    assert (to_np(srb)[:, nb:] == SENT_SCALE).all() and (to_np(scb)[:, cols:] == SENT_SCALE).all()
    assert not first_mismatch(to_np(dr), want["data_row"], (rows, cols))
    assert not first_mismatch(to_np(dc), want["data_col"], (rows, cols))


def test_quantize_row_only_ignores_columnwise_buffers():
    rows, cols = 64, 256
    x = wl.random_matrix(rows, cols, "fp32", seed=9, kind="normal")
    want = expected(x, rows, cols, [(0, rows * cols)], False, False)
    sr = torch.full((rows, 8), SENT_SCALE, dtype=torch.uint8, device=DEV)
    sc = torch.full((2, cols), SENT_SCALE, dtype=torch.uint8, device=DEV)
    ac = torch.full((2, cols), 7.0, dtype=torch.float32, device=DEV)
    dr = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    B.mxfp8_quantize(B.make_piece(rows, cols, 0, to_dev(x), amax_col=ac, scale_row=sr,
                                  scale_col=sc, data_row=dr))
    torch.cuda.synchronize()
    assert not first_mismatch(to_np(sr), want["scale_row"])
    assert not first_mismatch(to_np(dr), want["data_row"], (rows, cols))
    assert (to_np(sc) == SENT_SCALE).all() and (to_np(ac) == 7.0).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_full_size_16384x6144(dtype):
    m = wl.matrix_large(dtype)
    want = expected(m.data, m.rows, m.cols, [(0, m.rows * m.cols)], True, False)
    got = run_quantize(m.data, m.rows, m.cols, [(0, m.rows * m.cols)], True, False)
    check(got, want, m.rows, m.cols, "16384x6144: ")


def test_quantize_square_4096_preround():
    m = wl.matrix_square("fp32")
    n = m.rows * m.cols
    frags = band_fragments(m.rows, m.cols, [0, 37, 128])
    want = expected(m.data, m.rows, m.cols, frags, True, True)
    got = run_quantize(m.data, m.rows, m.cols, frags, True, True, "own")
    check(got, want, m.rows, m.cols, "4096 pre: ")
    assert sum(l for _, l in frags) == n


def test_quantize_layer_batch_weights_in_one_call():
    """The transformer layer's four weights, each quantized whole, in one call (mixed
    row-only and bidirectional pieces)."""
    batch = wl.layer_batch()
    xd = to_dev(batch.data)
    outs, pieces = [], []
    for i, (name, r, c, colwise) in enumerate(batch.tensors):
        o = batch.offsets[i]
        sr = torch.zeros(r, c // 32, dtype=torch.uint8, device=DEV)
        dr = torch.zeros(r * c, dtype=torch.uint8, device=DEV)
        sc = torch.zeros(r // 32, c, dtype=torch.uint8, device=DEV) if colwise else None
        dc = torch.zeros(r * c, dtype=torch.uint8, device=DEV) if colwise else None
        ar = torch.zeros(r, c // 32, dtype=torch.bfloat16, device=DEV)
        ac = torch.zeros(r // 32, c, dtype=torch.bfloat16, device=DEV) if colwise else None
        outs.append((ar, ac, sr, sc, dr, dc))
        pieces.append(B.make_piece(r, c, 0, xd[o:o + r * c], amax_row=ar, amax_col=ac,
                                   scale_row=sr, scale_col=sc, data_row=dr, data_col=dc))
    B.mxfp8_quantize(pieces)
    torch.cuda.synchronize()
    for i, (name, r, c, colwise) in enumerate(batch.tensors):
        o = batch.offsets[i]
        want = oracle.writeback(batch.data[o:o + r * c], r, c, [(0, r * c)], colwise)
        got = dict(zip(("amax_row", "amax_col", "scale_row", "scale_col", "data_row",
                        "data_col"), [None if t is None else to_np(t) for t in outs[i]]))
        for k, w in want.items():
            if w is None:
                continue
            msg = first_mismatch(bits(got[k]), bits(w))
            assert not msg, f"{name} {k}: {msg}"


# ------------------------------------------------------------------ writeback with single_pass


def splits(n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cuts = np.sort(g.integers(0, n + 1, k - 1))
    cuts = np.concatenate([[0], cuts, [n]])
    return [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]


@pytest.mark.parametrize("rows,cols", [(100, 64), (37, 45), (256, 96), (97, 2048), (64, 1056)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_writeback_single_pass_matches_oracle(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=rows + 5 * cols, kind="mixed")
    n = rows * cols
    band = 32 * cols
    fragsets = [[(0, n)], splits(n, 3, rows), splits(n, 5, cols),
                [(0, band + 5), (band + 5, n - band - 5)],  # one cut inside the second band
                [(0, band), (band, n - band)]]               # a cut on a band boundary
    for frags in fragsets:
        if any(l < 0 for _, l in frags):
            continue
        for colwise in (True, False):
            want = oracle.writeback(x, rows, cols, frags, colwise)
            for shared in (True, False):
                got = run_matrix(x, rows, cols, frags, colwise, inputs="own", shared=shared,
                                 single_pass=True)
                assert_same(got, want, rows, cols, f"{frags} colwise={colwise} shared={shared}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_writeback_single_pass_large_four_fragments(dtype):
    """The benchmark's launch configuration through the single-pass writeback."""
    m = wl.matrix_large(dtype)
    n = m.rows * m.cols
    cuts = [0, n // 4 + 17, n // 2 + 17, 3 * n // 4 + 17, n]
    four = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
    want = oracle.writeback(m.data, m.rows, m.cols, [(0, n)], True)
    got = run_matrix(m.data, m.rows, m.cols, four, True, inputs="views", shared=False,
                     single_pass=True)
    assert_same(got, want, m.rows, m.cols, "single pass, 4 fragments: ")
    plan = got["wb"].plan([torch.empty(l, dtype=torch.bfloat16 if dtype == "bf16" else
                                       torch.float32, device=DEV) for _, l in four])
    assert plan.n_quant == 4 and plan.n_cast == 6  # a head and / or tail at each inner cut
    # the combine covers only the 3 bands at the inner cuts: 32 rows of row-wise entries and
    # one row of column-wise entries each
    wb = got["wb"]
    assert sum(c for _, _, c in wb.combine_calls) == 3 * (32 * m.cols // 32 + m.cols)


def test_writeback_single_pass_rowonly_and_layer_batch():
    r = wl.matrix_rowonly_fragments()
    want = oracle.writeback(r.data, r.rows, r.cols, r.runs["fragments"], colwise=False)
    got = run_matrix(r.data, r.rows, r.cols, r.runs["fragments"], False, inputs="own",
                     shared=False, single_pass=True)
    assert_same(got, want, r.rows, r.cols, "row-only: ")
    batch = wl.layer_batch()
    specs = [W.WeightSpec(rr, c, colwise) for (_, rr, c, colwise) in batch.tensors]
    x_dev = to_dev(batch.data)
    wb = W.Writeback(specs, torch.bfloat16, DEV, batch.fragments, shared=False, single_pass=True)
    plan = wb.plan([x_dev[s:s + l] for s, l in batch.fragments])
    assert [nm for nm, _ in plan.stages()] == ["zero", "amax", "quantize", "combine",
                                                "scales_cast"]
    plan.run()
    torch.cuda.synchronize()
    for i, (name, rr, c, colwise) in enumerate(batch.tensors):
        o = batch.offsets[i]
        pieces = []
        for fs, fl in batch.fragments:
            lo, hi = max(fs, o), min(fs + fl, o + rr * c)
            if lo < hi:
                pieces.append((lo - o, hi - lo))
        want = oracle.writeback(batch.data[o:o + rr * c], rr, c, pieces, colwise)
        ar, ac = wb.combined.views(i)
        st = wb.storage[i]
        got = {"amax_row": to_np(ar), "amax_col": to_np(ac) if colwise else None,
               "scale_row": to_np(st.scale_row),
               "scale_col": to_np(st.scale_col) if colwise else None,
               "data_row": to_np(st.data_row),
               "data_col": to_np(st.data_col) if colwise else None}
        assert_same(got, want, rr, c, f"{name}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_pieces_in_one_call_fused_and_quantize(dtype):
    """More pieces than one launch groups (16): the library splits them over launches."""
    rows, cols = 40 * 32, 96
    x = wl.random_matrix(rows, cols, dtype, seed=77, kind="mixed")
    band = 32 * cols
    frags = [(b * band, band) for b in range(40)]           # 40 band-sized pieces
    want = expected(x, rows, cols, frags, True, False)
    got = run_quantize(x, rows, cols, frags, True, False, "own")
    check(got, want, rows, cols, "40 quantize pieces: ")
    # the fused scales + cast over 37 uneven pieces, reading the amax the quantize produced
    cuts = np.linspace(0, rows * cols, 38).astype(np.int64) + np.arange(38) % 5
    cuts[0], cuts[-1] = 0, rows * cols
    pieces37 = [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]
    xd = to_dev(x)
    ar, ac = amax_dev(got["amax_row"]), amax_dev(got["amax_col"])
    sr = torch.full((rows, cols // 32), SENT_SCALE, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows // 32, cols), SENT_SCALE, dtype=torch.uint8, device=DEV)
    dr = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    dc = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    B.mxfp8_scales_and_cast([B.make_piece(rows, cols, s, xd[s:s + l], amax_row=ar, amax_col=ac,
                                          scale_row=sr, scale_col=sc, data_row=dr[s:s + l],
                                          data_col=dc[s:s + l]) for s, l in pieces37])
    torch.cuda.synchronize()
    for k, t in (("scale_row", sr), ("scale_col", sc), ("data_row", dr), ("data_col", dc)):
        msg = first_mismatch(to_np(t), want[k])
        assert not msg, f"37 fused pieces {k}: {msg}"
