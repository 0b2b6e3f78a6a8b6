"""GPU parity on edge cases and per-kernel contracts, byte for byte against the oracle:
ragged shapes, short last bands, tiny fragments, padded leading dimensions, amax entries
over non-zero values (set for whole blocks, MAX-merged for cut blocks), every BF16 code at
every scale byte through the cast, scales for every non-negative BF16 amax, K-way combines,
omitted column-wise outputs, untouched bytes outside the fragment, consecutive updates with
stable pointers, determinism, and many pieces of one weight merging in a single call."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import (DEV, assert_same, bits, first_mismatch, require_gpu, run_matrix, to_dev,
                      to_np, torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def splits(n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cuts = np.sort(g.integers(0, n + 1, k - 1))
    cuts = np.concatenate([[0], cuts, [n]])
    return [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]


# ------------------------------------------------------------------ shapes and fragments

SHAPES = [(37, 45), (33, 40), (1, 70), (70, 1), (96, 33), (65, 96), (100, 64), (31, 4128),
          (64, 64), (2, 32)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_shapes_full_and_split(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=rows * 7 + cols, kind="mixed")
    n = rows * cols
    for frags in ([(0, n)], splits(n, 3, rows + cols), splits(n, 5, rows * cols)):
        for colwise in (True, False):
            want = oracle.writeback(x, rows, cols, frags, colwise)
            for inputs in ("views", "own"):
                for shared in (True, False):
                    got = run_matrix(x, rows, cols, frags, colwise, inputs=inputs, shared=shared)
                    assert_same(got, want, rows, cols,
                                f"{frags} colwise={colwise} {inputs} shared={shared}: ")


@pytest.mark.parametrize("kind", ["tiny", "huge", "normal"])
@pytest.mark.parametrize("pre", [False, True])
def test_value_ranges_fp32(kind, pre):
    rows, cols = 96, 160
    x = wl.random_matrix(rows, cols, "fp32", seed=5, kind=kind)
    for frags in ([(0, rows * cols)], [(17, 5000), (5017, rows * cols - 5017)]):
        want = oracle.writeback(x, rows, cols, frags, True, pre)
        for inputs in ("views", "own"):
            got = run_matrix(x, rows, cols, frags, True, pre, inputs=inputs)
            assert_same(got, want, rows, cols, f"{kind} pre={pre} {frags} {inputs}: ")


@pytest.mark.parametrize("start,length", [(0, 1), (5, 1), (31, 1), (0, 31), (1, 31), (16, 32),
                                          (31, 2), (95, 66), (160 * 33 - 7, 40),
                                          (160 * 95, 160), (160 * 96 - 1, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tiny_fragments(start, length, dtype):
    rows, cols = 96, 160
    x = wl.random_matrix(rows, cols, dtype, seed=start + length, kind="mixed")
    frags = [(start, length)]
    want = oracle.writeback(x, rows, cols, frags, True)
    for inputs in ("views", "own"):
        got = run_matrix(x, rows, cols, frags, True, inputs=inputs)
        assert_same(got, want, rows, cols, f"{inputs}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("inputs", ["views", "own"])
@pytest.mark.parametrize("base", ["mid_row", "row_end"])
def test_cut_at_every_position_of_a_chunk(dtype, inputs, base):
    """Two fragments cut at every element position of two 16-byte chunks (both 4-byte word
    parities for BF16): the edge tiles load each cut chunk as the words that hold its
    fragment elements, and the two fragments merge the cut blocks."""
    rows, cols = 64, 256
    n = rows * cols
    E = 8 if dtype == "bf16" else 4
    b0 = 37 * cols + 64 if base == "mid_row" else 38 * cols - 2 * E
    x = wl.random_matrix(rows, cols, dtype, seed=11 + cols, kind="mixed")
    for j in range(2 * E):
        cut = b0 + j
        frags = [(0, cut), (cut, n - cut)]
        want = oracle.writeback(x, rows, cols, frags, True)
        got = run_matrix(x, rows, cols, frags, True, inputs=inputs, shared=False)
        assert_same(got, want, rows, cols, f"cut {cut}: ")


def test_vector_and_element_paths_are_both_exercised():
    x = torch.zeros(64 * 64, dtype=torch.bfloat16, device=DEV)
    ar = torch.zeros(64, 2, dtype=torch.bfloat16, device=DEV)
    p_view = B.make_piece(64, 64, 17, x[17:117], amax_row=ar)
    own = x[17:117].clone()                     # input - start at 2 mod 4: shifted loads
    p_own = B.make_piece(64, 64, 17, own, amax_row=ar)
    assert B.mxfp8_query_path(p_view, 0) == 1
    assert B.mxfp8_query_path(p_own, 0) == 1
    y = torch.zeros(40 * 44, dtype=torch.bfloat16, device=DEV)
    ar44 = torch.zeros(40, 2, dtype=torch.bfloat16, device=DEV)
    assert B.mxfp8_query_path(B.make_piece(40, 44, 0, y, amax_row=ar44), 0) == 0
    # rows of whole 16-byte chunks with a short last block stay on the vector path
    ar40 = torch.zeros(40, 2, dtype=torch.bfloat16, device=DEV)
    assert B.mxfp8_query_path(B.make_piece(40, 40, 0, y[:1600], amax_row=ar40), 0) == 1


# rows of whole 16-byte chunks whose last 32-value block is short (cols % 32 != 0): the vector
# kernels, with the short block in the last tile of each row (1028: FP32 only, BF16 takes the
# element-wise path)
VEC_SHORT = [(40, 4104), (33, 520), (100, 1000), (64, 72), (37, 8), (70, 1028)]


@pytest.mark.parametrize("rows,cols", VEC_SHORT)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_vector_path_with_short_last_block(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=rows + 3 * cols, kind="mixed")
    n = rows * cols
    p = B.make_piece(rows, cols, 0, to_dev(x), amax_row=torch.zeros(rows, (cols + 31) // 32,
                                                                    dtype=torch_dtype(x),
                                                                    device=DEV))
    esize = 2 if dtype == "bf16" else 4
    assert B.mxfp8_query_path(p, 0) == (1 if cols % (16 // esize) == 0 else 0)
    for frags in ([(0, n)], splits(n, 3, cols), splits(n, 6, rows), [(17, n - 17)]):
        for colwise in (True, False):
            want = oracle.writeback(x, rows, cols, frags, colwise)
            for inputs in ("views", "own"):
                for shared in (True, False):
                    got = run_matrix(x, rows, cols, frags, colwise, inputs=inputs, shared=shared)
                    assert_same(got, want, rows, cols,
                                f"{frags} colwise={colwise} {inputs} shared={shared}: ")


@pytest.mark.parametrize("cols", [1536, 1544])
@pytest.mark.parametrize("mode", ["separate", "fused", "single_pass"])
def test_bf16_shifted_input_whole_and_partial_wave_rows(cols, mode):
    """BF16 fragments in allocations of their own, with input - start 2 bytes off a dword
    boundary: rows of whole 64-lane chunk runs take the dword after each lane's 16 bytes from
    the next lane (lane 63's from one load per row), a row's short last tile (1544 columns)
    loads it per lane.  Fragments start at odd elements, inside and on band boundaries."""
    rows = 100
    x = wl.random_matrix(rows, cols, "bf16", seed=cols, kind="mixed")
    n = rows * cols
    frags = [(0, 33 * cols + 7), (33 * cols + 7, 31 * cols), (64 * cols + 7, n - 64 * cols - 7)]
    assert all(s % 2 == 1 for s, _ in frags[1:])
    want = oracle.writeback(x, rows, cols, frags, True)
    for shared in (True, False):
        got = run_matrix(x, rows, cols, frags, True, inputs="own", shared=shared,
                         fused=mode == "fused", single_pass=mode == "single_pass")
        assert_same(got, want, rows, cols, f"{mode} shared={shared}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("offset", [0, 4, 36, 5, 64 + 2])
@pytest.mark.parametrize("fused", [False, True])
def test_fragment_outputs_on_and_off_64_byte_boundaries(dtype, offset, fused):
    """Fragment-sized outputs (fresh allocations) of fragments starting `offset` elements
    past a band boundary, on a weight with several tiles per row: data - start sits on a
    64-byte boundary (0: the common tile, streaming stores), off one but dword aligned (4, 36:
    the general tile, ordinary stores) or off a dword (5, 66: window stores)."""
    rows, cols = 96, 1536
    x = wl.random_matrix(rows, cols, dtype, seed=offset + 11, kind="mixed")
    n = rows * cols
    s = 32 * cols + offset
    l = 48 * cols - 2 * offset
    tdt = torch_dtype(x)
    xd = to_dev(x)
    nb, nbands = cols // 32, rows // 32
    ar = torch.zeros(rows, nb, dtype=tdt, device=DEV)
    ac = torch.zeros(nbands, cols, dtype=tdt, device=DEV)
    sr = torch.zeros(rows, nb, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(nbands, cols, dtype=torch.uint8, device=DEV)
    dr = torch.full((l,), 0xA5, dtype=torch.uint8, device=DEV)
    dc = torch.full((l,), 0xA5, dtype=torch.uint8, device=DEV)
    assert (dr.data_ptr() - s) % 64 == (-offset) % 64
    xs = xd[s:s + l]
    B.mxfp8_partial_amax(B.make_piece(rows, cols, s, xs, amax_row=ar, amax_col=ac))
    if fused:
        B.mxfp8_scales_and_cast(B.make_piece(rows, cols, s, xs, amax_row=ar, amax_col=ac,
                                             scale_row=sr, scale_col=sc, data_row=dr,
                                             data_col=dc))
    else:
        B.mxfp8_compute_scales(B.make_piece(rows, cols, s, None, length=l, in_dtype=tdt,
                                            amax_row=ar, amax_col=ac, scale_row=sr,
                                            scale_col=sc))
        B.mxfp8_partial_cast(B.make_piece(rows, cols, s, xs, scale_row=sr, scale_col=sc,
                                          data_row=dr, data_col=dc))
    torch.cuda.synchronize()
    want = oracle.writeback(x, rows, cols, [(s, l)], True)
    assert not first_mismatch(to_np(dr), want["data_row"][s:s + l])
    assert not first_mismatch(to_np(dc), want["data_col"][s:s + l])


# ------------------------------------------------------------------ padded leading dimensions


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_padded_leading_dimensions_and_padding_untouched(dtype):
    rows, cols = 70, 96
    x = wl.random_matrix(rows, cols, dtype, seed=3, kind="mixed")
    nb, nbands = 3, 3
    tdt = torch_dtype(x)
    xd = to_dev(x)
    frag = (40, rows * cols - 100)
    xs = xd[frag[0]:frag[0] + frag[1]]
    # padded arrays: padding holds a sentinel the library must never touch
    ar = torch.full((rows, nb + 5), 3.0, dtype=tdt, device=DEV)
    ac = torch.full((nbands, cols + 7), 3.0, dtype=tdt, device=DEV)
    ar[:, :nb] = 0
    ac[:, :cols] = 0
    sr = torch.full((rows, nb + 2), 0xEE, dtype=torch.uint8, device=DEV)
    sc = torch.full((nbands, cols + 9), 0xEE, dtype=torch.uint8, device=DEV)
    dr = torch.full((rows * cols,), 0xCD, dtype=torch.uint8, device=DEV)
    dc = torch.full((rows * cols,), 0xCD, dtype=torch.uint8, device=DEV)
    s, l = frag
    B.mxfp8_partial_amax(B.make_piece(rows, cols, s, xs, amax_row=ar, amax_col=ac))
    B.mxfp8_compute_scales(B.make_piece(rows, cols, s, None, length=l, in_dtype=tdt,
                                        amax_row=ar, amax_col=ac, scale_row=sr, scale_col=sc))
    B.mxfp8_partial_cast(B.make_piece(rows, cols, s, xs, scale_row=sr, scale_col=sc,
                                      data_row=dr[s:s + l], data_col=dc[s:s + l]))
    torch.cuda.synchronize()
    o = oracle.new_buffers(rows, cols, oracle.dtype_of(x), True)
    oracle.partial_amax(x[s:s + l], rows, cols, s, o["amax_row"], o["amax_col"])
    osr = np.full((rows, nb), 0xEE, np.uint8)
    osc = np.full((nbands, cols), 0xEE, np.uint8)
    oracle.compute_scales(rows, cols, s, l, o["amax_row"], osr, o["amax_col"], osc)
    odr = np.full(rows * cols, 0xCD, np.uint8)
    odc = np.full(rows * cols, 0xCD, np.uint8)
    oracle.partial_cast(x[s:s + l], rows, cols, s, osr, odr[s:s + l], osc, odc[s:s + l])
    assert_same({"amax_row": to_np(ar)[:, :nb], "amax_col": to_np(ac)[:, :cols],
                 "scale_row": to_np(sr)[:, :nb], "scale_col": to_np(sc)[:, :cols],
                 "data_row": to_np(dr), "data_col": to_np(dc)},
                {"amax_row": o["amax_row"], "amax_col": o["amax_col"], "scale_row": osr,
                 "scale_col": osc, "data_row": odr, "data_col": odc}, rows, cols)
    sentinel = bits(to_np(torch.full((1,), 3.0, dtype=tdt)))[0]
    assert (bits(to_np(ar)[:, nb:]) == sentinel).all()
    assert (bits(to_np(ac)[:, cols:]) == sentinel).all()
    assert (to_np(sr)[:, nb:] == 0xEE).all() and (to_np(sc)[:, cols:] == 0xEE).all()


# ------------------------------------------------------------------ per-kernel contracts


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("inputs", ["views", "own"])
@pytest.mark.parametrize("cols,frag", [
    (128, (1000, 6000)),               # vector path: interior tiles, cut bands, cut row blocks
    (128, (32 * 128 + 17, 96 * 128 - 32 * 128 - 22)),  # edge tiles holding whole column blocks
    (4104, (4104 * 32 + 5, 4104 * 40)),  # vector path, short last row block in every row
    (99, (1000, 6000)),                # element-wise path
    (99, (32 * 99 + 17, 96 * 99 - 32 * 99 - 22)),
])
def test_amax_sets_whole_blocks_and_merges_cut_blocks(dtype, inputs, cols, frag):
    """Entries start at random non-negative values, often above the block maxima: blocks the
    fragment holds whole must come out as their max, cut blocks as the max with the entry,
    untouched blocks unchanged (the oracle's rule), on every amax kernel path."""
    rows = 96
    x = wl.random_matrix(rows, cols, dtype, seed=9, kind="normal")
    nb = B.nblocks(cols)
    g = np.random.Generator(np.random.PCG64(1))
    init = np.abs(g.standard_normal((rows, nb)) * 1.5).astype(np.float32)
    initc = np.abs(g.standard_normal((3, cols)) * 1.5).astype(np.float32)
    if dtype == "bf16":
        init, initc = wl.to_dtype(init, "bf16").reshape(rows, nb), wl.to_dtype(initc, "bf16").reshape(3, cols)
    s, l = frag
    ar, ac = to_dev(init.ravel()).view(rows, nb), to_dev(initc.ravel()).view(3, cols)
    xd = to_dev(x)
    xs = xd[s:s + l] if inputs == "views" else xd[s:s + l].clone()
    piece = B.make_piece(rows, cols, s, xs, amax_row=ar, amax_col=ac)
    assert B.mxfp8_query_path(piece, 0) == (1 if cols % 8 == 0 else 0)
    B.mxfp8_partial_amax(piece)
    torch.cuda.synchronize()
    war, wac = init.copy(), initc.copy()
    oracle.partial_amax(x[s:s + l], rows, cols, s, war, wac)
    assert not first_mismatch(bits(to_np(ar)), bits(war))
    assert not first_mismatch(bits(to_np(ac)), bits(wac))
    # the case holds blocks of every kind in both directions
    assert (bits(war) != bits(init)).any() and (bits(wac) != bits(initc)).any()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("frags", [
    [(1000, 6000)],                                   # one piece: it owns the amax arrays
    [(1000, 3001), (4001, 2999)],                     # two pieces in one call sharing them
    [(17, 128 * 96 // 4)],                            # a quarter at offset 17
])
def test_amax_merges_with_entries_on_any_alignment(dtype, offset, frags):
    """Entries start at random values; the amax arrays start `offset` entries into their
    allocations (BF16 at offset 1: rows of both arrays off 4-byte boundaries, so entries are
    updated one by one rather than in aligned pairs).  Pieces alone in a call and pieces
    sharing the arrays in one call must both give the oracle's entries."""
    rows, cols = 96, 128
    x = wl.random_matrix(rows, cols, dtype, seed=31, kind="normal")
    nb = B.nblocks(cols)
    g = np.random.Generator(np.random.PCG64(2))
    init = np.abs(g.standard_normal(rows * nb + offset) * 1.5).astype(np.float32)
    initc = np.abs(g.standard_normal(3 * cols + offset) * 1.5).astype(np.float32)
    if dtype == "bf16":
        init, initc = wl.to_dtype(init, "bf16"), wl.to_dtype(initc, "bf16")
    ard, acd = to_dev(init), to_dev(initc)
    ar = ard[offset:].view(rows, nb)
    ac = acd[offset:].view(3, cols)
    xd = to_dev(x)
    pieces = [B.make_piece(rows, cols, s, xd[s:s + l], amax_row=ar, amax_col=ac) for s, l in frags]
    B.mxfp8_partial_amax(pieces)
    torch.cuda.synchronize()
    war = init[offset:].reshape(rows, nb).copy()
    wac = initc[offset:].reshape(3, cols).copy()
    for s, l in frags:
        oracle.partial_amax(x[s:s + l], rows, cols, s, war, wac)
    assert not first_mismatch(bits(to_np(ar)), bits(war))
    assert not first_mismatch(bits(to_np(ac)), bits(wac))
    assert (bits(to_np(ard)[:offset]) == bits(init[:offset])).all()
    assert (bits(war) != bits(init[offset:].reshape(rows, nb))).any()


def test_scales_for_every_nonnegative_bf16_amax():
    codes = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite, subnormals included
    codes = np.concatenate([codes, np.zeros((-codes.size) % 64, np.uint16)])
    rows, cols = codes.size // 64, 64 * 32  # every row: 64 row-wise blocks
    ar = to_dev(codes).view(rows, 64)
    sr = torch.zeros(rows, 64, dtype=torch.uint8, device=DEV)
    B.mxfp8_compute_scales(B.make_piece(rows, cols, 0, None, length=rows * cols,
                                        in_dtype=torch.bfloat16, amax_row=ar, scale_row=sr))
    want = np.zeros((rows, 64), np.uint8)
    oracle.compute_scales(rows, cols, 0, rows * cols, codes.reshape(rows, 64), want)
    assert not first_mismatch(to_np(sr), want)


def test_scales_fp32_binade_edges():
    vals = []
    for k in range(-149, 128):
        p = np.float32(2.0 ** k)
        vals += [p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(np.inf))]
    vals += [np.float32(0), np.finfo(np.float32).max]
    v = np.array(vals, np.float32)
    v = np.concatenate([v, np.zeros((-v.size) % 32, np.float32)])
    rows, nb = v.size // 32, 32
    ar = to_dev(v).view(rows, nb)
    sr = torch.zeros(rows, nb, dtype=torch.uint8, device=DEV)
    B.mxfp8_compute_scales(B.make_piece(rows, nb * 32, 0, None, length=rows * nb * 32,
                                        in_dtype=torch.float32, amax_row=ar, scale_row=sr))
    want = np.zeros((rows, nb), np.uint8)
    oracle.compute_scales(rows, nb * 32, 0, rows * nb * 32, v.reshape(rows, nb), want)
    assert not first_mismatch(to_np(sr), want)


@pytest.mark.parametrize("k", [1, 2, 8, 9, 17])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("offset", [0, 1])
def test_combine_k_buffers(k, dtype, offset):
    count = 100003
    g = np.random.Generator(np.random.PCG64(k))
    srcs_np = [np.abs(g.standard_normal(count + offset)).astype(np.float32) for _ in range(k)]
    if dtype == "bf16":
        srcs_np = [wl.to_dtype(s, "bf16") for s in srcs_np]
    srcs = [to_dev(s)[offset:] for s in srcs_np]  # offset 1: misaligned -> scalar path
    dst = torch.empty_like(srcs[0])
    B.mxfp8_combine_amax(dst, srcs)
    want = oracle.combine_amax([s[offset:] for s in srcs_np])
    assert not first_mismatch(bits(to_np(dst)), bits(want))
    # in place on the first source
    B.mxfp8_combine_amax(srcs[0], srcs)
    assert not first_mismatch(bits(to_np(srcs[0])), bits(want))


def _probe_matrix():
    bits16 = np.arange(0x10000, dtype=np.uint32)
    finite = ((bits16 >> 7) & 0xFF) != 0xFF
    codes = bits16[finite].astype(np.uint16)      # 65024 values, a multiple of 32
    scales = np.arange(255, dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("inputs", ["views", "own"])
def test_cast_every_bf16_value_at_every_scale_byte(dtype, inputs):
    """Pins the hardware conversion (v_ldexp_f32, v_med3_f32, v_cvt_pk_fp8_f32): every finite
    BF16 value (as BF16, or widened to FP32) at every scale byte 0..254, both directions."""
    codes, scales = _probe_matrix()
    cols, rows = codes.size, scales.size
    x = np.tile(codes, rows)
    if dtype == "fp32":
        x = (x.astype(np.uint32) << 16).view(np.float32)
    scale_row = np.repeat(scales[:, None], cols // 32, axis=1).copy()
    nbands = (rows + 31) // 32
    scale_col = np.zeros((nbands, cols), np.uint8)  # column blocks: a cycle of scale bytes
    scale_col[:] = (np.arange(cols) % 255).astype(np.uint8)[None, :]
    scale_col = (scale_col + np.arange(nbands, dtype=np.uint8)[:, None] * 37) % 255
    scale_col = scale_col.astype(np.uint8)
    s = 3 if inputs == "own" else 0   # a fragment in its own buffer: element-wise kernel
    n = rows * cols - s
    xd = to_dev(x)
    xs = xd[s:] if inputs == "views" else xd[s:].clone()
    dr = torch.zeros(n, dtype=torch.uint8, device=DEV)
    dc = torch.zeros(n, dtype=torch.uint8, device=DEV)
    B.mxfp8_partial_cast(B.make_piece(rows, cols, s, xs, scale_row=to_dev_u8(scale_row),
                                      scale_col=to_dev_u8(scale_col), data_row=dr, data_col=dc))
    torch.cuda.synchronize()
    wr = np.zeros(n, np.uint8)
    wc = np.zeros(n, np.uint8)
    oracle.partial_cast(x[s:], rows, cols, s, scale_row, wr, scale_col, wc)
    assert not first_mismatch(to_np(dr), wr, (rows, cols))
    assert not first_mismatch(to_np(dc), wc, (rows, cols))


def to_dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_fp32_specific_values_through_the_cast():
    """FP32 values BF16 cannot hold: E4M3 midpoints and their neighbours, subnormals, ties
    of the BF16 pre-rounding, at unit and extreme scales."""
    mids = []
    for c in range(0x7E):
        a = (c >> 3, c & 7)
        va = (a[1] / 8) * 2.0 ** -6 if a[0] == 0 else (1 + a[1] / 8) * 2.0 ** (a[0] - 7)
        b = ((c + 1) >> 3, (c + 1) & 7)
        vb = (b[1] / 8) * 2.0 ** -6 if b[0] == 0 else (1 + b[1] / 8) * 2.0 ** (b[0] - 7)
        m = np.float32((va + vb) / 2)
        mids += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    g = np.random.Generator(np.random.PCG64(2))
    sub = (g.integers(1, 1 << 23, 2000).astype(np.uint32)).view(np.float32)
    # exact ties of the BF16 pre-rounding; high halves stay below BF16's overflow threshold
    ties = ((g.integers(1, 0x7F7E, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    v = np.concatenate([np.array(mids, np.float32), sub, ties])
    v = np.concatenate([v, -v])
    v = np.concatenate([v, np.zeros((-v.size) % 32, np.float32)])
    cols = v.size
    for scale in (127, 0, 100, 200, 254):
        for pre in (False, True):
            scale_row = np.full((1, cols // 32), scale, np.uint8)
            d = torch.zeros(cols, dtype=torch.uint8, device=DEV)
            B.mxfp8_partial_cast(B.make_piece(1, cols, 0, to_dev(v), scale_row=to_dev_u8(scale_row),
                                              data_row=d, preround=pre))
            want = np.zeros(cols, np.uint8)
            oracle.partial_cast(v, 1, cols, 0, scale_row, want, preround=pre)
            assert not first_mismatch(to_np(d), want), (scale, pre)


# ------------------------------------------------------------------ direction selection, sentinels


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_omitted_columnwise_output_skips_its_work_and_ignores_its_scales(dtype):
    rows, cols = 64, 96
    x = wl.random_matrix(rows, cols, dtype, seed=4, kind="mixed")
    xd = to_dev(x)
    o = oracle.writeback(x, rows, cols, [(0, rows * cols)], colwise=False)
    sr = to_dev_u8(o["scale_row"])
    garbage_sc = torch.full((2, cols), 0xFF, dtype=torch.uint8, device=DEV)  # would be invalid
    dr = torch.zeros(rows * cols, dtype=torch.uint8, device=DEV)
    B.mxfp8_partial_cast(B.make_piece(rows, cols, 0, xd, scale_row=sr, scale_col=garbage_sc,
                                      data_row=dr, data_col=None))
    torch.cuda.synchronize()
    assert not first_mismatch(to_np(dr), o["data_row"])
    # a requested column-wise output without scales is an error, and nothing is written
    dc = torch.full((rows * cols,), 0x5A, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.Mxfp8Error) as e:
        B.mxfp8_partial_cast(B.make_piece(rows, cols, 0, xd, scale_row=sr, data_row=dr,
                                          data_col=dc))
    assert e.value.status == B.ERR_MISSING
    assert (to_np(dc) == 0x5A).all()


@pytest.mark.parametrize("inputs", ["views", "own"])
def test_bytes_outside_the_fragment_are_untouched(inputs):
    rows, cols = 96, 160
    x = wl.random_matrix(rows, cols, "bf16", seed=12, kind="mixed")
    s, l = 1000 + 17, 7000
    o = oracle.writeback(x, rows, cols, [(s, l)])
    xd = to_dev(x)
    xs = xd[s:s + l] if inputs == "views" else xd[s:s + l].clone()
    dr = torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    dc = torch.full((rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    B.mxfp8_partial_cast(B.make_piece(rows, cols, s, xs, scale_row=to_dev_u8(o["scale_row"]),
                                      scale_col=to_dev_u8(o["scale_col"]), data_row=dr[s:s + l],
                                      data_col=dc[s:s + l]))
    torch.cuda.synchronize()
    gr, gc = to_np(dr), to_np(dc)
    assert (gr[:s] == 0xAB).all() and (gr[s + l:] == 0xAB).all()
    assert (gc[:s] == 0xAB).all() and (gc[s + l:] == 0xAB).all()
    assert not first_mismatch(gr[s:s + l], o["data_row"][s:s + l])
    assert not first_mismatch(gc[s:s + l], o["data_col"][s:s + l])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("start", [17, 18, 19, 20, 5, 1030])
@pytest.mark.parametrize("cols", [128, 1088])
def test_fragment_sized_outputs(dtype, start, cols):
    """FSDP-style outputs: the data buffers hold only the fragment, so they sit at any byte
    offset from the block grid (window stores), and the input is the rank's own buffer
    (shifted loads for BF16); several tiles per row, a partial last tile, edge tiles."""
    rows = 96
    x = wl.random_matrix(rows, cols, dtype, seed=13 + start, kind="mixed")
    l = rows * cols - start - 300
    o = oracle.writeback(x, rows, cols, [(start, l)])
    xs = to_dev(x)[start:start + l].clone()
    for pad in (0, 1, 2, 3):  # output buffer offset from an aligned allocation
        drb = torch.full((l + 8,), 0xA5, dtype=torch.uint8, device=DEV)
        dcb = torch.full((l + 8,), 0xA5, dtype=torch.uint8, device=DEV)
        dr, dc = drb[pad:pad + l], dcb[pad:pad + l]
        p = B.make_piece(rows, cols, start, xs, scale_row=to_dev_u8(o["scale_row"]),
                         scale_col=to_dev_u8(o["scale_col"]), data_row=dr, data_col=dc)
        # rows of whole 128-byte lines take the line-owned tiles, the others window stores
        assert B.mxfp8_query_path(p, 1) == (2 if cols % 128 == 0 and (pad - start) % 128 else 1)
        B.mxfp8_partial_cast(p)
        torch.cuda.synchronize()
        gr, gc = to_np(drb), to_np(dcb)
        assert not first_mismatch(gr[pad:pad + l], o["data_row"][start:start + l]), pad
        assert not first_mismatch(gc[pad:pad + l], o["data_col"][start:start + l]), pad
        assert (gr[:pad] == 0xA5).all() and (gr[pad + l:] == 0xA5).all()
        assert (gc[:pad] == 0xA5).all() and (gc[pad + l:] == 0xA5).all()


# ------------------------------------------------------------------ updates, pointers, determinism


def test_consecutive_updates_keep_pointers_and_give_second_update_bytes():
    rows, cols = 128, 256
    frags = [(0, 10000 + 17), (10017, 12000), (22017, rows * cols - 22017)]
    x1 = wl.random_matrix(rows, cols, "fp32", seed=1, kind="mixed")
    x2 = wl.random_matrix(rows, cols, "fp32", seed=2, kind="normal")
    wb = W.Writeback([W.WeightSpec(rows, cols, True)], torch.float32, DEV, frags, shared=False)
    st = wb.storage[0]
    ptrs = (st.data_row.data_ptr(), st.data_col.data_ptr(), st.scale_row.data_ptr(),
            st.scale_col.data_ptr())
    for x in (x1, x2):
        xd = to_dev(x)
        wb([xd[s:s + l] for s, l in frags])
    torch.cuda.synchronize()
    assert ptrs == (st.data_row.data_ptr(), st.data_col.data_ptr(), st.scale_row.data_ptr(),
                    st.scale_col.data_ptr())
    want = oracle.writeback(x2, rows, cols, frags)
    ar, ac = wb.combined.views(0)
    got = {"amax_row": to_np(ar), "amax_col": to_np(ac), "scale_row": to_np(st.scale_row),
           "scale_col": to_np(st.scale_col), "data_row": to_np(st.data_row),
           "data_col": to_np(st.data_col)}
    assert_same(got, want, rows, cols)


def test_repeated_runs_are_bitwise_identical():
    rows, cols = 256, 512
    x = wl.random_matrix(rows, cols, "bf16", seed=8, kind="mixed")
    frags = splits(rows * cols, 7, 3)
    outs = [run_matrix(x, rows, cols, frags, True, inputs="own", shared=True) for _ in range(3)]
    for o in outs[1:]:
        assert_same(o, outs[0], rows, cols)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_pieces_of_one_weight_in_one_call_share_an_amax_buffer(dtype):
    rows, cols = 256, 512
    x = wl.random_matrix(rows, cols, dtype, seed=21, kind="mixed")
    frags = splits(rows * cols, 16, 5)
    xd = to_dev(x)
    tdt = torch_dtype(x)
    ar = torch.zeros(rows, cols // 32, dtype=tdt, device=DEV)
    ac = torch.zeros(rows // 32, cols, dtype=tdt, device=DEV)
    # odd pieces read views of one buffer, even pieces their own copies (kept alive: a piece
    # holds raw pointers)
    inputs = [xd[s:s + l] if i % 2 else xd[s:s + l].clone() for i, (s, l) in enumerate(frags)]
    pieces = [B.make_piece(rows, cols, s, xi, amax_row=ar, amax_col=ac)
              for (s, l), xi in zip(frags, inputs)]
    B.mxfp8_partial_amax(pieces)
    torch.cuda.synchronize()
    want = oracle.new_buffers(rows, cols, oracle.dtype_of(x), True)
    oracle.partial_amax(x, rows, cols, 0, want["amax_row"], want["amax_col"])
    assert not first_mismatch(bits(to_np(ar)), bits(want["amax_row"]))
    assert not first_mismatch(bits(to_np(ac)), bits(want["amax_col"]))
