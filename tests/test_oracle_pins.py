"""Pins for the CPU oracle (oracle/mxfp8_oracle.c) against things other than itself.

* hand-worked blocks (tests/golden/hand_worked_blocks.json), in both block directions;
* nearest-code search over every E4M3 code for every finite BF16 value at every scale byte;
* an E8M0 search (the byte that puts amax in E4M3's top binade) at every power-of-two edge;
* torch's float8_e4m3fn and bfloat16 CPU conversions (library routines the oracle never calls);
* numpy block maxima;
* a pure-Python rational brute force of the whole path on tiny inputs;
* invariants: fragments + MAX-combine = full, shared buffer = K buffers + combine,
  transpose symmetry, power-of-two scaling, row-only = row half, pre-round = BF16 path.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce as bf
from mxfp8_block_scaled_partial_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_blocks.json")


# ------------------------------------------------------------------ helpers


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bf16_exact(values):
    """BF16 bit patterns of values that are exactly representable in BF16."""
    out = []
    for v in values:
        b = f32_bits(v)
        assert b & 0xFFFF == 0, f"{v} is not a BF16 value"
        out.append(b >> 16)
    return np.array(out, np.uint16)


def parse(v):
    return float.fromhex(v) if v.lstrip("-").startswith("0x") else float(v)


def amax_value(a, dtype):
    a = np.asarray(a)
    if dtype == oracle.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def run_full(x, rows, cols, colwise=True, preround=False):
    return oracle.writeback(x, rows, cols, [(0, rows * cols)], colwise, preround)


def same(a, b):
    for k in ("amax_row", "amax_col", "scale_row", "scale_col", "data_row", "data_col"):
        if a[k] is None or b[k] is None:
            assert a[k] is None and b[k] is None, k
        else:
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)


# ------------------------------------------------------------------ hand-worked blocks


@pytest.mark.parametrize("block", json.load(open(GOLDEN))["blocks"], ids=lambda b: b["name"][:1])
def test_hand_worked_blocks(block):
    vals = [parse(v) for v in block["values"]]
    n = len(vals)
    padded = vals + [0.0] * (32 - n)
    if block["dtype"] == "bf16":
        x = bf16_exact(padded)
        dt = oracle.BF16
    else:
        x = np.array(padded, np.float32)
        dt = oracle.FP32
    # as one 1x32 row block
    r = run_full(x, 1, 32, colwise=False)
    assert amax_value(r["amax_row"], dt)[0, 0] == np.float64(np.float32(parse(block["amax"])))
    assert r["scale_row"][0, 0] == block["scale"]
    assert list(r["data_row"][:n]) == block["data"]
    # as one 32x1 column block: the column direction must give the same bytes
    c = run_full(x, 32, 1, colwise=True)
    assert c["scale_col"][0, 0] == block["scale"]
    assert list(c["data_col"][:n]) == block["data"]


# ------------------------------------------------------------------ E8M0 scale rule


def test_scale_rule_matches_search_at_every_binade_edge():
    cases = []
    for k in range(-149, 128):
        p = np.float32(2.0 ** k)
        cases.append(p)
        below = np.nextafter(p, np.float32(0))
        if below > 0:
            cases.append(below)
        cases.append(np.nextafter(p, np.float32(np.inf)))
    cases += [np.float32(0.0), np.finfo(np.float32).max, np.float32(1.75), np.float32(448.0)]
    for a in cases:
        want = bf.e8m0_search(Fraction(float(a)))
        assert oracle.e8m0_scale(float(a)) == want, float(a)


# ------------------------------------------------------------------ E4M3 rounding


def _nearest_codes(v):
    """Vectorised nearest-code search (ties to even code) over the decoded E4M3 table;
    v >= 0 in float64.  Differences are exact for v >= 2^-12 (<= 24 significant bits
    against multiples of 2^-9 below 2^9); smaller v are nearer to 0 than to 2^-9."""
    codes = np.array([c for c, _ in bf.E4M3_TABLE])
    vals = np.array([float(f) for _, f in bf.E4M3_TABLE])
    order = np.argsort(vals)
    codes, vals = codes[order], vals[order]
    i = np.clip(np.searchsorted(vals, v), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = v - lo, hi - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[i] % 2 == 0))
    out = np.where(pick_hi, codes[i], codes[i - 1])
    return np.where(v >= vals[-1], codes[-1], out).astype(np.uint8)


def test_e4m3_exhaustive_bf16_codes_all_scale_bytes():
    """Every finite BF16 value at every scale byte 0..254 (16.5M cases), via the oracle's
    cast, against the nearest-code search."""
    bits = np.arange(0x10000, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    cols = bits.size                      # 65024, a multiple of 32
    scales = np.arange(255, dtype=np.uint8)
    rows = scales.size
    x = np.tile(bits, rows)
    scale_row = np.repeat(scales[:, None], cols // 32, axis=1).copy()
    data = np.zeros(rows * cols, np.uint8)
    oracle.partial_cast(x, rows, cols, 0, scale_row, data)
    w = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sign = (bits >> 15).astype(np.uint8) << 7
    for b in range(rows):
        v = np.abs(w) * 2.0 ** (127 - b)
        want = _nearest_codes(v) | sign
        got = data[b * cols:(b + 1) * cols]
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (b, hex(bits[bad[0]]), got[bad[0]], want[bad[0]])


def test_e4m3_matches_torch_float8_e4m3fn():
    """FP32 inputs at unit scale (byte 127) against torch's float8_e4m3fn conversion, after
    clamping to +-448 (torch turns overflow into NaN instead of saturating)."""
    g = np.random.Generator(np.random.PCG64(11))
    n = 1 << 16
    x = (g.standard_normal(n) * np.exp2(g.uniform(-16, 10, n))).astype(np.float32)
    # exact E4M3 midpoints and their neighbours
    mids = []
    for c in range(0x7E):
        a, b = float(bf._e4m3_decode(c)), float(bf._e4m3_decode(c + 1))
        m = np.float32((a + b) / 2)
        mids += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    mids = np.array(mids, np.float32)
    x = np.concatenate([x, mids, -mids, np.float32([0.0, -0.0, 448, 464, 480, 1e6, -1e6])])
    x = np.concatenate([x, np.zeros((-x.size) % 32, np.float32)])
    scale = np.full((1, x.size // 32), 127, np.uint8)
    data = np.zeros(x.size, np.uint8)
    oracle.partial_cast(x, 1, x.size, 0, scale, data)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    np.testing.assert_array_equal(data, ref.numpy())


def test_preround_matches_torch_bfloat16():
    g = np.random.Generator(np.random.PCG64(12))
    n = 40000
    x = (g.standard_normal(n) * np.exp2(g.uniform(-149, 127, n))).astype(np.float32)
    ties = (g.integers(1, 0x7F7F, 4000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32),
                        np.float32([0.0, -0.0, 1e-45, -1e-45, 3.3e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_to_bf16(float(v)) for v in x])
    np.testing.assert_array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


# ------------------------------------------------------------------ amax against numpy


@pytest.mark.parametrize("rows,cols,dtype", [(64, 96, "bf16"), (37, 45, "fp32"),
                                             (96, 33, "bf16"), (1, 70, "fp32")])
def test_amax_matches_numpy_block_max(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=rows * cols, kind="mixed")
    dt = oracle.dtype_of(x)
    xv = amax_value(x, dt).reshape(rows, cols) if dtype == "bf16" else x.astype(np.float64).reshape(rows, cols)
    nb, nr = oracle.nblocks(cols), oracle.nblocks(rows)
    # padded leading dimensions, sentinel-filled padding must stay untouched
    adt = oracle.amax_np_dtype(dt)
    ar = np.zeros((rows, nb + 3), adt)
    ac = np.zeros((nr, cols + 5), adt)
    ar[:, nb:] = 7
    ac[:, cols:] = 7
    oracle.partial_amax(x, rows, cols, 0, ar, ac)
    p = np.zeros((rows, nb * 32))
    p[:, :cols] = np.abs(xv)
    np.testing.assert_array_equal(amax_value(ar[:, :nb], dt), p.reshape(rows, nb, 32).max(axis=2))
    q = np.zeros((nr * 32, cols))
    q[:rows] = np.abs(xv)
    np.testing.assert_array_equal(amax_value(ac[:, :cols], dt), q.reshape(nr, 32, cols).max(axis=1))
    assert (ar[:, nb:] == 7).all() and (ac[:, cols:] == 7).all()


# ------------------------------------------------------------------ brute force, tiny inputs


@pytest.mark.parametrize("rows,cols,dtype,frags,colwise,pre", [
    (33, 40, "bf16", [(0, 33 * 40)], True, False),
    (33, 40, "bf16", [(17, 600), (617, 100)], True, False),
    (64, 32, "fp32", [(5, 1000), (1005, 1043)], True, False),
    (40, 64, "fp32", [(0, 1300), (1300, 1260)], False, True),
    (35, 70, "fp32", [(3, 2000)], True, True),
])
def test_oracle_matches_bruteforce(rows, cols, dtype, frags, colwise, pre):
    x = wl.random_matrix(rows, cols, dtype, seed=7 + rows, kind="mixed")
    o = oracle.writeback(x, rows, cols, frags, colwise, pre)
    b = bf.writeback(x, rows, cols, frags, colwise, pre)
    dt = oracle.dtype_of(x)
    for (r, j), a in b["amax_row"].items():
        assert Fraction(float(amax_value(o["amax_row"][r, j], dt))) == a
        assert o["scale_row"][r, j] == b["scale_row"][(r, j)]
    for (bb, c), a in b["amax_col"].items():
        assert Fraction(float(amax_value(o["amax_col"][bb, c], dt))) == a
        assert o["scale_col"][bb, c] == b["scale_col"][(bb, c)]
    np.testing.assert_array_equal(o["data_row"], b["data_row"])
    if colwise:
        np.testing.assert_array_equal(o["data_col"], b["data_col"])


@pytest.mark.parametrize("kind", ["tiny", "huge"])
def test_oracle_matches_bruteforce_range_ends(kind):
    rows, cols = 32, 64
    x = wl.random_matrix(rows, cols, "fp32", seed=3, kind=kind)
    o = run_full(x, rows, cols)
    b = bf.writeback(x, rows, cols, [(0, rows * cols)])
    np.testing.assert_array_equal(o["data_row"], b["data_row"])
    np.testing.assert_array_equal(o["data_col"], b["data_col"])
    for (r, j), s in b["scale_row"].items():
        assert o["scale_row"][r, j] == s


# ------------------------------------------------------------------ invariants


@pytest.mark.parametrize("rows,cols,dtype", [(64, 64, "bf16"), (40, 72, "fp32")])
def test_two_fragment_splits_equal_full(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=21, kind="mixed")
    n = rows * cols
    full = run_full(x, rows, cols)
    splits = sorted(set(list(range(0, n + 1, 37)) + [0, 1, 31, 32, 33, cols, cols + 1, n - 1, n]
                        + [32 * cols + k for k in (-1, 0, 1)]))
    for p in splits:
        got = oracle.writeback(x, rows, cols, [(0, p), (p, n - p)])
        same(got, full)


def test_random_k_splits_with_empty_fragments_equal_full():
    rows, cols = 96, 160
    x = wl.random_matrix(rows, cols, "bf16", seed=5, kind="mixed")
    n = rows * cols
    full = run_full(x, rows, cols)
    g = np.random.Generator(np.random.PCG64(99))
    for k in (3, 5, 8):
        cuts = np.sort(g.integers(0, n + 1, k - 1))
        cuts = np.concatenate([[0], cuts, [cuts[0]], [n]])  # one repeated cut: an empty fragment
        cuts.sort()
        frags = [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]
        same(oracle.writeback(x, rows, cols, frags), full)


def test_shared_buffer_accumulation_equals_k_buffers_and_combine():
    rows, cols = 64, 96
    x = wl.random_matrix(rows, cols, "fp32", seed=8, kind="mixed")
    frags = [(0, 1000), (1000, 17), (1017, 3000), (4017, rows * cols - 4017)]
    b = oracle.new_buffers(rows, cols, oracle.FP32, True)
    for s, l in frags:
        oracle.partial_amax(x[s:s + l], rows, cols, s, b["amax_row"], b["amax_col"])
    k = oracle.writeback(x, rows, cols, frags)
    np.testing.assert_array_equal(b["amax_row"], k["amax_row"])
    np.testing.assert_array_equal(b["amax_col"], k["amax_col"])


@pytest.mark.parametrize("rows,cols,dtype", [(96, 160, "bf16"), (64, 45, "fp32")])
def test_transpose_symmetry(rows, cols, dtype):
    x = wl.random_matrix(rows, cols, dtype, seed=4, kind="mixed")
    xt = np.ascontiguousarray(x.reshape(rows, cols).T).ravel()
    a = run_full(x, rows, cols)
    t = run_full(xt, cols, rows)
    np.testing.assert_array_equal(a["scale_col"], t["scale_row"].T)
    np.testing.assert_array_equal(a["amax_col"], t["amax_row"].T)
    np.testing.assert_array_equal(a["data_col"].reshape(rows, cols), t["data_row"].reshape(cols, rows).T)


def test_power_of_two_scaling_shifts_scales_only():
    rows, cols = 64, 64
    g = np.random.Generator(np.random.PCG64(3))
    x = (g.standard_normal(rows * cols) * 4.0).astype(np.float32)
    base = run_full(x, rows, cols)
    for k in (-30, -1, 1, 17, 60):
        y = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
        r = run_full(y, rows, cols)
        np.testing.assert_array_equal(r["data_row"], base["data_row"])
        np.testing.assert_array_equal(r["data_col"], base["data_col"])
        np.testing.assert_array_equal(r["scale_row"].astype(int), base["scale_row"].astype(int) + k)
        np.testing.assert_array_equal(r["scale_col"].astype(int), base["scale_col"].astype(int) + k)


def test_row_only_equals_row_half_of_bidirectional():
    rows, cols = 70, 96
    x = wl.random_matrix(rows, cols, "bf16", seed=6, kind="mixed")
    frags = [(17, 3000), (3017, 2000)]
    bi = oracle.writeback(x, rows, cols, frags, colwise=True)
    ro = oracle.writeback(x, rows, cols, frags, colwise=False)
    for k in ("amax_row", "scale_row", "data_row"):
        np.testing.assert_array_equal(bi[k], ro[k])
    assert ro["amax_col"] is None and ro["data_col"] is None


def test_preround_equals_bf16_path():
    rows, cols = 64, 96
    x = wl.random_matrix(rows, cols, "fp32", seed=10, kind="mixed")
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    frags = [(17, 3000), (3017, rows * cols - 3017)]
    p = oracle.writeback(x, rows, cols, frags, preround=True)
    b = oracle.writeback(xb, rows, cols, frags)
    for k in ("scale_row", "scale_col", "data_row", "data_col"):
        np.testing.assert_array_equal(p[k], b[k])
    np.testing.assert_array_equal(amax_value(p["amax_row"], oracle.FP32),
                                  amax_value(b["amax_row"], oracle.BF16))


def test_untouched_entries_keep_their_value_and_cut_blocks_merge():
    rows, cols = 64, 64
    x = wl.random_matrix(rows, cols, "fp32", seed=2, kind="normal")
    b = oracle.new_buffers(rows, cols, oracle.FP32, True)
    b["amax_row"][:] = 0.5
    b["amax_col"][:] = 0.5
    s, l = 100, 50                       # rows 1..2 only
    oracle.partial_amax(x[s:s + l], rows, cols, s, b["amax_row"], b["amax_col"])
    xv = np.abs(x.astype(np.float64))
    for r in range(rows):
        for j in range(2):
            idx = [r * cols + 32 * j + t for t in range(32) if s <= r * cols + 32 * j + t < s + l]
            want = max([0.5] + [xv[i] for i in idx])
            assert b["amax_row"][r, j] == np.float32(want)
    assert (b["amax_col"][1:] == 0.5).all()


@pytest.mark.parametrize("rows,cols,dtype,frag", [
    (96, 128, "bf16", (1000, 6000)),   # whole blocks in both directions, cuts inside blocks
    (70, 45, "fp32", (17, 70 * 45 - 17)),  # to the end: short last row blocks, short last band
    (64, 64, "fp32", (64 * 32, 64 * 32)),  # one whole band: every touched block is whole
    (40, 96, "bf16", (5, 20)),         # inside one row block: nothing is whole
])
def test_whole_blocks_are_set_and_cut_blocks_merge(rows, cols, dtype, frag):
    """Entries start at a sentinel above every |value|.  Blocks the fragment holds whole must
    come out as the numpy block max of the fragment's values (a merge would keep the
    sentinel); blocks a boundary cuts and untouched blocks must keep the sentinel (setting
    them would lower it)."""
    x = wl.random_matrix(rows, cols, dtype, seed=rows + cols, kind="mixed")
    dt = oracle.dtype_of(x)
    s, l = frag
    nb, nr = oracle.nblocks(cols), oracle.nblocks(rows)
    xv = amax_value(x, dt) if dtype == "bf16" else x.astype(np.float64)
    inside = np.zeros(rows * cols, bool)
    inside[s:s + l] = True
    # padded to whole blocks: padding is "inside" for the whole-block test and 0 for the max
    pad = ((0, nr * 32 - rows), (0, nb * 32 - cols))
    held = np.pad(inside.reshape(rows, cols), pad, constant_values=True)
    vals = np.pad(np.where(inside, np.abs(xv), 0.0).reshape(rows, cols), pad)
    row_whole = held.reshape(nr * 32, nb, 32).all(axis=2)[:rows]
    row_max = vals.reshape(nr * 32, nb, 32).max(axis=2)[:rows]
    col_whole = held.reshape(nr, 32, nb * 32).all(axis=1)[:, :cols]
    col_max = vals.reshape(nr, 32, nb * 32).max(axis=1)[:, :cols]
    big = 2.0 ** 100
    sent = np.float32(big) if dtype == "fp32" else wl.to_dtype(np.float32([big]), "bf16")[0]
    ar = np.full((rows, nb), sent)
    ac = np.full((nr, cols), sent)
    oracle.partial_amax(x[s:s + l], rows, cols, s, ar, ac)
    np.testing.assert_array_equal(amax_value(ar, dt), np.where(row_whole, row_max, big))
    np.testing.assert_array_equal(amax_value(ac, dt), np.where(col_whole, col_max, big))
    # the cases hold what they claim: whole blocks (except the last), cut blocks (except
    # the band-aligned one)
    assert row_whole.any() == (frag != (5, 20))
    assert (~row_whole & np.pad(inside.reshape(rows, cols), pad).reshape(
        nr * 32, nb, 32).any(axis=2)[:rows]).any() == (frag[0] % cols != 0)


def test_config_fragments_equal_full():
    m = wl.matrix_rowonly_fragments()
    full = oracle.writeback(m.data, m.rows, m.cols, m.runs["full"], colwise=False)
    frag = oracle.writeback(m.data, m.rows, m.cols, m.runs["fragments"], colwise=False)
    same(frag, full)
    assert any(l == 0 for _, l in m.runs["fragments"])


# ------------------------------------------------------------------ argument checks


def test_oracle_rejects_bad_arguments():
    x = np.zeros(64, np.float32)
    ar = np.zeros((2, 1), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.partial_amax(x, 2, 32, 1, ar)              # runs past the end
    with pytest.raises(oracle.OracleError):
        oracle.partial_amax(x, 2, 32, 0, np.zeros((2, 0), np.float32))  # ld too small
    with pytest.raises(oracle.OracleError):
        oracle.partial_cast(np.zeros(64, np.uint16), 2, 32, 0, np.zeros((2, 1), np.uint8),
                            np.zeros(64, np.uint8), preround=True)  # pre-round needs FP32
    with pytest.raises(oracle.OracleError):
        oracle.partial_amax(np.float32([np.inf] * 64), 2, 32, 0, ar)
    with pytest.raises(oracle.OracleError):
        oracle.partial_cast(x, 2, 32, 0, np.full((2, 1), 255, np.uint8), np.zeros(64, np.uint8))
