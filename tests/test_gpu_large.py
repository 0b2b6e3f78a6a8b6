"""Parity at sizes past the 32-bit limits.

* A weight of more than 2^31 elements, cut into two fragments at element 2^31 + 17, so every
  offset of the second fragment and of its outputs needs 64-bit arithmetic.
* Tall, narrow weights whose calls need more than 2^20 workgroups: the library splits such
  a call into several launches (tiles numbered from a per-launch base), and the scales of
  more than 2^24 rows into launches of whole rows.

Inputs are drawn on the device (``workloads.device_matrix``).  The oracle checks sampled
32-row bands: once every fragment's amax is merged, a band's amax, scales and E4M3 bytes
depend only on the band's own values, so the oracle runs on the band as a weight of its own
(one fragment over all of it).  The bands sampled are the first and last, the ones around
the fragment cut, and the ones on each side of a launch split.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import DEV, bits, first_mismatch, require_gpu, to_np

pytestmark = pytest.mark.gpu

MODES = [dict(), dict(fused=True), dict(single_pass=True)]
MODE_IDS = ["separate", "fused", "single_pass"]
LAUNCH_GROUPS = 1 << 20   # workgroups per launch before a call is split
SCALE_ROWS = 1 << 24      # rows per scales launch (one 8-entry item per row when cols <= 256)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def check_band(wb, spec, x, b, label):
    rows, cols = spec.rows, spec.cols
    r0, r1 = 32 * b, min(32 * b + 32, rows)
    want = oracle.writeback(to_np(x[r0 * cols:r1 * cols]), r1 - r0, cols,
                            [(0, (r1 - r0) * cols)], spec.colwise)
    ar, ac = wb.combined.views(0)
    st = wb.storage[0]
    got = {"amax_row": ar[r0:r1], "scale_row": st.scale_row[r0:r1],
           "data_row": st.data_row[r0 * cols:r1 * cols]}
    if spec.colwise:
        got.update(amax_col=ac[b:b + 1], scale_col=st.scale_col[b:b + 1],
                   data_col=st.data_col[r0 * cols:r1 * cols])
    for k, g in got.items():
        msg = first_mismatch(bits(to_np(g)), bits(want[k]), (r1 - r0, cols))
        assert not msg, f"{label} band {b} {k}: {msg}"


def run_and_check(rows, cols, dtype, cut, mode, extra_bands, label, path=None):
    n = rows * cols
    print(f"\n{label}: {rows}x{cols} {dtype}, cut {cut}, {mode}", flush=True)
    x = wl.device_matrix(rows, cols, dtype, seed=rows % 1000 + cols, device=DEV)
    spec = W.WeightSpec(rows, cols, True)
    frags = [(0, cut), (cut, n - cut)]
    if path is not None:
        ar = torch.empty(rows, B.nblocks(cols), dtype=x.dtype, device=DEV)
        assert B.mxfp8_query_path(B.make_piece(rows, cols, cut, x[cut:], amax_row=ar), 0) == path
        del ar
    wb = W.Writeback([spec], x.dtype, DEV, frags, shared=False, **mode)
    wb([x[:cut], x[cut:]])
    torch.cuda.synchronize()
    last = (rows - 1) // 32
    bcut = (cut // cols) // 32
    bands = {0, last, bcut, max(0, bcut - 1), min(last, bcut + 1)}
    bands |= {b for b in extra_bands if 0 <= b <= last}
    for b in sorted(bands):
        check_band(wb, spec, x, b, label)
    del wb, x


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_weight_past_2_31_elements(dtype, mode):
    rows, cols = 40000, 53760                  # 2,150,400,000 elements
    assert rows * cols > 1 << 31
    first_past = ((1 << 31) // cols) // 32     # band holding element 2^31
    run_and_check(rows, cols, dtype, (1 << 31) + 17, mode, [first_past], "past 2^31", path=1)


# (dtype, cols, rows, path, tiles per workgroup): every shape needs more than 2^20
# workgroups, with a ragged last band of 5 rows
TALL = [("bf16", 8, (1 << 20) * 32 + 5, 1, 1),
        ("fp32", 4, (1 << 20) * 32 + 5, 1, 1),
        ("bf16", 7, (1 << 22) * 32 + 5, 0, 4)]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dtype,cols,rows,path,per_wg", TALL,
                         ids=[f"{d}-{c}cols-{'vector' if p else 'element'}"
                              for d, c, _, p, _ in TALL])
def test_calls_split_over_launches(dtype, cols, rows, path, per_wg, mode):
    n = rows * cols
    cut = n // 2 + 17
    bcut = (cut // cols) // 32
    split = LAUNCH_GROUPS * per_wg  # first tile of the second launch (a tile is a band here)
    assert -(-rows // 32) > split
    # The two fragments' pieces share launches, piece 1's tiles numbered after piece 0's
    # (rounded up to whole workgroups); the piece boundary sits at band bcut, or one band on
    # for the single-pass mode's whole-band pieces.  Bands around every candidate split, and
    # around each piece's first scales-launch boundary, are checked.
    align = lambda t: -(-t // per_wg) * per_wg
    cands = {split, bcut + split - align(bcut + 1), bcut + 1 + split - align(bcut),
             SCALE_ROWS // 32, (cut // cols + SCALE_ROWS) // 32}
    extra = {b + d for b in cands for d in (-2, -1, 0, 1, 2)}
    run_and_check(rows, cols, dtype, cut, mode, extra, "split launches", path=path)
