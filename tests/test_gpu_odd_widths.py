"""Odd widths at sizes that span many tiles.

Rows that are not whole 16-byte chunks (cols % 8 != 0 for BF16, cols % 4 != 0 for FP32) run
the element-wise kernels: a wave per 32-row x 64-column tile, many tiles per row and many
workgroups per launch.  The weights here are cut into four fragments whose boundaries fall
inside 32-value blocks (and one that cuts a tile's row-wise block between its two halves),
and the whole writeback in every mode, with one shared amax buffer and with one per fragment,
must give the oracle's bytes: amax, scales and both directions' data.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl

from gpu_util import DEV, assert_same, require_gpu, run_matrix

pytestmark = pytest.mark.gpu

MODES = [dict(), dict(fused=True), dict(single_pass=True)]
MODE_IDS = ["separate", "fused", "single_pass"]
SHAPES = [(1000, 4095), (333, 1001), (2049, 2047), (4100, 7), (96, 130)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def cuts(n, cols):
    """Four fragments: boundaries inside blocks, one of them 40 columns into a row (inside
    the second block of a 64-column tile)."""
    c = sorted({n // 4 + 17, n // 2 + 5, min(n - 1, 3 * (n // (4 * cols)) * cols + 40)})
    c = [0] + c + [n]
    return [(a, b - a) for a, b in zip(c[:-1], c[1:])]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_odd_width_writeback(rows, cols, dtype, mode):
    x = wl.random_matrix(rows, cols, dtype, seed=rows * 7 + cols, kind="mixed")
    n = rows * cols
    frags = cuts(n, cols)
    esize = 2 if dtype == "bf16" else 4
    xd = torch.empty(n, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=DEV)
    ar = torch.empty(rows, B.nblocks(cols), dtype=xd.dtype, device=DEV)
    assert B.mxfp8_query_path(B.make_piece(rows, cols, 0, xd, amax_row=ar), 0) == \
        (1 if cols % (16 // esize) == 0 else 0)
    for colwise in (True, False):
        want = oracle.writeback(x, rows, cols, frags, colwise)
        for shared in (True, False):
            got = run_matrix(x, rows, cols, frags, colwise, shared=shared, **mode)
            assert_same(got, want, rows, cols,
                        f"{rows}x{cols} {dtype} {mode} colwise={colwise} shared={shared}: ")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_odd_width_own_allocations_and_preround(dtype):
    """Fragments held in allocations of their own (BF16: input - start off a dword boundary)
    and, for FP32, the BF16 pre-rounding, on the element-wise kernels."""
    rows, cols = 517, 1023
    x = wl.random_matrix(rows, cols, dtype, seed=5, kind="mixed")
    n = rows * cols
    frags = cuts(n, cols)
    for pre in ((False, True) if dtype == "fp32" else (False,)):
        want = oracle.writeback(x, rows, cols, frags, True, preround=pre)
        for mode in MODES:
            got = run_matrix(x, rows, cols, frags, True, preround=pre, inputs="own",
                             shared=False, **mode)
            assert_same(got, want, rows, cols, f"{dtype} pre={pre} {mode}: ")
