"""mxfp8_time_next_call: the runtime stamps the two events at the timed call's first kernel
start and last kernel end.  A timed call writes the same bytes as an untimed one (and as the
oracle), its kernel time lies inside the interval of markers recorded around it on the
stream, a call of two kernels is covered from the first's start to the second's end, and the
events time one call only."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl

from gpu_util import DEV, require_gpu, to_dev, to_np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from bench import TimingEvent  # noqa: E402  (timing-only HIP events on torch's stream)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cast_pieces(m, frags, colwise_flags):
    """One cast piece per (fragment, direction flag) of matrix m, with scales from the oracle."""
    rows, cols = m.rows, m.cols
    want = oracle.writeback(m.data, rows, cols, [(0, rows * cols)], colwise=True)
    x = to_dev(m.data)
    sr = torch.from_numpy(want["scale_row"]).to(DEV)
    sc = torch.from_numpy(want["scale_col"]).to(DEV)
    outs, pieces = [], []
    for (s, l), colwise in zip(frags, colwise_flags):
        dr = torch.zeros(l, dtype=torch.uint8, device=DEV)
        dc = torch.zeros(l, dtype=torch.uint8, device=DEV) if colwise else None
        pieces.append(B.make_piece(rows, cols, s, x[s:s + l], scale_row=sr, scale_col=sc,
                                   data_row=dr, data_col=dc))
        outs.append((s, l, dr, dc))
    return want, x, outs, pieces


def test_timed_call_writes_the_same_bytes_and_sits_inside_the_markers():
    m = wl.matrix_square("bf16", rows=4096, cols=4096)
    n = m.rows * m.cols
    want, x, outs, pieces = _cast_pieces(m, [(17, n // 2)], [True])
    e0, e1, k0, k1 = TimingEvent(), TimingEvent(), TimingEvent(), TimingEvent()
    e0.record()
    B.mxfp8_time_next_call(k0.ev.value, k1.ev.value)
    B.mxfp8_partial_cast(pieces)
    e1.record()
    torch.cuda.synchronize()
    kernel_ms, bracket_ms = k0.elapsed_time(k1), e0.elapsed_time(e1)
    assert 0 < kernel_ms <= bracket_ms
    s, l, dr, dc = outs[0]
    assert np.array_equal(to_np(dr), want["data_row"][s:s + l])
    assert np.array_equal(to_np(dc), want["data_col"][s:s + l])
    # the events timed one call: an untimed call after it leaves them as they were
    B.mxfp8_partial_cast(pieces)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms


def test_a_call_of_two_kernels_is_timed_from_first_start_to_last_end():
    """Row-only and bidirectional pieces of a large call (4096 tiles, well above the size
    under which a call holding both directions goes out as one launch) go out as two launches;
    the interval covers both.  Each launch timed alone also holds its own ramp-up and drain,
    so the pair takes somewhat less than the sum."""
    m = wl.matrix_square("fp32", rows=8192, cols=4096)
    n = m.rows * m.cols
    frags = [(0, n // 2), (n // 2, n // 2)]
    want, x, outs, pieces = _cast_pieces(m, frags, [True, False])
    def timed(ps):  # the fastest of three timed calls, after a warm-up call
        B.mxfp8_partial_cast(ps)
        best = None
        for _ in range(3):
            k0, k1 = TimingEvent(), TimingEvent()
            B.mxfp8_time_next_call(k0.ev.value, k1.ev.value)
            B.mxfp8_partial_cast(ps)
            torch.cuda.synchronize()
            ms = k0.elapsed_time(k1)
            best = ms if best is None else min(best, ms)
        return best

    singles = [timed([p]) for p in pieces]  # each launch alone
    both = timed(pieces)
    assert both > max(singles) and both >= 0.8 * sum(singles), (both, singles)
    for (s, l, dr, dc) in outs:
        assert np.array_equal(to_np(dr), want["data_row"][s:s + l])
        if dc is not None:
            assert np.array_equal(to_np(dc), want["data_col"][s:s + l])
