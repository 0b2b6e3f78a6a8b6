"""The writeback captured once in a HIP graph and replayed: every replay must give the
oracle's bytes for the input values current at replay time.  Between replays the test does
eager work of its own (it overwrites the inputs and clobbers the outputs), and each replay is
checked, for the separate-scales, fused and single-pass plans."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import DEV, assert_same, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("mode", ["separate", "fused", "single_pass"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_graph_replays_match_oracle(mode, dtype):
    rows, cols = 320, 1024
    n = rows * cols
    band = 32 * cols
    frags = [(0, band + 17), (band + 17, 3 * band), (4 * band + 17, n - 4 * band - 17)]
    xs = [wl.random_matrix(rows, cols, dtype, seed=s, kind="mixed") for s in (1, 2, 3)]
    x_dev = to_dev(xs[0])
    wb = W.Writeback([W.WeightSpec(rows, cols, True)], x_dev.dtype, DEV, frags, shared=False,
                     fused=mode == "fused", single_pass=mode == "single_pass")
    plan = wb.plan([x_dev[s:s + l] for s, l in frags])
    plan.run()  # eager first
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run()
    st = wb.storage[0]
    for rep, x in enumerate(xs + xs[:1]):
        x_dev.copy_(to_dev(x))                     # new master values, written eagerly
        for t in (st.data_row, st.data_col, st.scale_row, st.scale_col):
            t.fill_(0x5A)                          # stale outputs the replay must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.writeback(x, rows, cols, frags, True)
        ar, ac = wb.combined.views(0)
        got = {"amax_row": to_np(ar), "amax_col": to_np(ac),
               "scale_row": to_np(st.scale_row), "scale_col": to_np(st.scale_col),
               "data_row": to_np(st.data_row), "data_col": to_np(st.data_col)}
        # bytes outside every fragment are not the writeback's: compare inside them only
        gap = np.ones(n, bool)
        for s, l in frags:
            gap[s:s + l] = False
        for k in ("data_row", "data_col"):
            got[k] = np.where(gap, 0, got[k])
        assert_same(got, want, rows, cols, f"replay {rep}: ")
    del g
