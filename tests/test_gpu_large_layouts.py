"""The benchmark's weight (16384 x 6144, BF16 and FP32, four fragments cut inside 32-value
blocks) in the layouts the large, residency-capped launches see least often: fragments held in
allocations of their own (for BF16, input - start 2 bytes off a dword boundary: every chunk
load takes the 2-byte realign) and FSDP fragment-sized outputs (data pointers at 3 mod 4 from
the element index: every tile takes the window stores).  Every writeback mode, one packed
buffer per fragment, compared with the oracle byte for byte over the whole weight."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import DEV, assert_same, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

MODES = [dict(), dict(fused=True), dict(single_pass=True)]
MODE_IDS = ["separate", "fused", "single_pass"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


_cache = {}


def weight_and_oracle(dtype):
    if dtype not in _cache:
        m = wl.matrix_large(dtype)
        n = m.rows * m.cols
        cuts = [0, n // 4 + 17, n // 2 + 17, 3 * n // 4 + 17, n]
        frags = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
        _cache.clear()
        _cache[dtype] = (m, frags, oracle.writeback(m.data, m.rows, m.cols, frags, True))
    return _cache[dtype]


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("fragment_outputs", [False, True], ids=["in_place", "fragment_outputs"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_large_own_inputs_and_fragment_outputs(dtype, fragment_outputs, mode):
    m, frags, want = weight_and_oracle(dtype)
    print(f"\n16384x6144 {dtype} fragment_outputs={fragment_outputs} {mode}", flush=True)
    x = to_dev(m.data)
    spec = W.WeightSpec(m.rows, m.cols, True)
    wb = W.Writeback([spec], x.dtype, DEV, frags, shared=False,
                     fragment_outputs=fragment_outputs, **mode)
    own = [x[s:s + l].clone() for s, l in frags]  # each fragment in an allocation of its own
    del x
    wb(own)
    torch.cuda.synchronize()
    ar, ac = wb.combined.views(0)
    st = wb.storage[0]
    got = {"amax_row": to_np(ar), "amax_col": to_np(ac), "scale_row": to_np(st.scale_row),
           "scale_col": to_np(st.scale_col)}
    if fragment_outputs:
        got["data_row"] = np.concatenate([to_np(fo.data_row) for fo in wb.fragment_outputs])
        got["data_col"] = np.concatenate([to_np(fo.data_col) for fo in wb.fragment_outputs])
    else:
        got["data_row"], got["data_col"] = to_np(st.data_row), to_np(st.data_col)
    assert_same(got, want, m.rows, m.cols, f"{dtype} fo={fragment_outputs} {mode}: ")
