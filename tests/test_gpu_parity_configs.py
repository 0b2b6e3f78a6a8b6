"""GPU parity on the five workloads: the HIP path, called through the C ABI, must equal the
oracle byte for byte (amax bit patterns, E8M0 scales, E4M3 data) on every run, at full size.

Workloads (mxfp8_block_scaled_partial_amd.workloads): 160x96 BF16; 1024x1024 FP32 row-only in
4 fragments (one empty, cuts inside blocks); 4096x4096 BF16 / FP32 (+ BF16 pre-rounding);
16384x6144 BF16 / FP32; a transformer layer's four weights in one BF16 buffer cut into 8
fragments.  Fragment inputs are either views of one flat master buffer or separate
allocations (a rank's own shard), which exercises the vector and the element-wise kernels.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import DEV, assert_same, require_gpu, run_matrix, to_dev, to_np, fragment_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_cache = {}


def cached(key, fn):
    if key not in _cache:
        _cache[key] = fn()
    return _cache[key]


# ------------------------------------------------------------------ 160x96 BF16


@pytest.mark.parametrize("run", ["full", "partial"])
@pytest.mark.parametrize("inputs", ["views", "own"])
def test_small_bf16(run, inputs):
    m = cached("small", wl.matrix_small)
    frags = m.runs[run]
    want = oracle.writeback(m.data, m.rows, m.cols, frags, True)
    got = run_matrix(m.data, m.rows, m.cols, frags, True, inputs=inputs)
    assert_same(got, want, m.rows, m.cols)


# ------------------------------------------------------------------ 1024x1024 FP32 row-only


@pytest.mark.parametrize("inputs", ["views", "own"])
@pytest.mark.parametrize("shared", [True, False])
def test_rowonly_fragments_fp32(inputs, shared):
    m = cached("rowonly", wl.matrix_rowonly_fragments)
    frags = m.runs["fragments"]
    assert any(l == 0 for _, l in frags)
    want = cached("rowonly-oracle",
                  lambda: oracle.writeback(m.data, m.rows, m.cols, frags, colwise=False))
    full = cached("rowonly-full", lambda: oracle.writeback(m.data, m.rows, m.cols,
                                                           m.runs["full"], colwise=False))
    got = run_matrix(m.data, m.rows, m.cols, frags, False, inputs=inputs, shared=shared)
    assert_same(got, want, m.rows, m.cols)
    # four fragments + MAX-combine give the bytes of a single full cast
    assert_same(got, full, m.rows, m.cols, "vs full: ")


# ------------------------------------------------------------------ 4096x4096


CASES_SQ = [("bf16", "full", False), ("bf16", "partial", False), ("fp32", "full", False),
            ("fp32", "partial", False), ("fp32", "full", True), ("fp32", "partial", True)]


@pytest.mark.parametrize("dtype,run,pre", CASES_SQ)
def test_square_4096(dtype, run, pre):
    m = cached(f"sq-{dtype}", lambda: wl.matrix_square(dtype))
    frags = m.runs[run]
    want = oracle.writeback(m.data, m.rows, m.cols, frags, True, pre)
    got = run_matrix(m.data, m.rows, m.cols, frags, True, pre, inputs="views")
    assert_same(got, want, m.rows, m.cols)
    if run == "partial":
        got = run_matrix(m.data, m.rows, m.cols, frags, True, pre, inputs="own")
        assert_same(got, want, m.rows, m.cols, "own buffer: ")


# ------------------------------------------------------------------ 16384x6144 (full size)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("run", ["full", "partial"])
def test_large_16384x6144(dtype, run):
    m = cached(f"large-{dtype}", lambda: wl.matrix_large(dtype))
    frags = m.runs[run]
    want = oracle.writeback(m.data, m.rows, m.cols, frags, True)
    got = run_matrix(m.data, m.rows, m.cols, frags, True, inputs="views")
    assert_same(got, want, m.rows, m.cols)
    # the launch configuration the benchmark times: one flat master, 4 fragments with
    # boundaries inside blocks, one packed amax per fragment, MAX-combined
    if run == "full":
        n = m.rows * m.cols
        cuts = [0, n // 4 + 17, n // 2 + 17, 3 * n // 4 + 17, n]
        four = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
        got4 = run_matrix(m.data, m.rows, m.cols, four, True, inputs="views", shared=False)
        assert_same(got4, want, m.rows, m.cols, "4 fragments: ")


# ------------------------------------------------------------------ transformer-layer batch


def _layer_oracle(batch):
    out = []
    for i, (name, r, c, colwise) in enumerate(batch.tensors):
        o = batch.offsets[i]
        pieces = []
        for fs, fl in batch.fragments:
            lo, hi = max(fs, o), min(fs + fl, o + r * c)
            if lo < hi:
                pieces.append((lo - o, hi - lo))
        out.append(oracle.writeback(batch.data[o:o + r * c], r, c, pieces, colwise))
    return out


@pytest.mark.parametrize("shared", [True, False])
def test_layer_batch_8_fragments(shared):
    batch = cached("layer", wl.layer_batch)
    want = cached("layer-oracle", lambda: _layer_oracle(batch))
    specs = [W.WeightSpec(r, c, colwise) for (_, r, c, colwise) in batch.tensors]
    x_dev = to_dev(batch.data)
    wb = W.Writeback(specs, torch.bfloat16, DEV, batch.fragments, shared=shared)
    plan = wb.plan(fragment_inputs(x_dev, batch.fragments, "views"))
    plan.run()
    torch.cuda.synchronize()
    assert plan.n_amax > len(batch.fragments)  # some fragments span two weights
    for i, (name, r, c, colwise) in enumerate(batch.tensors):
        ar, ac = wb.combined.views(i)
        st = wb.storage[i]
        got = {"amax_row": to_np(ar), "amax_col": to_np(ac) if colwise else None,
               "scale_row": to_np(st.scale_row),
               "scale_col": to_np(st.scale_col) if colwise else None,
               "data_row": to_np(st.data_row), "data_col": to_np(st.data_col) if colwise else None}
        assert_same(got, want[i], r, c, f"{name}: ")
    # the packed buffer holds exactly the present directions
    assert wb.combined.numel == sum(s.amax_row_entries + s.amax_col_entries for s in specs)
