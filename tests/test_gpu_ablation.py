"""The runtime-guard ablation library (libmxfp8partial_guards.so, built by ``build.py
--ablation``): one amax and one cast kernel per dtype serve row-only and bidirectional calls,
their column-wise work selected at run time by the column-wise pointer, as in the kernels the
PR page ("Bidirectional kernel performance") measured before the compile-time
specialization.  Its timings are only meaningful if its bytes are the product's: the whole
writeback runs through it on the 160x96 workload (full and the fragment at offset 17), the
1024x1024 row-only fragments and the 16384x6144 quarter fragment at offset 17, row-only and
bidirectional, and is compared with the oracle byte for byte."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import build as hip_build
from mxfp8_block_scaled_partial_amd import workloads as wl

from gpu_util import assert_same, require_gpu, run_matrix

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture
def guards(monkeypatch):
    """Every binding call of the test goes to the runtime-guard library."""
    monkeypatch.setattr(B, "_lib", B.load_library(hip_build.GUARDS_LIB))
    yield
    torch.cuda.synchronize()


def check(m, frags, colwise, label, **kw):
    want = oracle.writeback(m.data, m.rows, m.cols, frags, colwise=colwise)
    got = run_matrix(m.data, m.rows, m.cols, frags, colwise, **kw)
    assert_same(got, want, m.rows, m.cols, label)


@pytest.mark.parametrize("colwise", [True, False], ids=["bidirectional", "row_only"])
def test_small_matrix_full_and_fragment(guards, colwise):
    m = wl.matrix_small()
    for run in ("full", "partial"):
        check(m, m.runs[run], colwise, f"160x96 {run} colwise={colwise}: ")
    # two fragments of the weight in their own allocations, per-fragment buffers + combine
    n = m.rows * m.cols
    check(m, [(0, 17 + 3000), (3017, n - 3017)], colwise, "160x96 two pieces: ",
          inputs="own", shared=False)


def test_rowonly_fragments_with_combine(guards):
    m = wl.matrix_rowonly_fragments()
    check(m, m.runs["fragments"], False, "1024x1024 fp32 row-only: ", shared=False)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("colwise", [True, False], ids=["bidirectional", "row_only"])
def test_large_quarter_fragment(guards, dtype, colwise):
    m = wl.matrix_large(dtype)
    print(f"\n16384x6144 {dtype} quarter colwise={colwise} (runtime-guard library)", flush=True)
    check(m, m.runs["partial"], colwise, f"16384x6144 {dtype} quarter colwise={colwise}: ")


def test_mixed_directions_in_one_call(guards):
    """A batch with row-only and bidirectional weights: the guarded library sends both kinds
    of piece through one kernel launch."""
    from mxfp8_block_scaled_partial_amd import writeback as W
    from gpu_util import DEV, to_dev, to_np

    specs = [W.WeightSpec(64, 256, True), W.WeightSpec(96, 128, False),
             W.WeightSpec(40, 384, True)]
    parts = [wl.random_matrix(sp.rows, sp.cols, "bf16", seed=60 + i, kind="mixed")
             for i, sp in enumerate(specs)]
    flat = np.concatenate(parts)
    total = flat.size
    frags = [(0, 10000 + 5), (10005, 12000), (22005, total - 22005)]
    wb = W.Writeback(specs, torch.bfloat16, DEV, frags, shared=True)
    x = to_dev(flat)
    wb([x[s:s + l] for s, l in frags])
    torch.cuda.synchronize()
    o = 0
    for i, sp in enumerate(specs):
        pieces = []
        for fs, fl in frags:
            lo, hi = max(fs, o), min(fs + fl, o + sp.numel)
            if lo < hi:
                pieces.append((lo - o, hi - lo))
        want = oracle.writeback(flat[o:o + sp.numel], sp.rows, sp.cols, pieces, sp.colwise)
        ar, ac = wb.combined.views(i)
        st = wb.storage[i]
        got = {"amax_row": to_np(ar), "amax_col": to_np(ac) if sp.colwise else None,
               "scale_row": to_np(st.scale_row),
               "scale_col": to_np(st.scale_col) if sp.colwise else None,
               "data_row": to_np(st.data_row),
               "data_col": to_np(st.data_col) if sp.colwise else None}
        assert_same(got, want, sp.rows, sp.cols, f"weight {i}: ")
        o += sp.numel
