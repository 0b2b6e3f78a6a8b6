"""The batch helper's two update interfaces: in place into full-size MXFP8 storage, and
FSDP-style fragment outputs (each fragment's E4M3 bytes in buffers of the fragment's own
size).  Both must give the oracle's bytes, for batches of many weights (mixed row-only and
bidirectional, ragged shapes) cut into fragments that span weight boundaries, in every plan
mode (separate scales, fused, single pass; shared or per-fragment amax), with storage pointers
that stay put across consecutive updates."""
import numpy as np
import pytest
import torch

import oracle
from mxfp8_block_scaled_partial_amd import workloads as wl
from mxfp8_block_scaled_partial_amd import writeback as W

from gpu_util import DEV, bits, first_mismatch, require_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu

MODES = [dict(), dict(fused=True), dict(single_pass=True)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def batch(seed, dtype):
    """12 weights of assorted shapes (some with cols % 32 != 0) in one flat buffer."""
    shapes = [(64, 96, True), (37, 45, False), (100, 64, True), (33, 40, True), (128, 256, False),
              (70, 1, True), (1, 70, False), (96, 33, True), (256, 128, True), (65, 96, False),
              (31, 4128, True), (200, 64, True)]
    specs = [W.WeightSpec(r, c, cw) for r, c, cw in shapes]
    parts = [wl.random_matrix(r, c, dtype, seed=seed + i, kind="mixed")
             for i, (r, c, _) in enumerate(shapes)]
    return specs, np.concatenate(parts)


def fragments_of(total, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cuts = np.sort(g.integers(0, total + 1, k - 1))
    cuts = np.concatenate([[0], cuts, [total]])
    return [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]


def expected(specs, flat, frags):
    """The oracle per weight over the pieces the fragments give it."""
    out, o = [], 0
    for sp in specs:
        pieces = []
        for fs, fl in frags:
            lo, hi = max(fs, o), min(fs + fl, o + sp.numel)
            if lo < hi:
                pieces.append((lo - o, hi - lo))
        out.append(oracle.writeback(flat[o:o + sp.numel], sp.rows, sp.cols, pieces, sp.colwise))
        o += sp.numel
    return out


def check(wb, specs, frags, want, label):
    offs = np.cumsum([0] + [sp.numel for sp in specs])
    for i, sp in enumerate(specs):
        ar, ac = wb.combined.views(i)
        st = wb.storage[i]
        for k, g in (("amax_row", ar), ("amax_col", ac), ("scale_row", st.scale_row),
                     ("scale_col", st.scale_col if sp.colwise else None)):
            if want[i][k] is None:
                continue
            msg = first_mismatch(bits(to_np(g)), bits(want[i][k]))
            assert not msg, f"{label} weight {i} {k}: {msg}"
        if wb.fragment_outputs is None:
            msg = first_mismatch(to_np(st.data_row), want[i]["data_row"], (sp.rows, sp.cols))
            assert not msg, f"{label} weight {i} data_row: {msg}"
            if sp.colwise:
                msg = first_mismatch(to_np(st.data_col), want[i]["data_col"], (sp.rows, sp.cols))
                assert not msg, f"{label} weight {i} data_col: {msg}"
    if wb.fragment_outputs is None:
        return
    for f, (fs, fl) in enumerate(frags):
        fo = wb.fragment_outputs[f]
        got_r, got_c = to_np(fo.data_row), to_np(fo.data_col)
        want_r = np.zeros(fl, np.uint8)
        want_c = np.zeros(got_c.size, np.uint8)
        for i, sp in enumerate(specs):
            lo, hi = max(fs, offs[i]), min(fs + fl, offs[i + 1])
            if lo >= hi:
                continue
            want_r[lo - fs:hi - fs] = want[i]["data_row"][lo - offs[i]:hi - offs[i]]
            if sp.colwise:
                want_c[lo - fs:hi - fs] = want[i]["data_col"][lo - offs[i]:hi - offs[i]]
        assert not first_mismatch(got_r, want_r), f"{label} fragment {f} data_row"
        assert not first_mismatch(got_c, want_c), f"{label} fragment {f} data_col"


@pytest.mark.parametrize("mode", MODES, ids=["separate", "fused", "single_pass"])
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("fragment_outputs", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_weights_both_interfaces(mode, shared, fragment_outputs, dtype):
    specs, flat = batch(10, dtype)
    frags = fragments_of(flat.size, 5, 3)
    want = expected(specs, flat, frags)
    x = to_dev(flat)
    wb = W.Writeback(specs, x.dtype, DEV, frags, shared=shared,
                     fragment_outputs=fragment_outputs, **mode)
    wb([x[s:s + l].clone() for s, l in frags])
    torch.cuda.synchronize()
    check(wb, specs, frags, want, f"{mode} shared={shared} fo={fragment_outputs}: ")


@pytest.mark.parametrize("mode", MODES, ids=["separate", "fused", "single_pass"])
def test_consecutive_updates_keep_fragment_output_pointers(mode):
    specs, flat1 = batch(20, "bf16")
    _, flat2 = batch(40, "bf16")
    frags = fragments_of(flat1.size, 4, 9)
    wb = W.Writeback(specs, torch.bfloat16, DEV, frags, shared=False, fragment_outputs=True,
                     **mode)
    ptrs = [(fo.data_row.data_ptr(), fo.data_col.data_ptr()) for fo in wb.fragment_outputs]
    ptrs += [(st.scale_row.data_ptr(), st.scale_col.data_ptr()) for st in wb.storage]
    for flat in (flat1, flat2):
        x = to_dev(flat)
        wb([x[s:s + l] for s, l in frags])
    torch.cuda.synchronize()
    now = [(fo.data_row.data_ptr(), fo.data_col.data_ptr()) for fo in wb.fragment_outputs]
    now += [(st.scale_row.data_ptr(), st.scale_col.data_ptr()) for st in wb.storage]
    assert now == ptrs
    check(wb, specs, frags, expected(specs, flat2, frags), f"{mode} second update: ")


def test_layer_batch_fragment_outputs():
    b = wl.layer_batch()
    specs = [W.WeightSpec(r, c, colwise) for (_, r, c, colwise) in b.tensors]
    want = expected(specs, b.data, b.fragments)
    x = to_dev(b.data)
    wb = W.Writeback(specs, torch.bfloat16, DEV, b.fragments, shared=False,
                     fragment_outputs=True, single_pass=True)
    wb([x[s:s + l] for s, l in b.fragments])
    torch.cuda.synchronize()
    check(wb, specs, b.fragments, want, "layer batch: ")


def test_cast_master_fragments_helper():
    specs, flat = batch(60, "bf16")
    frags = fragments_of(flat.size, 3, 11)
    x = to_dev(flat)
    wb = W.cast_master_fragments([(s, x[s:s + l].clone()) for s, l in frags], specs,
                                 shared=False, fused=True)
    torch.cuda.synchronize()
    check(wb, specs, frags, expected(specs, flat, frags), "helper: ")
