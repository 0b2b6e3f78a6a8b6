"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path
through the C ABI (binding + batch helper), and compare with the oracle byte for byte."""
from __future__ import annotations

import numpy as np
import torch

from mxfp8_block_scaled_partial_amd import binding as B
from mxfp8_block_scaled_partial_amd import writeback as W

DEV = torch.device("cuda:0")


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()  # raises LibraryNotBuilt loudly when the HIP library is missing


def to_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 arrays are BF16 bit patterns; float32 arrays stay float32."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    raise ValueError(a.dtype)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    """Bit patterns of an amax array for exact comparison (float32 -> uint32)."""
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def torch_dtype(a: np.ndarray):
    return torch.bfloat16 if a.dtype == np.uint16 else torch.float32


def fragment_inputs(x_dev: torch.Tensor, fragments, mode: str):
    """Fragment tensors: ``views`` of the full flat buffer (input - start stays aligned) or
    ``own`` allocations, one per fragment, as a rank holding only its shard would have."""
    out = []
    for s, l in fragments:
        v = x_dev[s:s + l]
        out.append(v if mode == "views" else v.clone())
    return out


def run_matrix(x: np.ndarray, rows: int, cols: int, fragments, colwise=True, preround=False,
               inputs="views", shared=True, fused=False, single_pass=False):
    """The whole path on the GPU for one matrix held as ``fragments``; numpy results."""
    x_dev = to_dev(x)
    wb = W.Writeback([W.WeightSpec(rows, cols, colwise)], torch_dtype(x), DEV, fragments,
                     shared=shared, preround=preround, fused=fused, single_pass=single_pass)
    wb(fragment_inputs(x_dev, fragments, inputs))
    torch.cuda.synchronize()
    ar, ac = wb.combined.views(0)
    st = wb.storage[0]
    return {"amax_row": to_np(ar), "amax_col": to_np(ac) if colwise else None,
            "scale_row": to_np(st.scale_row), "scale_col": to_np(st.scale_col) if colwise else None,
            "data_row": to_np(st.data_row), "data_col": to_np(st.data_col) if colwise else None,
            "wb": wb}


def first_mismatch(got: np.ndarray, want: np.ndarray, shape=None) -> str:
    bad = np.nonzero(got.ravel() != want.ravel())[0]
    if bad.size == 0:
        return ""
    i = int(bad[0])
    where = f"flat {i}"
    if shape is not None:
        where += f" (row {i // shape[1]}, col {i % shape[1]})"
    return f"{bad.size} mismatches; first at {where}: got {got.ravel()[i]:#x}, want {want.ravel()[i]:#x}"


def assert_same(got: dict, want: dict, rows: int, cols: int, label: str = ""):
    for k in ("amax_row", "amax_col", "scale_row", "scale_col", "data_row", "data_col"):
        g, w = got.get(k), want.get(k)
        if w is None:
            assert g is None, f"{label}{k}: expected absent"
            continue
        g, w = bits(g), bits(w)
        assert g.shape == w.shape, f"{label}{k}: shape {g.shape} vs {w.shape}"
        shape = (rows, cols) if k.startswith("data") else w.shape
        msg = first_mismatch(g, w, shape)
        assert not msg, f"{label}{k}: {msg}"
