"""Seeded synthetic inputs for the MXFP8 master-weight writeback.

This module generates inputs only; it holds none of the method's arithmetic, and both the
GPU path's tests / benchmark and the CPU oracle's tests draw from it.  Values are drawn
with ``numpy.random.Generator(PCG64(seed))`` in float64, rounded to FP32 by numpy, and to
BF16 (round-to-nearest-even, via torch's CPU conversion) for BF16 workloads.  BF16 arrays
are returned as ``uint16`` bit patterns, FP32 arrays as ``float32``; every array is the
row-major flattening of the weight.

The shapes are the matrices timed in "Support row-only MXFP8 distributed master-weight
casts" (section "Bidirectional kernel performance": 160x96, 1024x1024, 4096x4096 and
16384x6144 in BF16 and FP32, full input and a quarter fragment starting at offset 17) plus a
transformer-layer batch (4096x12288 QKV, 4096x4096 output projection, 4096x14336 up and
14336x4096 down projections) split into equal fragments, as several ranks would hold it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_dtype(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> FP32 (numpy, RNE) -> optionally BF16 bit patterns (torch, RNE)."""
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == FP32:
        return x32
    import torch

    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Matrix:
    """One 2-D weight, flattened, with the fragment runs a test or benchmark applies."""
    name: str
    rows: int
    cols: int
    dtype: str
    data: np.ndarray                      # flat, rows*cols elements
    colwise: bool = True
    runs: dict = field(default_factory=dict)   # run name -> list of (start, length)
    preround_runs: tuple = ()             # run names also done with BF16 pre-rounding


@dataclass
class Batch:
    """Several weights laid end to end in one flat buffer, cut into equal fragments."""
    name: str
    tensors: list                         # [(name, rows, cols, colwise)]
    offsets: list                         # flat offset of each tensor
    dtype: str
    data: np.ndarray
    fragments: list                       # [(start, length)] over the flat buffer


# ------------------------------------------------------------------ the five workloads


def matrix_small(seed: int = 0) -> Matrix:
    """160x96 BF16: N(0,1) times a per-row magnitude 2^U, U ~ Uniform[-10, 4]; the 32x32
    tile at rows 32-63, cols 32-63 is zero.  Runs: full, and the fragment [17, 17+3840)."""
    rows, cols = 160, 96
    g = _rng(seed)
    x = g.standard_normal((rows, cols)) * np.exp2(g.uniform(-10.0, 4.0, size=(rows, 1)))
    x[32:64, 32:64] = 0.0
    return Matrix("160x96-bf16", rows, cols, BF16, to_dtype(x.ravel(), BF16), True,
                  {"full": [(0, rows * cols)], "partial": [(17, rows * cols // 4)]})


def matrix_rowonly_fragments(seed: int = 1) -> Matrix:
    """1024x1024 FP32, row-wise only: N(0, 0.02) with 0.1% of the entries (chosen without
    replacement) multiplied by 1000.  The flat buffer is cut into 4 contiguous fragments at
    offsets 0, 262161, 262161, 786447, 1048576: the second fragment is empty and the other
    boundaries fall inside 32-value blocks."""
    rows, cols = 1024, 1024
    g = _rng(seed)
    x = g.normal(0.0, 0.02, size=rows * cols)
    idx = g.choice(rows * cols, size=(rows * cols) // 1000, replace=False)
    x[idx] *= 1000.0
    cuts = [0, 262161, 262161, 786447, rows * cols]
    frags = [(cuts[i], cuts[i + 1] - cuts[i]) for i in range(4)]
    return Matrix("1024x1024-fp32-rowonly", rows, cols, FP32, to_dtype(x, FP32), False,
                  {"fragments": frags, "full": [(0, rows * cols)]})


def matrix_square(dtype: str, seed: int = 2, rows: int = 4096, cols: int = 4096) -> Matrix:
    """4096x4096: N(0,1) times a per-column magnitude 2^U, U ~ Uniform[-8, 8].  Runs: full,
    and the quarter fragment [17, 17 + N/4); FP32 also with BF16 pre-rounding."""
    g = _rng(seed)
    x = g.standard_normal((rows, cols)) * np.exp2(g.uniform(-8.0, 8.0, size=(1, cols)))
    n = rows * cols
    pre = ("full", "partial") if dtype == FP32 else ()
    return Matrix(f"{rows}x{cols}-{dtype}", rows, cols, dtype, to_dtype(x.ravel(), dtype), True,
                  {"full": [(0, n)], "partial": [(17, n // 4)]}, pre)


def matrix_large(dtype: str, seed: int = 3, rows: int = 16384, cols: int = 6144,
                 n_zero_tiles: int = 16) -> Matrix:
    """16384x6144: N(0, 0.02) weights, a 1e-4 fraction of entries replaced by +-U[100, 448]
    spikes, then 16 randomly placed, 32-aligned 32x32 tiles set to zero.  Runs: full, and
    the quarter fragment [17, 17 + N/4)."""
    g = _rng(seed)
    n = rows * cols
    x = g.normal(0.0, 0.02, size=n)
    k = int(n * 1e-4)
    idx = g.choice(n, size=k, replace=False)
    x[idx] = g.uniform(100.0, 448.0, size=k) * np.where(g.random(k) < 0.5, -1.0, 1.0)
    x = x.reshape(rows, cols)
    tr = g.choice(rows // 32, size=n_zero_tiles, replace=True)
    tc = g.choice(cols // 32, size=n_zero_tiles, replace=True)
    for a, b in zip(tr, tc):
        x[32 * a:32 * a + 32, 32 * b:32 * b + 32] = 0.0
    return Matrix(f"{rows}x{cols}-{dtype}", rows, cols, dtype, to_dtype(x.ravel(), dtype), True,
                  {"full": [(0, n)], "partial": [(17, n // 4)]})


LAYER_TENSORS = [("qkv", 4096, 12288, True), ("out_proj", 4096, 4096, False),
                 ("up", 4096, 14336, True), ("down", 14336, 4096, False)]


def layer_batch(seed: int = 4, n_fragments: int = 8, tensors=None) -> Batch:
    """Transformer-layer weights end to end in one BF16 buffer, N(0, 0.02), alternating
    bidirectional and row-only outputs (bidirectional first), cut into ``n_fragments`` equal
    contiguous fragments (one per rank)."""
    tensors = list(LAYER_TENSORS if tensors is None else tensors)
    g = _rng(seed)
    offsets, total = [], 0
    for (_, r, c, _) in tensors:
        offsets.append(total)
        total += r * c
    x = g.normal(0.0, 0.02, size=total)
    if total % n_fragments:
        raise ValueError("fragments must be equal")
    f = total // n_fragments
    return Batch("layer-bf16", tensors, offsets, BF16, to_dtype(x, BF16),
                 [(i * f, f) for i in range(n_fragments)])


# ------------------------------------------------------------------ generic small inputs


def random_matrix(rows: int, cols: int, dtype: str, seed: int, kind: str = "mixed") -> np.ndarray:
    """Small synthetic matrices for edge-case tests.

    kinds: ``normal`` N(0,1); ``mixed`` N(0,1) times per-row 2^U[-20, 20] with a zero block and
    exact powers of two; ``tiny`` values around FP32/BF16 subnormals; ``huge`` values near
    the top of FP32's range (below BF16's overflow threshold)."""
    g = _rng(seed)
    if kind == "normal":
        x = g.standard_normal((rows, cols))
    elif kind == "mixed":
        x = g.standard_normal((rows, cols)) * np.exp2(g.uniform(-20, 20, size=(rows, 1)))
        x[: min(rows, 32), : min(cols, 32)] = 0.0
        if rows > 40 and cols > 8:
            x[40, :8] = np.exp2(np.arange(8) - 4.0) * np.where(np.arange(8) % 2, -1.0, 1.0)
    elif kind == "tiny":
        x = g.standard_normal((rows, cols)) * np.exp2(g.uniform(-149, -110, size=(rows, cols)))
    elif kind == "huge":
        sign = np.where(g.random((rows, cols)) < 0.5, -1.0, 1.0)
        x = sign * np.exp2(g.uniform(100.0, 127.95, size=(rows, cols)))
    else:
        raise ValueError(kind)
    return to_dtype(x.ravel(), dtype)


def device_matrix(rows: int, cols: int, dtype: str, seed: int, device) -> "torch.Tensor":
    """A large weight drawn on the device, for tests past the 32-bit size limits where a
    host-side draw would take minutes: N(0,1) times a per-row magnitude 2^U, U ~ Uniform[-20,
    20] (the "mixed" distribution of ``random_matrix`` without its fixed blocks), from torch's
    seeded device generator, rounded to FP32 and then, for BF16, to BF16 (both RNE).  Returns
    the flat row-major weight as a bfloat16 or float32 device tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    out = torch.empty(rows * cols, dtype=tdt, device=device)
    mag = torch.exp2(torch.rand(rows, generator=g, device=device) * 40.0 - 20.0)
    step = max(1, (1 << 26) // cols)  # rows per draw: about 2^26 values at a time
    for r in range(0, rows, step):
        n = min(step, rows - r)
        x = torch.randn(n, cols, generator=g, device=device, dtype=torch.float32)
        x *= mag[r:r + n, None]
        out[r * cols:(r + n) * cols] = x.reshape(-1).to(tdt)
    return out
