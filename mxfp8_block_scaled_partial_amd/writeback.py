"""Batch helper for the distributed master-weight writeback into MXFP8, on one GPU.

Several weights lie end to end in one flat master buffer, which ranks hold as contiguous
fragments ("Support row-only MXFP8 distributed master-weight casts", sections Changes and
Validation: mixed row-only / bidirectional batches, fragment outputs, boundaries inside a
32-value block, empty shards).  This module only plans calls into the C ABI:

  * every fragment is split into per-weight pieces;
  * the amax of every present direction of the batch lives in one packed buffer (weights in
    batch order, row-wise then column-wise), so the combine is one call per batch -- the
    single-GPU stand-in for the one packed MAX all-reduce;
  * either all fragments accumulate into one shared packed buffer (cut blocks merge through
    the kernel's atomic max), or each fragment gets its own packed buffer, as a rank would,
    and ``mxfp8_combine_amax`` MAX-combines them;
  * scales are computed once per weight over the range its fragments cover, and every
    piece is cast in place into caller-owned, full-size MXFP8 storage; with ``fused=True``
    each piece instead derives its scales from the combined amax inside its cast
    (``mxfp8_scales_and_cast``), so the scales take no pass of their own.

All arithmetic runs in the library's kernels; buffers are zero-filled with torch's fill.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass(frozen=True)
class WeightSpec:
    rows: int
    cols: int
    colwise: bool

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def amax_row_entries(self) -> int:
        return self.rows * B.nblocks(self.cols)

    @property
    def amax_col_entries(self) -> int:
        return B.nblocks(self.rows) * self.cols if self.colwise else 0


class MXFP8Storage:
    """MXFP8 outputs of one weight: E4M3 data in row-major order for each present direction
    and E8M0 scales ([rows][ceil(cols/32)] row-wise, [ceil(rows/32)][cols] column-wise).
    Allocated once; the writeback only writes into it, so its pointers never change."""

    def __init__(self, spec: WeightSpec, device):
        nb, nbands = B.nblocks(spec.cols), B.nblocks(spec.rows)
        self.spec = spec
        self.data_row = torch.zeros(spec.numel, dtype=torch.uint8, device=device)
        self.scale_row = torch.zeros(spec.rows, nb, dtype=torch.uint8, device=device)
        if spec.colwise:
            self.data_col = torch.zeros(spec.numel, dtype=torch.uint8, device=device)
            self.scale_col = torch.zeros(nbands, spec.cols, dtype=torch.uint8, device=device)
        else:  # row-only: the column-wise outputs are absent (empty handles)
            self.data_col = torch.empty(0, dtype=torch.uint8, device=device)
            self.scale_col = torch.empty(0, 0, dtype=torch.uint8, device=device)


class PackedAmax:
    """One flat buffer holding the amax of every present direction of a batch."""

    def __init__(self, specs, dtype: torch.dtype, device, buffer: torch.Tensor | None = None):
        self.specs = list(specs)
        self.offsets = []
        total = 0
        for s in self.specs:
            self.offsets.append(total)
            total += s.amax_row_entries + s.amax_col_entries
        self.numel = total
        self.buffer = (torch.zeros(total, dtype=dtype, device=device) if buffer is None
                       else buffer)
        if self.buffer.numel() != total or self.buffer.dtype != dtype:
            raise ValueError("packed buffer has the wrong size or dtype")

    def views(self, i: int):
        s, o = self.specs[i], self.offsets[i]
        nb, nbands = B.nblocks(s.cols), B.nblocks(s.rows)
        row = self.buffer[o:o + s.amax_row_entries].view(s.rows, nb)
        if not s.colwise:
            return row, None
        o += s.amax_row_entries
        return row, self.buffer[o:o + s.amax_col_entries].view(nbands, s.cols)


def split_fragment(specs, frag_start: int, frag_len: int):
    """Pieces of flat fragment [frag_start, frag_start + frag_len) of the batch's buffer:
    a list of (weight index, start within the weight, length, offset within the fragment)."""
    out, base = [], 0
    end = frag_start + frag_len
    for i, s in enumerate(specs):
        lo, hi = max(frag_start, base), min(end, base + s.numel)
        if lo < hi:
            out.append((i, lo - base, hi - lo, lo - frag_start))
        base += s.numel
    return out


class Plan:
    """Prepared C-ABI calls for one set of master fragments (pointers are baked in)."""

    def __init__(self, wb: "Writeback", fragments_values):
        self.wb = wb
        self.keep = list(fragments_values)       # keep the tensors alive
        amax_pieces, cast_pieces = [], []
        for f, ((fs, fl), x) in enumerate(zip(wb.fragments, self.keep)):
            if x.numel() != fl or x.dtype != wb.dtype:
                raise ValueError(f"fragment {f}: expected {fl} values of {wb.dtype}")
            packed = wb.packed[f if not wb.shared else 0]
            for (i, s, n, off) in split_fragment(wb.specs, fs, fl):
                spec, st = wb.specs[i], wb.storage[i]
                ar, ac = packed.views(i)
                xin = x[off:off + n]
                amax_pieces.append(B.make_piece(spec.rows, spec.cols, s, xin, amax_row=ar,
                                                amax_col=ac, preround=wb.preround))
                car, cac = wb.combined.views(i) if wb.fused else (None, None)
                cast_pieces.append(B.make_piece(
                    spec.rows, spec.cols, s, xin, amax_row=car, amax_col=cac,
                    scale_row=st.scale_row, scale_col=st.scale_col,
                    data_row=st.data_row[s:s + n],
                    data_col=st.data_col[s:s + n] if spec.colwise else None,
                    preround=wb.preround))
        self.amax = (B.Piece * len(amax_pieces))(*amax_pieces)
        self.cast = (B.Piece * len(cast_pieces))(*cast_pieces)
        self.n_amax, self.n_cast = len(amax_pieces), len(cast_pieces)

    def stages(self, stream=None):
        """The writeback as (name, callable) stages, in order: zero-fill of the packed amax,
        partial amax, MAX-combine (only with one packed buffer per fragment), then scales and
        cast, or one fused scales-and-cast stage."""
        wb = self.wb
        lib = B.lib()
        sp = B._stream(stream)

        def zero():
            wb.packed_storage.zero_()

        def amax():
            B._check(lib.mxfp8_partial_amax(self.amax, self.n_amax, sp))

        def combine():
            B._check(lib.mxfp8_combine_amax(wb.combine_dst, wb.combine_srcs, len(wb.packed),
                                            wb.combined.numel, B.dtype_code(wb.dtype), sp))

        def scales():
            B._check(lib.mxfp8_compute_scales(wb.scale_pieces, wb.n_scale, sp))

        def cast():
            B._check(lib.mxfp8_partial_cast(self.cast, self.n_cast, sp))

        def scales_cast():
            B._check(lib.mxfp8_scales_and_cast(self.cast, self.n_cast, sp))

        out = [("zero", zero), ("amax", amax)]
        if not wb.shared and len(wb.packed) > 1:
            out.append(("combine", combine))
        if wb.fused:
            return out + [("scales_cast", scales_cast)]
        return out + [("scales", scales), ("cast", cast)]

    def run(self, stream=None):
        for _, fn in self.stages(stream):
            fn()


class Writeback:
    """Writeback of one batch of weights, held as contiguous fragments of a flat buffer.

    ``shared=True`` accumulates every fragment's amax in one packed buffer; ``shared=False``
    gives each fragment its own packed buffer (one per rank) and MAX-combines them.
    ``fused=True`` computes the scales inside the cast."""

    def __init__(self, specs, dtype: torch.dtype, device, fragments, shared: bool = True,
                 preround: bool = False, fused: bool = False):
        self.specs = list(specs)
        self.dtype = dtype
        self.fused = fused
        self.fragments = [(int(s), int(l)) for s, l in fragments]
        self.shared = shared
        self.preround = preround
        total = sum(s.numel for s in self.specs)
        for s, l in self.fragments:
            if s < 0 or l < 0 or s + l > total:
                raise ValueError(f"fragment [{s}, {s + l}) outside the batch of {total}")
        self.storage = [MXFP8Storage(s, device) for s in self.specs]
        n_bufs = 1 if shared else max(1, len(self.fragments))
        # all packed buffers in one allocation (one zero-fill per update); each starts on a
        # 16-byte boundary so the combine can move 16-byte vectors
        entries = PackedAmax(self.specs, dtype, "meta").numel
        per = -(-entries * torch.tensor([], dtype=dtype).element_size() // 16) * 16
        per //= torch.tensor([], dtype=dtype).element_size()
        self.packed_storage = torch.zeros(n_bufs * per, dtype=dtype, device=device)
        self.packed = [PackedAmax(self.specs, dtype, device,
                                  self.packed_storage[i * per:i * per + entries])
                       for i in range(n_bufs)]
        self.combined = self.packed[0]
        import ctypes
        self.combine_dst = self.combined.buffer.data_ptr()
        self.combine_srcs = (ctypes.c_void_p * n_bufs)(*[p.buffer.data_ptr() for p in self.packed])
        # scales: one piece per weight and maximal run of adjacent fragments
        pieces = []
        for i, (spec, st) in enumerate(zip(self.specs, self.storage)):
            runs = []
            for fs, fl in self.fragments:
                for (j, s, n, _) in split_fragment(self.specs, fs, fl):
                    if j == i:
                        runs.append([s, s + n])
            runs.sort()
            merged = []
            for lo, hi in runs:
                if merged and lo <= merged[-1][1]:
                    merged[-1][1] = max(merged[-1][1], hi)
                else:
                    merged.append([lo, hi])
            ar, ac = self.combined.views(i)
            for lo, hi in merged:
                pieces.append(B.make_piece(spec.rows, spec.cols, lo, None, length=hi - lo,
                                           in_dtype=dtype, amax_row=ar, amax_col=ac,
                                           scale_row=st.scale_row, scale_col=st.scale_col))
        self.scale_pieces = (B.Piece * len(pieces))(*pieces)
        self.n_scale = len(pieces)

    def plan(self, fragments_values) -> Plan:
        return Plan(self, fragments_values)

    def __call__(self, fragments_values, stream=None):
        self.plan(fragments_values).run(stream)
        return self
