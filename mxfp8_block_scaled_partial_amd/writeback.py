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
    (``mxfp8_scales_and_cast``), so the scales take no pass of their own;
  * with ``single_pass=True`` the whole 32-row bands inside a piece, whose blocks no other
    fragment touches and whose amax are therefore final without the combine, go through the
    one-pass ``mxfp8_quantize``, which writes their amax straight into the combined buffer;
    only the partial bands at the piece's two ends take the amax -> combine -> scales + cast
    path, the combine covers only their entries (the single-GPU form of all-reducing just
    the blocks that fragments share), and the two run overlapped on two streams.

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

    def __init__(self, spec: WeightSpec, device, with_data: bool = True):
        nb, nbands = B.nblocks(spec.cols), B.nblocks(spec.rows)
        self.spec = spec
        n = spec.numel if with_data else 0
        self.data_row = torch.zeros(n, dtype=torch.uint8, device=device)
        self.scale_row = torch.zeros(spec.rows, nb, dtype=torch.uint8, device=device)
        if spec.colwise:
            self.data_col = torch.zeros(n, dtype=torch.uint8, device=device)
            self.scale_col = torch.zeros(nbands, spec.cols, dtype=torch.uint8, device=device)
        else:  # row-only: the column-wise outputs are absent (empty handles)
            self.data_col = torch.empty(0, dtype=torch.uint8, device=device)
            self.scale_col = torch.empty(0, 0, dtype=torch.uint8, device=device)


class FragmentOutputs:
    """E4M3 data of one fragment of the flat batch, FSDP style: byte k of ``data_row`` /
    ``data_col`` belongs to flat element ``start + k`` of the batch.  ``data_col`` holds the
    column-wise bytes of the bidirectional weights' elements; its bytes at row-only weights'
    elements are not written.  Allocated once, written in place."""

    def __init__(self, start: int, length: int, any_colwise: bool, device):
        self.start, self.length = start, length
        self.data_row = torch.zeros(length, dtype=torch.uint8, device=device)
        self.data_col = torch.zeros(length if any_colwise else 0, dtype=torch.uint8,
                                    device=device)


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


def whole_bands(spec: WeightSpec, a: int, b: int):
    """The largest [lo, hi) inside [a, b) made of whole 32-row bands of the weight (the short
    last band counts as whole); lo >= hi when there is none."""
    band = 32 * spec.cols
    lo = -(-a // band) * band
    hi = b if b == spec.numel else (b // band) * band
    return lo, hi


def boundary_spans(specs, fragments, dtype=torch.float32):
    """Packed-entry ranges [lo, hi) of the bands that a partial piece (the part of a
    fragment's piece outside its whole bands) touches, merged: the row-wise entries of the
    band's rows and, for bidirectional weights, the band's column-wise entries."""
    spans = []
    offsets = PackedAmax(specs, dtype, "meta").offsets
    for fs, fl in fragments:
        for (i, s, n, _) in split_fragment(specs, fs, fl):
            spec = specs[i]
            lo, hi = whole_bands(spec, s, s + n)
            parts = [(s, s + n)] if lo >= hi else [(s, lo), (hi, s + n)]
            nb, band = B.nblocks(spec.cols), 32 * spec.cols
            for a, b in parts:
                if a >= b:
                    continue
                for bd in range(a // band, (b - 1) // band + 1):
                    r0, r1 = 32 * bd, min(32 * bd + 32, spec.rows)
                    o = offsets[i]
                    spans.append((o + r0 * nb, o + r1 * nb))
                    if spec.colwise:
                        oc = o + spec.amax_row_entries + bd * spec.cols
                        spans.append((oc, oc + spec.cols))
    spans.sort()
    merged = []
    for lo, hi in spans:
        if merged and lo <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], hi)
        else:
            merged.append([lo, hi])
    return [(lo, hi) for lo, hi in merged]


class Plan:
    """Prepared C-ABI calls for one set of master fragments (pointers are baked in)."""

    def __init__(self, wb: "Writeback", fragments_values):
        self.wb = wb
        self.keep = list(fragments_values)       # keep the tensors alive
        amax_pieces, cast_pieces, quant_pieces = [], [], []
        # (weight index, start, end) of every amax / cast piece and every quantize piece
        self.partial_ranges, self.quant_ranges = [], []
        for f, ((fs, fl), x) in enumerate(zip(wb.fragments, self.keep)):
            if x.numel() != fl or x.dtype != wb.dtype:
                raise ValueError(f"fragment {f}: expected {fl} values of {wb.dtype}")
            packed = wb.packed[f if not wb.shared else 0]
            fo = wb.fragment_outputs[f] if wb.fragment_outputs else None
            for (i, s, n, off) in split_fragment(wb.specs, fs, fl):
                spec, st = wb.specs[i], wb.storage[i]
                ar, ac = packed.views(i)
                car, cac = wb.combined.views(i)
                ranges = [(s, s + n)]
                if wb.single_pass:
                    lo, hi = whole_bands(spec, s, s + n)
                    if lo < hi:
                        ranges = [(s, lo), (hi, s + n)]
                        # no other fragment touches these blocks: their amax are final and go
                        # straight into the combined buffer
                        quant_pieces.append(self._piece(spec, st, fo, x, off - s, lo, hi, car,
                                                        cac))
                        self.quant_ranges.append((i, lo, hi))
                for a, b in ranges:
                    if a == b:
                        continue
                    xin = x[off + a - s:off + b - s]
                    amax_pieces.append(B.make_piece(spec.rows, spec.cols, a, xin, amax_row=ar,
                                                    amax_col=ac, preround=wb.preround))
                    cast_pieces.append(self._piece(spec, st, fo, x, off - s, a, b,
                                                   *((car, cac) if wb.fused else (None, None))))
                    self.partial_ranges.append((i, a, b))
        self.amax = (B.Piece * len(amax_pieces))(*amax_pieces)
        self.cast = (B.Piece * len(cast_pieces))(*cast_pieces)
        self.quant = (B.Piece * len(quant_pieces))(*quant_pieces)
        self.n_amax, self.n_cast = len(amax_pieces), len(cast_pieces)
        self.n_quant = len(quant_pieces)

    def _piece(self, spec, st, fo, x, shift, a, b, amax_row, amax_col):
        """Piece [a, b) of a weight whose values sit at x[a + shift]; its data go to the
        weight's full storage, or to the fragment's outputs ``fo`` at the same offsets as x."""
        if fo is None:
            dr, dc = st.data_row[a:b], st.data_col[a:b] if spec.colwise else None
        else:
            dr = fo.data_row[a + shift:b + shift]
            dc = fo.data_col[a + shift:b + shift] if spec.colwise else None
        return B.make_piece(
            spec.rows, spec.cols, a, x[a + shift:b + shift], amax_row=amax_row,
            amax_col=amax_col, scale_row=st.scale_row, scale_col=st.scale_col,
            data_row=dr, data_col=dc, preround=self.wb.preround)

    def _calls(self, stream):
        """The library calls of the writeback on torch stream ``stream``, by name."""
        import torch
        wb = self.wb
        lib = B.lib()
        code = B.dtype_code(wb.dtype)
        sp = stream.cuda_stream

        def zero():
            with torch.cuda.stream(stream):
                wb.packed_storage.zero_()

        def zero_combined():
            with torch.cuda.stream(stream):
                wb.packed_storage[:wb.per_buffer].zero_()

        def zero_partials():
            with torch.cuda.stream(stream):
                wb.packed_storage[wb.per_buffer:].zero_()

        def amax():
            B._check(lib.mxfp8_partial_amax(self.amax, self.n_amax, sp))

        def combine():
            for dst, srcs, count in wb.combine_calls:
                B._check(lib.mxfp8_combine_amax(dst, srcs, len(wb.packed), count, code, sp))

        def scales():
            B._check(lib.mxfp8_compute_scales(wb.scale_pieces, wb.n_scale, sp))

        def cast():
            B._check(lib.mxfp8_partial_cast(self.cast, self.n_cast, sp))

        def scales_cast():
            B._check(lib.mxfp8_scales_and_cast(self.cast, self.n_cast, sp))

        def quantize():
            B._check(lib.mxfp8_quantize(self.quant, self.n_quant, sp))

        return dict(zero=zero, zero_combined=zero_combined, zero_partials=zero_partials,
                    amax=amax, combine=combine, scales=scales, cast=cast,
                    scales_cast=scales_cast, quantize=quantize)

    def stages(self, stream=None):
        """The writeback as (name, callable) stages in one stream, in order: zero-fill of the
        packed amax, partial amax, the single-pass quantize of whole bands (``single_pass``
        only), MAX-combine (only with one packed buffer per fragment), then scales and cast,
        or one fused scales-and-cast stage.  ``stream`` is a torch stream (None: the current
        stream when this is called)."""
        import torch
        wb = self.wb
        c = self._calls(torch.cuda.current_stream() if stream is None else stream)
        out = [("zero", c["zero"]), ("amax", c["amax"])]
        if wb.single_pass:
            out.append(("quantize", c["quantize"]))
        if not wb.shared and len(wb.packed) > 1:
            out.append(("combine", c["combine"]))
        if wb.fused:
            return out + [("scales_cast", c["scales_cast"])]
        return out + [("scales", c["scales"]), ("cast", c["cast"])]

    def run(self, stream=None):
        """Run the writeback.  With ``single_pass`` the quantize of whole bands runs on a side
        stream, overlapped with the partial chain (amax -> combine -> scales + cast of the
        bands at the cuts), which touches none of its blocks; both start after the combined
        buffer is cleared and the call returns with the caller's stream waiting on both."""
        wb = self.wb
        if not (wb.single_pass and self.n_quant and self.n_cast):
            for _, fn in self.stages(stream):
                fn()
            return
        import torch
        main = torch.cuda.current_stream() if stream is None else stream
        side = wb.side_stream
        c, cs = self._calls(main), self._calls(side)
        c["zero_combined"]()
        side.wait_stream(main)
        cs["quantize"]()
        if len(wb.packed) > 1:
            c["zero_partials"]()
        c["amax"]()
        if not wb.shared and len(wb.packed) > 1:
            c["combine"]()
        c["scales_cast"]()
        main.wait_stream(side)


class Writeback:
    """Writeback of one batch of weights, held as contiguous fragments of a flat buffer.

    ``shared=True`` accumulates every fragment's amax in one packed buffer; ``shared=False``
    gives each fragment its own packed buffer (one per rank) and MAX-combines them.
    ``fused=True`` computes the scales inside the cast; ``single_pass=True`` (which implies
    ``fused``) quantizes the whole bands inside each piece in one pass.

    The data go in place into full-size per-weight storage (``storage[i].data_row`` ...), or
    with ``fragment_outputs=True`` into one fragment-sized buffer per fragment and direction
    (``fragment_outputs[f]``), the FSDP-style interface; scales are per weight either way."""

    def __init__(self, specs, dtype: torch.dtype, device, fragments, shared: bool = True,
                 preround: bool = False, fused: bool = False, single_pass: bool = False,
                 fragment_outputs: bool = False):
        self.specs = list(specs)
        self.dtype = dtype
        self.single_pass = single_pass
        self.fused = fused or single_pass
        self.fragments = [(int(s), int(l)) for s, l in fragments]
        self.shared = shared
        self.preround = preround
        total = sum(s.numel for s in self.specs)
        for s, l in self.fragments:
            if s < 0 or l < 0 or s + l > total:
                raise ValueError(f"fragment [{s}, {s + l}) outside the batch of {total}")
        self.storage = [MXFP8Storage(s, device, with_data=not fragment_outputs)
                        for s in self.specs]
        any_col = any(s.colwise for s in self.specs)
        self.fragment_outputs = ([FragmentOutputs(s, l, any_col, device)
                                  for s, l in self.fragments] if fragment_outputs else None)
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
        self.per_buffer = per
        self.combined = self.packed[0]
        # MAX-combine calls as (dst pointer, source pointer array, entries): the whole packed
        # buffer, or with ``single_pass`` only the entries of bands that a partial piece
        # touches (the others hold the single-pass quantize's final amax)
        import ctypes
        esz = torch.tensor([], dtype=dtype).element_size()
        spans = ([(0, entries)] if not single_pass
                 else boundary_spans(self.specs, self.fragments, dtype))
        self.combine_calls = []
        for lo, hi in spans:
            srcs = (ctypes.c_void_p * n_bufs)(*[p.buffer.data_ptr() + lo * esz
                                                  for p in self.packed])
            self.combine_calls.append((self.combined.buffer.data_ptr() + lo * esz, srcs, hi - lo))
        self._side = None
        self.device = device
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

    @property
    def side_stream(self):
        """The second stream of the single-pass writeback (default priority)."""
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
        return self._side

    def plan(self, fragments_values) -> Plan:
        return Plan(self, fragments_values)

    def __call__(self, fragments_values, stream=None):
        self.plan(fragments_values).run(stream)
        return self


def cast_master_fragments(fragments, weights, **options) -> Writeback:
    """One writeback of a batch: ``fragments`` is a list of (start, values) pairs, each a
    contiguous shard of the batch's flat master buffer (``values`` a 1-D float32 / bfloat16
    device tensor holding elements ``start ... start + len - 1``); ``weights`` the batch's
    ``WeightSpec`` list in buffer order.  Splits every fragment into per-weight pieces and runs
    one partial-amax call, at most one combine, and the scale and cast calls (see
    ``Writeback`` for ``options``).  Returns the ``Writeback``, whose storage (or fragment
    outputs) hold the MXFP8 result; keep it to run later updates with stable pointers."""
    fragments = list(fragments)
    if not fragments:
        raise ValueError("need at least one fragment")
    values = [v for _, v in fragments]
    dtype = values[0].dtype
    if any(v.dtype != dtype for v in values):
        raise ValueError("all fragments must share one dtype")
    wb = Writeback(weights, dtype, values[0].device, [(int(s), v.numel()) for s, v in fragments],
                   **options)
    return wb(values)
