"""Algorithmic HBM bytes of each step, the numerator of the reported bandwidths.

What the method must move, each item once: the fragment's input values, the amax entries it
touches (written; the entry of a block the fragment holds whole is set without being read),
the scale bytes and the E4M3 outputs.  Re-reads, staging and padding are excluded, and so are
the reads of the entries of blocks a fragment boundary cuts (their merge reads them back: at
most 2 row-wise and cols column-wise blocks at each end of a fragment), so bytes / time is a
lower bound on the bandwidth the hardware actually delivered.

For a fragment [start, start + len) of a rows x cols weight, with s_in = input element bytes
(2 BF16, 4 FP32; amax entries have the same width), D = present directions, and T_row /
T_col the row-wise / column-wise blocks the fragment touches:

  partial amax    len * s_in + (T_row + T_col) * s_in
  compute scales  (T_row + T_col) * (s_in + 1)
  partial cast    len * s_in + (T_row + T_col) * 1 + len * D
  scales + cast   len * s_in + (T_row + T_col) * (s_in + 1) + len * D   (fused: amax entries
                  read, scale bytes written, no scale read-back)
  quantize        len * s_in + (T_row + T_col) * (s_in + 1) + len * D   (single pass over
                  whole bands: input read once, amax and scales written once)
  combine         (K + 1) * P * s_in     (K partial packed buffers of P entries -> one)
  zero-fill       K * P * s_in
"""
from __future__ import annotations

BLOCK = 32


def touched_row_blocks(rows: int, cols: int, start: int, length: int) -> int:
    if length <= 0:
        return 0
    end = start + length
    nb = (cols + BLOCK - 1) // BLOCK
    r0, r1 = start // cols, (end - 1) // cols
    if r0 == r1:
        return (end - 1 - r0 * cols) // BLOCK - (start - r0 * cols) // BLOCK + 1
    first = nb - (start - r0 * cols) // BLOCK
    last = (end - 1 - r1 * cols) // BLOCK + 1
    return first + last + (r1 - r0 - 1) * nb


def touched_col_blocks(rows: int, cols: int, start: int, length: int) -> int:
    """Column-wise blocks (b, c) holding at least one element of the fragment."""
    if length <= 0:
        return 0
    end = start + length
    b0, b1 = (start // cols) // BLOCK, ((end - 1) // cols) // BLOCK

    def band_count(b: int) -> int:
        lo, hi = b * BLOCK * cols, min((b + 1) * BLOCK, rows) * cols  # band's flat range
        s, e = max(start, lo), min(end, hi)
        if s >= e:
            return 0
        if e - s >= cols:
            return cols                   # a whole row's worth of columns is covered
        cs, ce = s % cols, (e - 1) % cols
        return ce - cs + 1 if cs <= ce else cols - cs + ce + 1

    if b0 == b1:
        return band_count(b0)
    return band_count(b0) + band_count(b1) + (b1 - b0 - 1) * cols


def piece_bytes(rows: int, cols: int, start: int, length: int, s_in: int, colwise: bool):
    """Per-step algorithmic bytes of one piece: dict with amax, scales, cast, scales_cast,
    quantize."""
    tr = touched_row_blocks(rows, cols, start, length)
    tc = touched_col_blocks(rows, cols, start, length) if colwise else 0
    d = 2 if colwise else 1
    return {"amax": length * s_in + (tr + tc) * s_in,
            "scales": (tr + tc) * (s_in + 1),
            "cast": length * s_in + (tr + tc) + length * d,
            "scales_cast": length * s_in + (tr + tc) * (s_in + 1) + length * d,
            "quantize": length * s_in + (tr + tc) * (s_in + 1) + length * d,
            "touched_row": tr, "touched_col": tc}


def combine_bytes(k: int, packed_entries: int, s_in: int) -> int:
    return (k + 1) * packed_entries * s_in


def zero_bytes(k: int, packed_entries: int, s_in: int) -> int:
    return k * packed_entries * s_in
