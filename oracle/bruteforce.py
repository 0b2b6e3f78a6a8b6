"""Brute-force MXFP8 checker for tiny inputs (exact rational arithmetic, nearest-code search).

TEST INFRASTRUCTURE ONLY: used by the oracle's self-tests to pin ``mxfp8_oracle.c`` to a
second formulation that shares none of its arithmetic.  Where the C oracle rounds with
frexp / ldexp / nearbyint, this module

  * decodes every non-negative finite E4M3 code from its bit fields (OFP8 E4M3: bias 7,
    3 mantissa bits, exponent field 0 = subnormal, 0x7F = NaN) and picks the code nearest
    to the scaled value, ties to the code with an even mantissa (round-to-nearest-even);
    values beyond 448 land on 448 because it is the largest finite code (saturation);
  * finds the E8M0 scale by searching the byte b in [0, 254] for which the block's amax
    times 2^(127-b) lies in [2^8, 2^9), i.e. whose largest element lands in E4M3's top
    binade (OCP MX, emax_elem = 8), clamping at the ends of the search;
  * rounds FP32 to BF16 by searching the table of every finite BF16 value;
  * walks the fragment element by element with Python integers for the block indices.

Everything is Python ``fractions.Fraction``; it is slow and meant for a few thousand
elements.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np


def _e4m3_decode(code: int) -> Fraction:
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(1, 64)           # m/8 * 2^(1-7)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


E4M3_TABLE = [(c, _e4m3_decode(c)) for c in range(0x7F)]  # 0x00 .. 0x7E, all finite >= 0


def nearest_e4m3(v: Fraction) -> int:
    """Nearest finite E4M3 code to v, ties to even mantissa; the sign bit follows v's sign
    (pass ``neg`` through :func:`nearest_e4m3_signed` for negative zero)."""
    a = abs(v)
    best, bestd = None, None
    for c, val in E4M3_TABLE:
        d = abs(a - val)
        if bestd is None or d < bestd or (d == bestd and (c & 1) == 0):
            best, bestd = c, d
    return best


def nearest_e4m3_signed(v: Fraction, negative: bool) -> int:
    return (0x80 if negative else 0) | nearest_e4m3(v)


def e8m0_search(amax: Fraction) -> int:
    if amax == 0:
        return 0
    for b in range(0, 255):
        scaled = amax * Fraction(2) ** (127 - b)
        if Fraction(256) <= scaled < Fraction(512):
            return b
    # no byte puts amax in E4M3's top binade: clamp to the nearer end of the range
    return 0 if amax * Fraction(2) ** 127 < 256 else 254


def fp32_fraction(x: float) -> Fraction:
    return Fraction(float(np.float32(x)))


def bf16_bits_fraction(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


def _bf16_table():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)              # +0 .. largest finite
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits, vals


_BF16_BITS, _BF16_VALS = _bf16_table()


def bf16_nearest(x: Fraction) -> Fraction:
    """Nearest finite BF16 value to x by table search, ties to the even bit pattern."""
    a = abs(x)
    i = int(np.searchsorted(_BF16_VALS, float(a)))  # float(a) is exact for FP32 inputs
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(_BF16_VALS)]
    best, bestd = None, None
    for j in cands:
        d = abs(a - Fraction(_BF16_VALS[j]))
        if bestd is None or d < bestd or (d == bestd and (int(_BF16_BITS[j]) & 1) == 0):
            best, bestd = j, d
    r = Fraction(_BF16_VALS[best])
    return -r if x < 0 else r


def _values(x_frag, preround):
    """Working values of the fragment as (Fraction, is_negative) pairs."""
    out = []
    for v in x_frag.tolist():
        if x_frag.dtype == np.uint16:
            f = bf16_bits_fraction(v)
            neg = bool(v & 0x8000)
        else:
            f = Fraction(float(v))
            neg = struct.unpack("<I", struct.pack("<f", v))[0] >> 31 == 1
            if preround:
                f = bf16_nearest(f)
        out.append((f, neg))
    return out


def writeback(x_full, rows, cols, fragments, colwise=True, preround=False):
    """Whole path over (start, length) fragments, brute force.  Returns the same keys as
    ``oracle.writeback`` with amax as Fractions in dicts keyed by block."""
    amax_r, amax_c = {}, {}
    vals = {}
    for (s, l) in fragments:
        for k, (f, neg) in enumerate(_values(x_full[s:s + l], preround)):
            i = s + k
            r, c = divmod(i, cols)
            vals[i] = (f, neg)
            key = (r, c // 32)
            amax_r[key] = max(amax_r.get(key, Fraction(0)), abs(f))
            if colwise:
                key = (r // 32, c)
                amax_c[key] = max(amax_c.get(key, Fraction(0)), abs(f))
    sc_r = {k: e8m0_search(a) for k, a in amax_r.items()}
    sc_c = {k: e8m0_search(a) for k, a in amax_c.items()}
    n = rows * cols
    data_r = np.zeros(n, np.uint8)
    data_c = np.zeros(n, np.uint8) if colwise else None
    for i, (f, neg) in vals.items():
        r, c = divmod(i, cols)
        b = sc_r[(r, c // 32)]
        data_r[i] = nearest_e4m3_signed(f * Fraction(2) ** (127 - b), neg)
        if colwise:
            b = sc_c[(r // 32, c)]
            data_c[i] = nearest_e4m3_signed(f * Fraction(2) ** (127 - b), neg)
    return {"amax_row": amax_r, "amax_col": amax_c, "scale_row": sc_r, "scale_col": sc_c,
            "data_row": data_r, "data_col": data_c}
