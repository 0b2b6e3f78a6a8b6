"""The algorithmic byte model's touched-block counts against a brute-force enumeration."""
import numpy as np
import pytest

from mxfp8_block_scaled_partial_amd import bytes_model as BM


def brute(rows, cols, start, length):
    i = np.arange(start, start + length)
    r, c = i // cols, i % cols
    return len(set(zip(r, c // 32))), len(set(zip(r // 32, c)))


@pytest.mark.parametrize("rows,cols", [(64, 64), (37, 45), (100, 96), (1, 70), (70, 1), (65, 32)])
def test_touched_counts_match_enumeration(rows, cols):
    n = rows * cols
    g = np.random.Generator(np.random.PCG64(rows + cols))
    cases = [(0, n), (0, 0), (17, 1), (n - 1, 1)] + [
        tuple(sorted(g.integers(0, n + 1, 2))) for _ in range(40)]
    for a, b in cases:
        s, l = (a, b) if (a, b) in ((0, n), (0, 0), (17, 1), (n - 1, 1)) else (a, b - a)
        if s + l > n:
            continue
        tr, tc = brute(rows, cols, s, l)
        assert BM.touched_row_blocks(rows, cols, s, l) == tr, (s, l)
        assert BM.touched_col_blocks(rows, cols, s, l) == tc, (s, l)


def test_bytes_per_element_at_full_size():
    rows, cols = 16384, 6144
    n = rows * cols
    b = BM.piece_bytes(rows, cols, 0, n, 2, True)
    assert b["touched_row"] == n // 32 and b["touched_col"] == n // 32
    assert b["amax"] / n == pytest.approx(2 + 2 * 2 / 32)  # input, then 2 entries per 32
    assert b["cast"] / n == pytest.approx(2 + 2 / 32 + 2)
    # fused: each element's share of its two blocks' amax entries (2 bytes) and scales (1)
    assert b["scales_cast"] / n == pytest.approx(2 + 2 * (2 + 1) / 32 + 2)
