"""Host-side pieces of bench.py (no GPU): the pair counts its FLOP figures use."""

import os
import sys

import numpy as np
import pytest

import oracle

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("grid,tile", [((64, 48, 80), (4, 12, 10)), ((64, 48, 79), (8, 6, 10)), ((3, 5, 7), (2, 2, 3)),
                                       ((7, 7, 7), (1, 2, 7)), ((4, 8, 8), (3, 4, 4)), ((5, 1, 9), (5, 1, 9))])
def test_present_pairs_count_the_padded_partition(grid, tile):
    """Query-key pairs of each pass = sum of squared present counts per window and
    per offset group of the oracle's padded window index."""
    idx = oracle.padded_window_index(grid, tile)
    present = idx >= 0
    assert bench.present_pairs(grid, tile) == (int((present.sum(1) ** 2).sum()), int((present.sum(0) ** 2).sum()))


def test_present_pairs_on_whole_tilings_are_n_w_and_n_g():
    n, W, G = 245760, 480, 512
    assert bench.present_pairs((64, 48, 80), (4, 12, 10)) == (n * W, n * G)
