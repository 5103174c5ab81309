"""The agreement metric of the synthetic prediction-quality report (bench.py
--quality): the fraction of the first n ranked blocks that two top-K rows
share, averaged over rows.  Checked on hand-made ranked lists whose agreement
is known by counting.  This is the synthetic analog of the pages' figures for
how often the draft query's top-K set matches the next step's (paperpeel v2
§3.1) and for how far the previous token's set drifts (v2 §2.2)."""
import numpy as np
import pytest

import bench


def test_identical_and_disjoint_rows():
    a = np.array([[5, 3, 9, 1]])
    assert bench.topk_overlap(a, a, 4) == 1.0
    assert bench.topk_overlap(a, np.array([[0, 2, 4, 6]]), 4) == 0.0


def test_order_inside_the_prefix_does_not_matter():
    # the same four blocks ranked differently: a set comparison
    assert bench.topk_overlap(np.array([[1, 2, 3, 4]]), np.array([[4, 3, 2, 1]]), 4) == 1.0


def test_prefix_length_cuts_both_rows():
    a = np.array([[10, 11, 12, 13, 14, 15]])
    b = np.array([[11, 10, 20, 21, 12, 13]])
    # first 2: {10, 11} vs {11, 10} -> 2/2
    assert bench.topk_overlap(a, b, 2) == 1.0
    # first 4: {10..13} vs {11, 10, 20, 21} -> 2/4
    assert bench.topk_overlap(a, b, 4) == 0.5
    # all 6: {10..15} vs {10, 11, 12, 13, 20, 21} -> 4/6
    assert bench.topk_overlap(a, b, 6) == pytest.approx(4 / 6)


def test_mean_over_leading_axes():
    # [layers=1][R=2][H=2][K=4]: per-row agreements 1, 3/4, 1/2, 0 -> mean 9/16
    a = np.array([[[[0, 1, 2, 3], [4, 5, 6, 7]], [[8, 9, 10, 11], [12, 13, 14, 15]]]])
    b = np.array([[[[3, 2, 1, 0], [4, 5, 6, 99]], [[8, 9, 98, 97], [1, 2, 3, 4]]]])
    assert bench.topk_overlap(a, b, 4) == pytest.approx(9 / 16)


def test_mismatched_rows_rejected():
    with pytest.raises(ValueError):
        bench.topk_overlap(np.zeros((2, 4), int), np.zeros((3, 4), int), 4)
