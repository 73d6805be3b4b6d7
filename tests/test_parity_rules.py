"""The selection margin rule of tests/parity.py on hand-made rows (CPU).

A rule that accepts a wrong selection would let a GPU bug through every parity
test, so the rule itself is checked on rows whose verdict is known.
"""
import math

import pytest
import torch

from parity import MARGIN, check_indices, sum_factor


def _case(scores, top_k):
    s = torch.tensor(scores, dtype=torch.float32).view(1, 1, -1)
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))[:top_k]
    want = torch.tensor(sorted(order), dtype=torch.int32).view(1, 1, -1)
    lens = torch.tensor([16 * len(scores)], dtype=torch.int32)
    return s, want, lens


def test_clear_margin_demands_the_exact_set():
    s, want, lens = _case([0.0, 0.5, 0.1, 0.4], 2)   # top-2 {1, 3}, margin 0.3
    st = check_indices(want, want, s, lens, 2)
    assert st["strict"] == 1 and st["near_tie"] == 0
    with pytest.raises(AssertionError):
        check_indices(torch.tensor([[[1, 2]]], dtype=torch.int32), want, s, lens, 2)


def test_near_tie_accepts_either_set_in_the_scaled_units():
    s, want, lens = _case([0.0, 0.5, 0.4002, 0.4], 2)  # margin 2e-4 < 1e-3
    other = torch.tensor([[[1, 3]]], dtype=torch.int32)
    st = check_indices(other, want, s, lens, 2)
    assert st["near_tie"] == 1 and st["differ"] == 1
    # a block below s_(k) - MARGIN is still rejected
    s2, want2, _ = _case([0.0, 0.5, 0.4002, 0.4, 0.39], 2)
    with pytest.raises(AssertionError):
        check_indices(torch.tensor([[[1, 4]]], dtype=torch.int32), want2, s2,
                      torch.tensor([80], dtype=torch.int32), 2)


def test_sum_units_demand_exactness_on_the_same_near_tie():
    s, want, lens = _case([0.0, 0.5, 0.4002, 0.4], 2)
    other = torch.tensor([[[1, 3]]], dtype=torch.int32)
    f = sum_factor(4, 128)
    assert math.isclose(f, 4 * math.sqrt(128))
    assert 2e-4 * f > MARGIN  # the margin exceeds the threshold in the sum's units
    with pytest.raises(AssertionError):
        check_indices(other, want, s, lens, 2, sum_units=f)
    st = check_indices(want, want, s, lens, 2, sum_units=f)
    assert st["strict_sum"] == 1 and st["near_tie"] == 1


def test_malformed_rows_fail():
    s, want, lens = _case([0.0, 0.5, 0.1, 0.4], 2)
    for bad in ([[[3, 1]]], [[[1, 1]]], [[[1, 9]]], [[[1, -1]]]):
        with pytest.raises(AssertionError):
            check_indices(torch.tensor(bad, dtype=torch.int32), want, s, lens, 2)


def test_k_covering_every_block_is_exact_and_padded():
    s, _, lens = _case([0.3, 0.1], 4)
    want = torch.tensor([[[0, 1, -1, -1]]], dtype=torch.int32)
    st = check_indices(want, want, s, lens, 4)
    assert st["strict"] == 1
    with pytest.raises(AssertionError):
        check_indices(torch.tensor([[[0, -1, -1, -1]]], dtype=torch.int32), want, s, lens, 4)
