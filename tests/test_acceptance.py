"""The GPU-vs-oracle acceptance helper itself (no GPU): exact ties must follow
the lower-id rule, near-ties get the tolerance window, clear gaps need the
oracle's exact set.  Each case feeds the helper a selection with one planted
mistake and checks that it is refused."""
import numpy as np
import pytest

import msa_cases as M
from oracle import msa_oracle as O


def scores_with_ties():
    # 10 documents; 3 and 7 tie exactly at the cut (k = 4), 1 and 5 tie
    # exactly inside the selection, 8 is far below
    s = np.array([[0.10, 0.50, 0.05, 0.30, 0.02, 0.50, 0.01, 0.30, 0.00, 0.60]])
    return s


def test_oracle_answer_passes():
    s = scores_with_ties()
    ids, vals = O.select_topk(s, 4)
    assert ids[0].tolist() == [9, 1, 5, 3]
    M.check_topk(ids, vals, s, 4)


def test_higher_id_at_an_exact_tie_is_refused():
    s = scores_with_ties()
    with pytest.raises(AssertionError):
        M.check_topk(np.array([[9, 1, 5, 7]]), np.array([[0.6, 0.5, 0.5, 0.3]]), s, 4)


def test_exact_tie_in_the_wrong_order_is_refused():
    s = scores_with_ties()
    with pytest.raises(AssertionError):
        M.check_topk(np.array([[9, 5, 1, 3]]), np.array([[0.6, 0.5, 0.5, 0.3]]), s, 4)


def test_near_tie_window_accepts_either_member():
    s = np.array([[0.5, 0.3, 0.3 - 5e-5, 0.1]])
    M.check_topk(np.array([[0, 2]]), np.array([[0.5, 0.3 - 5e-5]]), s, 2)
    M.check_topk(np.array([[0, 1]]), np.array([[0.5, 0.3]]), s, 2)
    with pytest.raises(AssertionError):  # outside the window
        M.check_topk(np.array([[0, 3]]), np.array([[0.5, 0.1]]), s, 2)


def test_clear_gap_needs_the_exact_set():
    s = np.array([[0.5, 0.3, 0.2, 0.1]])
    with pytest.raises(AssertionError):
        M.check_topk(np.array([[0, 2]]), np.array([[0.5, 0.2]]), s, 2)
