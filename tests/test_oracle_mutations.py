"""The position and score-orientation pins catch the slips they are meant to.

Each case plants a plausible mistake in the oracle (on the CPU, through
monkeypatch) and checks that at least one pin then fails: swapped h and w
fields, a row index taken as i // G_h, a transposed score grid, and swapped
query/key arguments of the score step.
"""
import numpy as np
import pytest

from oracle import rola as R
from tests import test_oracle_pins as P


def _positions_swapped_hw(grid, n):
    gt, gh, gw = grid
    i = np.arange(n)
    return np.stack([i // (gh * gw), i % gw, (i // gw) % gh], axis=1)


def _positions_row_by_gh(grid, n):
    gt, gh, gw = grid
    i = np.arange(n)
    return np.stack([i // (gh * gw), (i // gh) % gh, i % gw], axis=1)


def _positions_width_major(grid, n):
    gt, gh, gw = grid
    i = np.arange(n)
    return np.stack([i // (gh * gw), i % gh, (i // gh) % gw], axis=1)


POSITION_PINS = [P.test_o1_token_positions_by_hand, P.test_o1_positions_of_the_720p_latent_grid_by_hand]
SCORE_PINS = [P.test_o3_pooled_scores_by_hand_are_query_rows_key_columns,
              P.test_o3_asymmetric_scores_against_explicit_loops,
              P.test_o3_o4_top1_of_the_hybrid_follows_the_query_rows]


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("slip", [_positions_swapped_hw, _positions_row_by_gh, _positions_width_major])
def test_position_slips_are_caught(monkeypatch, slip):
    assert not _some_pin_fails(POSITION_PINS)
    monkeypatch.setattr(R, "token_positions", slip)
    assert _some_pin_fails(POSITION_PINS)


def test_transposed_score_grid_is_caught(monkeypatch):
    assert not _some_pin_fails(SCORE_PINS)
    orig = R.pooled_scores
    monkeypatch.setattr(R, "pooled_scores", lambda qbar, kbar: orig(qbar, kbar).T)
    assert _some_pin_fails(SCORE_PINS)


def test_swapped_score_arguments_in_the_hybrid_are_caught(monkeypatch):
    orig = R.pooled_scores
    monkeypatch.setattr(R, "pooled_scores", lambda qbar, kbar: orig(kbar, qbar))
    with pytest.raises(AssertionError):
        P.test_o3_o4_top1_of_the_hybrid_follows_the_query_rows()
