"""The e-book's analytic numbers: expected tokens, default-parameter speedup,
the gamma sweep and where its peak moves."""
import pytest

import oracle


def test_default_parameters():
    E = oracle.expected_tokens(0.8, 4)
    assert E == pytest.approx(1 + 0.8 + 0.64 + 0.512 + 0.4096, abs=1e-15)
    assert round(E, 3) == 3.362
    cost = 4 * 0.10 + 1.00
    assert round(cost, 2) == 1.40
    assert round(oracle.speedup(0.8, 4, 0.10, 1.00), 2) == 2.40
    assert round(cost / E, 3) == 0.416          # target passes per token
    assert round(E / (1 / (1 - 0.8)), 3) == 0.672  # fraction of the ceiling


def test_guessing_further():
    assert round(oracle.expected_tokens(0.8, 32), 3) == 4.997
    assert round(32 * 0.10 + 1.00, 2) == 4.20
    assert round(oracle.speedup(0.8, 32, 0.10, 1.00), 2) == 1.19
    assert oracle.best_gamma(0.8, 0.10, 1.00) == 6
    assert round(oracle.speedup(0.8, 6, 0.10, 1.00), 2) == 2.47


@pytest.mark.parametrize("alpha,peak", [(0.4, 2), (0.8, 6), (0.9, 10), (0.95, 15)])
def test_peak_moves_right_with_alpha(alpha, peak):
    assert oracle.best_gamma(alpha, 0.10, 1.00) == peak


@pytest.mark.parametrize("c_draft,peak", [(0.01, 14), (0.10, 6), (0.25, 3), (0.99, 0)])
def test_peak_moves_left_with_draft_cost(c_draft, peak):
    assert oracle.best_gamma(0.8, c_draft, 1.00) == peak


def test_free_draft_and_costly_verify():
    assert oracle.best_gamma(0.8, 0.0, 1.00) == 32
    assert round(oracle.speedup(0.8, 32, 0.0, 1.00), 2) == 5.00
    assert oracle.best_gamma(0.8, 0.10, 1.50) == 7


def test_ceiling_and_special_cases():
    assert oracle.expected_tokens(1.0, 4) == 5.0
    assert oracle.expected_tokens(0.0, 4) == 1.0
    assert oracle.expected_tokens(0.3, 0) == 1.0
    assert oracle.expected_tokens(0.8, 400) == pytest.approx(5.0, abs=1e-12)
