"""Pins of the typical-acceptance oracle (oracle/typical.py).

* T -> 0: the base distribution becomes one-hot at the argmax (entropy 0, bar
  min(eps, delta) < 1), so typical acceptance must equal greedy acceptance
  (oracle.accept, pinned separately) on every tree, and the drawn extra token
  must be the argmax for every u.
* Flat distributions (all scores equal): p = 1/V and H = ln V, so the bar is
  min(eps, delta / V): every candidate is accepted iff delta < 1 (and eps >
  1/V), none if delta > 1.
* Inverse transform sampling over a fine grid of u reproduces the
  distribution's probabilities exactly (the counts of a grid of M points
  differ from M p by at most one per token).
* Entropy against closed forms (uniform: ln V; two-point: the binary entropy).
"""
import numpy as np
import pytest

import medusa_inputs as mi
import oracle
from oracle.typical import base_distribution, sample_token, typical_accept, typical_threshold


def _tree(name):
    return {"tiny": mi.tiny_tree(), "sparse64": mi.sparse_tree(64), "chain5": mi.chain_tree(5)}[name]


@pytest.mark.parametrize("name", ["tiny", "sparse64", "chain5"])
def test_zero_temperature_is_greedy_acceptance(name):
    parent, rank = _tree(name).arrays()
    N, V = len(parent), 12
    r = np.random.default_rng(5)
    for trial in range(20):
        logits = r.normal(0, 1, (N, V))
        greedy = logits.argmax(axis=1)
        # candidates: half the time the parent's argmax, else another token
        tok = np.where(r.random(N) < 0.6, greedy[np.maximum(parent, 0)], r.integers(0, V, N))
        tok[0] = 3
        want = oracle.accept(parent, tok, greedy)
        got = typical_accept(parent, tok, logits, 1e-4, 0.09, 0.3, float(r.random()))
        assert got[0] == want[0]
        assert np.array_equal(got[1], want[1])
        assert np.array_equal(got[2], want[2])


def test_flat_distributions_accept_everything_iff_delta_below_one():
    parent, rank = mi.sparse_tree(64).arrays()
    N, V = len(parent), 50
    tok = np.random.default_rng(2).integers(0, V, N)
    logits = np.full((N, V), 0.7)
    L, path, _ = typical_accept(parent, tok, logits, 1.0, 0.09, 0.3, 0.5)
    assert L == max(mi.sparse_tree(64).depth)
    L, path, toks = typical_accept(parent, tok, logits, 1.0, 0.09, 1.5, 0.51)
    assert L == 0 and list(path) == [0]
    # flat: the draw is uniform over the vocabulary (u = 0.51 falls in token 25's interval [0.50, 0.52))
    assert toks[-1] == 25


def test_entropy_closed_forms():
    V = 40
    _, H = base_distribution(np.zeros(V), 1.0)
    assert abs(H - np.log(V)) < 1e-12
    q = 0.3
    lg = np.array([np.log(q), np.log(1 - q)])
    p, H = base_distribution(lg, 1.0)
    assert np.allclose(p, [q, 1 - q], atol=1e-15)
    assert abs(H - (-(q * np.log(q) + (1 - q) * np.log(1 - q)))) < 1e-12
    # temperature 2 on logits 2 s is temperature 1 on s
    s = np.random.default_rng(1).normal(0, 1, 7)
    assert np.allclose(base_distribution(2 * s, 2.0)[0], base_distribution(s, 1.0)[0], atol=1e-15)
    assert typical_threshold(0.0, 0.09, 0.3) == 0.09
    assert abs(typical_threshold(np.log(100.0), 0.09, 0.3) - 0.003) < 1e-15


def test_inverse_transform_reproduces_the_distribution():
    p = np.array([0.1, 0.0, 0.25, 0.05, 0.6])
    M = 20000
    counts = np.bincount([sample_token(p, (k + 0.5) / M) for k in range(M)], minlength=len(p))
    assert np.all(np.abs(counts - M * p) <= 1)
    assert counts[1] == 0
    assert sample_token(p, 0.0) == 0 and sample_token(p, 0.0999) == 0 and sample_token(p, 0.1) == 2
    assert sample_token(p, 0.9999999) == 4
