"""Pins of the speculative-sampling oracle (oracle/specsample.py).

* The e-book's toy pair: the surviving mass min(p, q) sums to 0.90, the
  rejection probability and the raw residual's total are both 0.10, the
  first token's residual normalises to 1, its output is 0.4 + 0.10 x 1 = 0.5
  = p, and the output column equals p on every row.
* The identity output = p holds exactly (to float64 rounding) for 729
  self-generated pairs of distributions (the page's 729 are not given),
  including pairs with zeros and p = q.
* Counting the rule's outputs over a fine grid of (u_accept, u_resample) for
  a draft drawn from q by a third grid coordinate reproduces p to the grid's
  resolution: the sampler itself, not only its formula, is exact.
* The acceptance probability is sum min(p, q) (0.90 for the toy pair) over a
  fine grid of uniforms, and a round returns the drafts before the first
  rejection and then one token (planted uniforms).
"""
import numpy as np

from oracle.specsample import TOY_P, TOY_Q, output_distribution, residual, speculative_sample_chain
from oracle.typical import sample_token


def test_toy_pair_columns():
    keep = np.minimum(TOY_P, TOY_Q)
    assert np.allclose(keep, [0.4, 0.25, 0.15, 0.10], atol=1e-15)
    assert abs(keep.sum() - 0.90) < 1e-12
    raw = np.maximum(0.0, TOY_P - TOY_Q)
    assert abs(raw.sum() - 0.10) < 1e-12 and abs((1 - keep.sum()) - 0.10) < 1e-12
    assert np.allclose(residual(TOY_P, TOY_Q), [1.0, 0.0, 0.0, 0.0], atol=1e-12)
    out = output_distribution(TOY_P, TOY_Q)
    assert abs(out[0] - (0.4 + 0.10 * 1.0)) < 1e-12 and abs(out[0] - 0.5) < 1e-12
    assert np.allclose(out, TOY_P, atol=1e-12)


def test_output_equals_target_on_729_pairs():
    r = np.random.default_rng(729)
    for k in range(729):
        V = 2 + k % 9
        p = r.dirichlet(np.full(V, 0.5))
        q = r.dirichlet(np.full(V, 0.5))
        if k % 27 == 0:
            p[r.integers(0, V)] = 0.0
            p /= p.sum()
        if k % 81 == 0:
            q = p.copy()
        assert np.allclose(output_distribution(p, q), p, atol=1e-12), k


def test_sampler_counts_reproduce_the_target():
    """Drafts x ~ q (grid over its inverse transform), acceptance and resample
    uniforms on grids: the output frequencies match p to the grids' resolution."""
    p, q = TOY_P, TOY_Q
    MA, MC = 120, 40
    counts = np.zeros(4)
    for a in range(MA):
        x = sample_token(q, (a + 0.5) / MA)
        for b in range(MA):
            ua = (b + 0.5) / MA
            for c in range(MC):
                n, toks = speculative_sample_chain(np.stack([p, p]), q[None], [x], [ua], [(c + 0.5) / MC, 0.5])
                if n == 1:        # accepted: the position's output is the draft for every resample point
                    counts[toks[0]] += MC
                    break
                counts[toks[0]] += 1
    freq = counts / (MA * MA * MC)
    assert np.allclose(freq, p, atol=0.02), freq


def test_acceptance_rate_is_the_overlap_and_the_chain_stops_at_the_first_rejection():
    """P(accept) = sum_x q(x) min(1, p/q) = sum min(p, q) (the e-book's 0.90 for
    the toy pair), hence (1 - alpha^(g+1)) / (1 - alpha) tokens per round;
    and a round returns the drafts before the first rejection, then one token."""
    p, q = TOY_P, TOY_Q
    M = 20000
    acc = 0.0
    for x in range(4):
        ua = (np.arange(M) + 0.5) / M
        hits = sum(1 for u in ua if speculative_sample_chain(np.stack([p, p]), q[None], [x], [u], [0.5, 0.5])[0] == 1)
        acc += q[x] * hits / M
    assert abs(acc - 0.90) < 1e-3
    gamma = 4
    assert abs((1 - acc ** (gamma + 1)) / (1 - acc) - 4.0951) < 0.01
    # drafts 0, 0, 1, 0: u planted to accept, accept, reject (token 1: p/q = 0.25/0.3 < 0.9), -
    P4, Q4 = np.tile(p, (5, 1)), np.tile(q, (4, 1))
    n, toks = speculative_sample_chain(P4, Q4, [0, 0, 1, 0], [0.99, 0.5, 0.9, 0.1], [0.3, 0.3, 0.7, 0.3, 0.3])
    assert n == 2 and toks[:2] == [0, 0] and toks[2] == 0   # the residual after a rejection is all on token 0
    n, toks = speculative_sample_chain(P4, Q4, [0, 0, 1, 0], [0.1, 0.1, 0.1, 0.1], [0.3, 0.3, 0.3, 0.3, 0.7])
    assert n == 4 and toks[:4] == [0, 0, 1, 0] and toks[4] == sample_token(p, 0.7) == 1
