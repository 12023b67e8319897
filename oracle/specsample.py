"""Float64 oracle of the speculative-sampling rule on a chain of drafts --
TEST INFRASTRUCTURE ONLY (imported by tests/ alone, never by the product path).

[SD-exact] (the e-book's section on being faster with the output unchanged):
a token x drawn from the draft distribution q is accepted with probability
min(1, p(x) / q(x)), p the target distribution; on a rejection the token is
drawn again from the residual max(0, p - q), normalised.  The output is then
distributed exactly as p, position by position: the mass that survives the
acceptance is min(p, q), and the residual's total equals the rejection
probability 1 - sum min(p, q) (both sum to one).  [SD-k+1]: a round of gamma
drafts yields the accepted prefix plus one more token; when every draft is
accepted that token comes from the target's next distribution.

Readings taken: the random draws are inputs (u_accept[i] decides draft i by
u q(x) < p(x), which is u < min(1, p/q) for q(x) > 0 and accepts any x with
p(x) > 0 when q(x) = 0; u_resample[i] draws the token after a rejection at i,
or the bonus token at i = gamma); draws use inverse transform sampling in
token-index order (oracle/typical.py's sample_token).  The toy pair's q is
not recoverable from the garbled table beyond q(first) = 0.4 and q >= p
elsewhere; q = (0.4, 0.3, 0.2, 0.1) is taken.
"""
from __future__ import annotations

import numpy as np

from .typical import sample_token

__all__ = ["residual", "output_distribution", "speculative_sample_chain", "TOY_P", "TOY_Q"]

# the e-book's four-token toy pair (rain, sun, wind, storm): p printed; q reading above
TOY_P = np.array([0.5, 0.25, 0.15, 0.10])
TOY_Q = np.array([0.4, 0.3, 0.2, 0.1])


def residual(p, q):
    """max(0, p - q), normalised (zeros if p <= q everywhere)."""
    r = np.maximum(0.0, np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64))
    t = r.sum()
    return r / t if t > 0 else r


def output_distribution(p, q):
    """The distribution of one position's output under the rule: the draft's
    surviving mass min(p, q) plus the rejection probability times the
    normalised residual."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    keep = np.minimum(p, q)
    return keep + (1.0 - keep.sum()) * residual(p, q)


def speculative_sample_chain(p, q, drafts, u_accept, u_resample):
    """One round on a chain of gamma drafts.

    p [gamma+1][V] target distributions (row i: after the first i drafts);
    q [gamma][V] draft distributions; drafts [gamma]; u_accept [gamma];
    u_resample [gamma+1].
    -> (n accepted, tokens [n+1]: the accepted drafts, then the redrawn or
    bonus token)"""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    gamma = len(drafts)
    for i in range(gamma):
        x = int(drafts[i])
        if not u_accept[i] * q[i, x] < p[i, x]:
            return i, [int(t) for t in drafts[:i]] + [sample_token(residual(p[i], q[i]), u_resample[i])]
    return gamma, [int(t) for t in drafts] + [sample_token(p[gamma], u_resample[gamma])]
