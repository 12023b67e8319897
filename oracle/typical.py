"""Float64 oracle of typical acceptance, the sampling-mode acceptance rule --
TEST INFRASTRUCTURE ONLY (imported by tests/ alone, never by the product path).

[MH-tree]: under sampling, Medusa keeps any candidate whose probability under
the base model exceeds a threshold tied to the entropy of the base model's
distribution; it accepts more tokens and gives up matching the distribution
exactly.

Readings taken (the page names the rule, not its form):

* the base distribution after a node is softmax(logits / T) at the sampling
  temperature T;
* the threshold after a node is min(eps, delta * exp(-H)), H the entropy (in
  nats) of that distribution: exp(-H) is the probability of a typical draw
  (one over the perplexity), so a flat distribution lowers the bar and a
  peaked one raises it, capped at eps;
* a candidate is accepted when its parent was and its probability after the
  parent exceeds the parent's threshold (strictly); the kept branch is the
  deepest accepted node's, the lowest node index among equally deep ones (as
  in greedy acceptance);
* the round's extra token is drawn from the base distribution after the
  deepest accepted node by inverse transform sampling with a given uniform u
  in [0, 1): the smallest token index whose cumulative probability (tokens in
  index order) exceeds u.

Pins (tests/test_oracle_typical.py): as T -> 0 the rule is greedy acceptance
(the distribution becomes one-hot at the argmax and the extra token is the
argmax for every u); on flat distributions the closed form p = 1/V > delta/V
accepts every candidate iff delta < 1; the draw's frequencies over a grid of
u equal the distribution exactly.
"""
from __future__ import annotations

import numpy as np

from .medusa import tree_depths

__all__ = ["base_distribution", "typical_threshold", "sample_token", "typical_accept"]


def base_distribution(logits, temperature):
    """softmax(logits / T) over the last axis, and its entropy in nats."""
    z = np.asarray(logits, dtype=np.float64) / temperature
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        H = -np.sum(np.where(p > 0, p * np.log(p), 0.0), axis=-1)
    return p, H


def typical_threshold(H, eps, delta):
    """The acceptance bar after a node: min(eps, delta * exp(-H))."""
    return np.minimum(eps, delta * np.exp(-np.asarray(H)))


def sample_token(p, u):
    """Inverse transform sampling: the smallest index j with
    p[0] + .. + p[j] > u (u in [0, 1)); the last index if rounding leaves
    the total at or below u."""
    c = np.cumsum(p)
    j = int(np.searchsorted(c, u, side="right"))
    return min(j, len(p) - 1)


def typical_accept(parent, node_tok, logits, temperature, eps, delta, u):
    """Typical acceptance over one sequence's tree.

    parent [N]; node_tok [N]; logits [N][V] (the base model's scores after
    every node); u the uniform that draws the extra token.
    -> L, path [L+1] (node ids, path[0] = 0), out_tokens [L+1] (the L
    accepted candidates, then the drawn token)"""
    parent = np.asarray(parent)
    N = len(parent)
    depth = tree_depths(parent)
    p, H = base_distribution(logits, temperature)
    thr = typical_threshold(H, eps, delta)
    acc = np.zeros(N, dtype=bool)
    acc[0] = True
    for i in range(1, N):
        a = parent[i]
        acc[i] = acc[a] and p[a, node_tok[i]] > thr[a]
    L = int(depth[acc].max())
    deepest = int(np.flatnonzero(acc & (depth == L))[0])
    path = []
    j = deepest
    while j >= 0:
        path.append(j)
        j = parent[j] if j > 0 else -1
    path = path[::-1]
    tokens = [int(node_tok[n]) for n in path[1:]] + [sample_token(p[deepest], u)]
    return L, np.asarray(path, dtype=np.int32), np.asarray(tokens, dtype=np.int32)
