"""The host reference of the planted continuation (the measurement aid that
stands in for a trained base model's agreement with the heads) draws ranks
with the prior it claims: accepted tokens per round average the analytic
1 + sum over nodes of the product of alpha (1 - alpha)^rank along the path
(5.699 for the sparse 64-node tree at alpha = 0.8), and a draw outside the
top-k never matches a candidate."""
import numpy as np

import medusa_inputs as mi
import oracle
from medusa_testlib import planted_greedy_ref


def _expected_tokens(tree, alpha):
    parent, rank = tree.arrays()
    depth = np.asarray(tree.depth)
    e = 1.0
    for i in range(1, tree.n):
        p, j = 1.0, i
        while j > 0:
            p *= alpha * (1 - alpha) ** rank[j]
            j = parent[j]
        e += p
    return e


def test_planted_continuation_accepts_at_the_prior_rate():
    tree = mi.sparse_tree(64)
    parent, rank = tree.arrays()
    K, topk, V, B = 5, 4, 32000, 3000
    r = np.random.default_rng(3)
    tk = np.stack([np.stack([r.choice(V, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    P = r.integers(0, 100000, B)
    g = planted_greedy_ref(tree.depth, tk, P, 0.8, 12345, V)
    root = np.zeros(B, dtype=np.int32)
    tok, _, _ = oracle.build_tree(parent, rank, tk, root, P)
    L = np.array([oracle.accept(parent, tok[b], g[b])[0] for b in range(B)])
    want = _expected_tokens(tree, 0.8)
    assert abs(want - 5.699) < 5e-4
    # E[L + 1] within 5 standard errors of the analytic value
    se = np.std(L + 1) / np.sqrt(B)
    assert abs(np.mean(L + 1) - want) < 5 * se, (np.mean(L + 1), want, se)


def test_outside_draws_miss_the_top_k():
    K, topk, V = 3, 4, 50
    r = np.random.default_rng(4)
    tk = np.stack([np.stack([r.choice(V, topk, replace=False) for _ in range(K)]) for _ in range(400)]).astype(np.int32)
    depth = np.array([0, 1, 2, 3])
    g = planted_greedy_ref(depth, tk, np.arange(400), 0.3, 7, V)     # alpha 0.3: many draws outside
    for b in range(400):
        for d in range(K):
            rank_hit = [j for j in range(topk) if tk[b, d, j] == g[b, d]]
            assert len(rank_hit) <= 1
    # alpha = 1: always the rank-0 guess; alpha = 0: never a guess
    g1 = planted_greedy_ref(depth, tk, np.arange(400), 1.0, 7, V)
    assert np.array_equal(g1[:, :K], tk[:, :, 0])
    g0 = planted_greedy_ref(depth, tk, np.arange(400), 0.0, 7, V)
    for b in range(400):
        for d in range(K):
            assert g0[b, d] not in tk[b, d]
