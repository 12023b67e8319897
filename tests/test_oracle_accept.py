"""Pins of the oracle's acceptance (a5 argmax, a6 accept, a7 compaction).

* the e-book's worked flag string (six rounds, 20 tokens, 14 of 18 accepted);
* Monte Carlo on a chain with independent acceptance alpha against the
  expected-tokens closed form, and its special cases;
* Monte Carlo on the sparse/dense trees under the synthetic rank prior against
  1 + sum over nodes of the product of priors;
* compaction against sequentially appending the accepted branch.
"""
import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle


def _chain_round(gamma, outcome, rng_tok):
    """Plant a chain round: position j (1..gamma) matches the base model's
    choice iff outcome[j-1]; returns (parent, node_tok, greedy)."""
    t = mi.chain_tree(gamma)
    parent, _ = t.arrays()
    tok = np.arange(100, 100 + gamma + 1, dtype=np.int32)
    g = np.empty(gamma + 1, dtype=np.int32)
    for j in range(1, gamma + 1):
        g[j - 1] = tok[j] if outcome[j - 1] else tok[j] + 1000
    g[gamma] = 5
    return parent, tok, g


def test_flag_string_worked_example():
    # gamma = 4, flags 111111001110101111: rounds accept 4,2,0,3,1,4 and yield
    # 5,3,1,4,2,5 tokens = 20 over 6 target passes; 14 of 18 flags are 1;
    # at draft cost 0.10 and verify cost 1.00 the rounds cost 8.40: 2.38x.
    flags, gamma = "111111001110101111", 4
    rounds = oracle.rounds_from_flags(flags, gamma)
    assert rounds == [4, 2, 0, 3, 1, 4]
    got, i = [], 0
    for a in rounds:
        read = flags[i:i + min(a + 1, gamma)]
        i += len(read)
        # after the first rejection the later positions are made to match
        # anyway: acceptance must still stop at the first mismatch
        outcome = [c == "1" for c in read] + [True] * (gamma - len(read))
        parent, tok, g = _chain_round(gamma, outcome, None)
        L, path, out = oracle.accept(parent, tok, g)
        assert len(out) == L + 1 and list(path) == list(range(L + 1))
        got.append(L)
    assert i == len(flags) == 18
    assert got == [4, 2, 0, 3, 1, 4]
    tokens = [L + 1 for L in got]
    assert tokens == [5, 3, 1, 4, 2, 5] and sum(tokens) == 20
    cost = len(got) * (gamma * 0.10 + 1.00)
    assert round(cost, 2) == 8.40 and round(sum(tokens) / cost, 2) == 2.38
    assert sum(got) == 14 and round(sum(got) / 18, 3) == 0.778


def _mc_chain(alpha, gamma, n, seed):
    r = np.random.default_rng(seed)
    parent = mi.chain_tree(gamma).arrays()[0]
    tok = np.arange(gamma + 1, dtype=np.int32) + 7
    draws = r.random((n, max(gamma, 1))) < alpha
    tot = 0
    for t in range(n):
        g = np.where(draws[t, :gamma], tok[1:], tok[1:] + 99) if gamma else np.zeros(0, np.int32)
        g = np.append(g, 0).astype(np.int32)
        L, _, out = oracle.accept(parent, tok, g)
        tot += len(out)
    return tot / n


def test_monte_carlo_chain_matches_expected_tokens():
    alpha, gamma, n = 0.8, 4, 200_000
    mean = _mc_chain(alpha, gamma, n, 0)
    E = oracle.expected_tokens(alpha, gamma)
    assert abs(E - 3.3616) < 1e-12
    # exact variance of L+1: P(L+1 >= m) = alpha^(m-1), m = 1..gamma+1
    E2 = sum((2 * m - 1) * alpha ** (m - 1) for m in range(1, gamma + 2))
    sigma = np.sqrt((E2 - E * E) / n)
    assert abs(mean - E) < 5 * sigma, (mean, E, sigma)


def test_special_cases_alpha_one_zero_gamma_zero():
    assert _mc_chain(1.0, 4, 200, 1) == 5.0 == oracle.expected_tokens(1.0, 4)
    assert _mc_chain(0.0, 4, 200, 2) == 1.0 == oracle.expected_tokens(0.0, 4)
    assert _mc_chain(0.7, 0, 200, 3) == 1.0 == oracle.expected_tokens(0.7, 0)


@pytest.mark.parametrize("tree,k", [(mi.sparse_tree(64), 4), (mi.dense_tree(256), 3)])
def test_monte_carlo_tree_prior(tree, k):
    """Plant the base model's choice at each depth as the head's rank-R token
    with P(R = r) = alpha (1-alpha)^r (r < k), else a token outside the top-k.
    Exactly one path can be accepted, so E[L+1] = 1 + sum_nodes prod prior."""
    alpha, n = 0.8, 20_000
    parent, rank = tree.arrays()
    depth = np.asarray(tree.depth)
    N, K = tree.n, depth.max()
    closed = 1 + sum(np.prod([mi.rank_prior(alpha, r) for r in p]) for p in tree.paths[1:])
    r = np.random.default_rng(7)
    pr = np.array([mi.rank_prior(alpha, j) for j in range(k)] + [1 - sum(mi.rank_prior(alpha, j) for j in range(k))])
    truth = r.choice(k + 1, size=(n, K), p=pr)
    tk = (np.arange(K * k).reshape(1, K, k) + 10).astype(np.int32)
    tok, _, _ = oracle.build_tree(parent, rank, tk, np.array([1]), np.array([0]))
    tok = tok[0]
    tot, tot2 = 0, 0
    for t in range(n):
        g = np.zeros(N, dtype=np.int32)
        for i in range(N):
            d = depth[i]
            if d < K:
                R = truth[t, d]
                g[i] = tk[0, d, R] if R < k else 9999
        L, path, out = oracle.accept(parent, tok, g)
        assert [int(rank[p]) for p in path[1:]] == list(truth[t, :L])
        tot += L + 1
        tot2 += (L + 1) ** 2
    mean = tot / n
    sd = np.sqrt((tot2 / n - mean ** 2) / n)
    assert abs(mean - closed) < 5 * sd, (mean, closed, sd)


def test_base_greedy_brute_force_and_rmsnorm():
    r = np.random.default_rng(8)
    o = r.normal(0, 1, (6, 32))
    lm = r.normal(0, 0.02, (50, 32))
    g, logits = oracle.base_greedy(o, lm, 1e-6)
    # RMS of each row by a plain loop, then the scores through torch
    n = np.stack([row / np.sqrt(sum(float(x) * float(x) for x in row) / len(row) + 1e-6) for row in o])
    ref = torch.from_numpy(n) @ torch.from_numpy(lm).T
    np.testing.assert_allclose(logits, ref.numpy(), rtol=1e-12, atol=1e-13)
    for row in range(6):
        lg = logits[row].astype(np.float32)
        best = max(range(50), key=lambda j: (lg[j], -j))
        assert g[row] == best
    # unit-weight RMSNorm is a positive factor per row: the top choice is that of lm_head . o, and
    # scaling a row by any positive constant changes nothing
    raw = o @ lm.T
    assert np.array_equal(g, np.argmax(raw, axis=1))
    g2, _ = oracle.base_greedy(o * np.array([[3.0], [0.01], [7.5], [1.0], [250.0], [0.5]]), lm, 0.0)
    g0, _ = oracle.base_greedy(o, lm, 0.0)
    assert np.array_equal(g2, g0)
    # RMSNorm: unit mean square (up to eps), scale invariant
    n = oracle.rmsnorm(o, 0.0)
    np.testing.assert_allclose((n * n).mean(1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(o * 37.0, 0.0), n, rtol=1e-13)
    # ties go to the lower index
    g, _ = oracle.base_greedy(np.ones((1, 4)), np.ones((5, 4)), 1e-6)
    assert g[0] == 0


def test_accept_one_accepted_node_per_depth_random():
    r = np.random.default_rng(9)
    tree = mi.sparse_tree(64)
    parent, rank = tree.arrays()
    depth = np.asarray(tree.depth)
    for _ in range(300):
        tk = r.integers(0, 6, size=(1, 5, 4)).astype(np.int32)
        for h in range(5):
            tk[0, h] = r.permutation(6)[:4]
        tok, _, _ = oracle.build_tree(parent, rank, tk, np.array([0]), np.array([0]))
        g = r.integers(0, 6, size=64).astype(np.int32)
        L, path, out = oracle.accept(parent, tok[0], g)
        # brute force: the deepest node whose whole chain matches
        best = 0
        for i in range(64):
            j, ok = i, True
            while j > 0:
                ok &= tok[0, j] == g[parent[j]]
                j = parent[j]
            if ok:
                best = max(best, depth[i])
        assert L == best
        assert out[-1] == g[path[-1]]


def test_compaction_equals_sequential_append():
    r = np.random.default_rng(10)
    tree = mi.sparse_tree(64)
    parent, _ = tree.arrays()
    depth = np.asarray(tree.depth)
    nKV, D, P = 2, 3, 5
    for leaf in [0, 1, 5, 23, 63]:
        path = []
        j = leaf
        while j >= 0:
            path.append(j)
            j = parent[j] if j > 0 else -1
        path = path[::-1]
        cache = r.normal(0, 1, (nKV, P + 64 + 2, D))
        k_tree = r.normal(0, 1, (1, 64, nKV, D))
        kc, _ = oracle.write_tree_kv(cache[None], cache[None], k_tree, k_tree, np.array([P]))
        out, newP = oracle.compact_kv(kc[0], P, np.array(path))
        assert newP == P + depth[leaf] + 1
        # sequential append of the branch's keys after the prefix
        ref = cache[:, :P].copy()
        for n_ in path:
            ref = np.concatenate([ref, k_tree[0, n_][:, None, :]], axis=1)
        assert np.array_equal(out[:, :newP], ref)


def test_compaction_overlap_reads_before_writes():
    # path [0, 2, 5]: slot P+1 <- P+2 and slot P+2 <- P+5; a descending
    # in-place copy would read an overwritten slot
    cache = np.arange(10, dtype=np.float64).reshape(1, 10, 1)
    out, newP = oracle.compact_kv(cache, 1, np.array([0, 2, 5]))
    assert newP == 4
    assert out[0, :, 0].tolist() == [0, 1, 3, 6, 4, 5, 6, 7, 8, 9]
