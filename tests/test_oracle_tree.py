"""Pins of the oracle's tree build (a3): the Cartesian-product invariants of
the tree section."""
import numpy as np
import pytest

import medusa_inputs as mi
import oracle


def _topk_idx(B, K, k, V, seed):
    r = np.random.default_rng(seed)
    out = np.empty((B, K, k), dtype=np.int32)
    for b in range(B):
        for h in range(K):
            out[b, h] = r.choice(V, size=k, replace=False)
    return out


@pytest.mark.parametrize("tree,K,k", [(mi.tiny_tree(), 3, 3), (mi.sparse_tree(64), 5, 4),
                                      (mi.dense_tree(256), 5, 3), (mi.chain_tree(4), 4, 1)])
def test_tree_invariants(tree, K, k):
    parent, rank = tree.arrays()
    B = 3
    tk = _topk_idx(B, K, k, 1000, 0)
    root = np.array([11, 22, 33])
    P = np.array([0, 5, 100])
    tok, pos, mask = oracle.build_tree(parent, rank, tk, root, P)
    depth = np.asarray(tree.depth)
    for b in range(B):
        assert tok[b, 0] == root[b]
        np.testing.assert_array_equal(pos[b], P[b] + depth)
    # ancestor mask: self + ancestors, popcount = depth + 1, parent's row is a subset
    assert np.array_equal(mask.sum(1), depth + 1)
    for i in range(1, tree.n):
        assert mask[i, i] and mask[i, parent[i]]
        assert np.all(mask[i] >= mask[parent[i]])
        assert mask[i].sum() == mask[parent[i]].sum() + 1
    assert np.all(np.tril(mask) == mask)  # BFS order: ancestors precede
    # All heads read the same hidden state: head d proposes the same tokens
    # under every branch of depth d-1.
    for d in range(1, depth.max() + 1):
        for b in range(B):
            by_rank = {}
            for i in np.flatnonzero(depth == d):
                by_rank.setdefault(int(rank[i]), set()).add(int(tok[b, i]))
            for r_, toks in by_rank.items():
                assert toks == {int(tk[b, d - 1, r_])}
    # siblings carry distinct tokens
    for i in range(tree.n):
        kids = np.flatnonzero(parent == i)
        for b in range(B):
            assert len(set(tok[b, kids].tolist())) == len(kids)
