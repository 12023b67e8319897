"""Pins of the oracle's tree attention (a4).

Tree attention lets each candidate see only its ancestors, so every
root-to-leaf branch must give exactly what plain causal attention over
prefix + branch gives.  The causal reference is torch's library routine
(scaled_dot_product_attention, float64, CPU)."""
import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle


def _inputs(tree, B, nH, nKV, D, P, seed):
    r = np.random.default_rng(seed)
    N = tree.n
    Lmax = max(P) + N + 3
    return dict(q=r.normal(0, 1, (B, N, nH, D)), k_tree=r.normal(0, 1, (B, N, nKV, D)),
                v_tree=r.normal(0, 1, (B, N, nKV, D)), k_cache=r.normal(0, 1, (B, nKV, Lmax, D)),
                v_cache=r.normal(0, 1, (B, nKV, Lmax, D)), cache_len=np.asarray(P))


def _causal_sdpa(q, k, v, scale):
    """q [T][nH][D], k/v [T][nKV][D] (GQA by repetition) -> [T][nH][D]."""
    nH, nKV = q.shape[1], k.shape[1]
    rep = nH // nKV
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2).contiguous()
    tv = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("tree,nH,nKV,P", [(mi.tiny_tree(), 4, 4, (7, 0)), (mi.tiny_tree(), 4, 2, (3, 9)),
                                           (mi.sparse_tree(64), 2, 1, (5,)), (mi.chain_tree(6), 2, 2, (4,))])
def test_every_branch_equals_causal_attention(tree, nH, nKV, P):
    D = 8
    B = len(P)
    x = _inputs(tree, B, nH, nKV, D, P, 0)
    parent, _ = tree.arrays()
    scale = 1 / np.sqrt(D)
    o = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                              x["cache_len"], parent, scale)
    leaves = [i for i in range(tree.n) if i not in set(parent.tolist())]
    for b in range(B):
        Pb = P[b]
        for leaf in leaves:
            path = []
            j = leaf
            while j >= 0:
                path.append(j)
                j = parent[j] if j > 0 else -1
            path = path[::-1]
            # sequence = prefix tokens then the branch; queries only on the branch
            kseq = np.concatenate([np.transpose(x["k_cache"][b, :, :Pb], (1, 0, 2)), x["k_tree"][b, path]])
            vseq = np.concatenate([np.transpose(x["v_cache"][b, :, :Pb], (1, 0, 2)), x["v_tree"][b, path]])
            qseq = np.concatenate([np.zeros((Pb, nH, D)), x["q"][b, path]])
            ref = _causal_sdpa(qseq, kseq, vseq, scale)[Pb:]
            np.testing.assert_allclose(o[b, path], ref, rtol=1e-12, atol=1e-12)


def test_single_visible_key_returns_its_value():
    tree = mi.chain_tree(0)
    x = _inputs(tree, 1, 2, 2, 4, (0,), 1)
    o = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                              np.array([0]), np.array([-1]), 0.5)
    np.testing.assert_allclose(o[0, 0], x["v_tree"][0, 0], rtol=0, atol=1e-15)


def test_zero_query_averages_visible_values():
    tree = mi.tiny_tree()
    x = _inputs(tree, 1, 2, 2, 4, (5,), 2)
    x["q"][:] = 0
    parent, _ = tree.arrays()
    o = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                              x["cache_len"], parent, 0.5)
    anc = oracle.ancestor_matrix(parent)
    for i in range(tree.n):
        vis = np.concatenate([x["v_cache"][0, :, :5], np.transpose(x["v_tree"][0, anc[i]], (1, 0, 2))], axis=1)
        np.testing.assert_allclose(o[0, i], vis.mean(axis=1), rtol=0, atol=1e-14)


def test_cache_slots_beyond_prefix_are_ignored():
    tree = mi.tiny_tree()
    x = _inputs(tree, 1, 2, 2, 4, (6,), 3)
    parent, _ = tree.arrays()
    o1 = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                               x["cache_len"], parent, 0.5)
    x["k_cache"][:, :, 6:] = 1e6
    x["v_cache"][:, :, 6:] = np.nan
    o2 = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                               x["cache_len"], parent, 0.5)
    assert np.array_equal(o1, o2)


def test_write_tree_kv_places_nodes_at_prefix_end():
    tree = mi.tiny_tree()
    x = _inputs(tree, 2, 2, 2, 4, (3, 6), 4)
    kc, vc = oracle.write_tree_kv(x["k_cache"], x["v_cache"], x["k_tree"], x["v_tree"], x["cache_len"])
    for b, P in enumerate((3, 6)):
        for i in range(tree.n):
            assert np.array_equal(kc[b, :, P + i], x["k_tree"][b, i])
            assert np.array_equal(vc[b, :, P + i], x["v_tree"][b, i])
        assert np.array_equal(kc[b, :, :P], x["k_cache"][b, :, :P])
