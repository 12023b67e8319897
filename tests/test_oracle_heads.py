"""Pins of the oracle's heads (a1/a2) and top-k against what the pages fix and
closed forms (no test re-types the oracle's own formula)."""
import math

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_zero_init_heads_reproduce_lm_head_exactly():
    # The heads page's sketch: 256 hidden, 1000 vocab, 3 heads, W1 and b1 zero,
    # W2 copied from lm_head; it prints [True, True, True] for exact equality.
    H, V, K = 256, 1000, 3
    r = _rng(0)
    lm_head = r.normal(0, 0.02, (V, H))
    W1 = np.zeros((K, H, H))
    b1 = np.zeros((K, H))
    W2 = np.stack([lm_head.copy() for _ in range(K)])
    h = r.normal(0, 1, (1, H))
    logits, z = oracle.medusa_heads(h, W1, b1, W2)
    base = oracle.lm_head_logits(h, lm_head)
    assert [bool(np.array_equal(logits[:, k, :], base)) for k in range(K)] == [True, True, True]
    assert np.array_equal(z[:, 0, :], h)


def test_unit_hidden_state_selects_a_column():
    H, V, K = 16, 40, 2
    r = _rng(1)
    W2 = r.normal(0, 1, (K, V, H))
    for j in (0, 5, 15):
        h = np.zeros((1, H)); h[0, j] = 1.0
        logits, _ = oracle.medusa_heads(h, np.zeros((K, H, H)), np.zeros((K, H)), W2)
        for k in range(K):
            assert np.array_equal(logits[0, k], W2[k][:, j])


def test_constant_bias_shift_closed_form():
    # W1 = 0, b1 = ln 3 everywhere: SiLU(ln 3) = ln 3 * sigmoid(ln 3) = 0.75 ln 3,
    # so z = h + 0.75 ln 3 and logits = W2 h + 0.75 ln 3 * rowsum(W2).
    H, V, K = 8, 12, 2
    r = _rng(2)
    W2 = r.normal(0, 1, (K, V, H))
    h = r.normal(0, 1, (3, H))
    b1 = np.full((K, H), math.log(3.0))
    logits, z = oracle.medusa_heads(h, np.zeros((K, H, H)), b1, W2)
    shift = 0.75 * math.log(3.0)
    np.testing.assert_allclose(z, np.repeat(h[:, None, :], K, axis=1) + shift, rtol=0, atol=1e-14)
    for k in range(K):
        np.testing.assert_allclose(logits[:, k], h @ W2[k].T + shift * W2[k].sum(1), rtol=0, atol=1e-12)


def test_w1_orientation_out_by_in():
    # W1[k][o][j] = w only: with h = e_j the pre-activation is w at output o
    # (a transposed W1 would put it at output j).
    H, K = 6, 1
    o_, j_, w = 4, 1, 2.0
    W1 = np.zeros((K, H, H)); W1[0, o_, j_] = w
    h = np.zeros((1, H)); h[0, j_] = 1.0
    _, z = oracle.medusa_heads(h, W1, np.zeros((K, H)), np.eye(H)[None])
    expect = h[0].copy(); expect[o_] += w / (1 + math.exp(-w))
    np.testing.assert_allclose(z[0, 0], expect, rtol=0, atol=1e-15)


def test_silu_matches_torch_and_identities():
    a = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.silu(a), torch.nn.functional.silu(torch.from_numpy(a)).numpy(),
                               rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(a) - oracle.silu(-a), a, rtol=0, atol=1e-12)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([-800.0]))[0] == 0.0


def test_heads_match_torch_module_composition():
    # The sketch's own composition out(h + F.silu(layer(h))) in float64 torch.
    H, V, K = 32, 50, 3
    r = _rng(3)
    W1, b1, W2 = r.normal(0, .3, (K, H, H)), r.normal(0, .3, (K, H)), r.normal(0, .3, (K, V, H))
    h = r.normal(0, 1, (2, H))
    logits, _ = oracle.medusa_heads(h, W1, b1, W2)
    th = torch.from_numpy(h)
    for k in range(K):
        lin1 = torch.nn.functional.linear(th, torch.from_numpy(W1[k]), torch.from_numpy(b1[k]))
        ref = torch.nn.functional.linear(th + torch.nn.functional.silu(lin1), torch.from_numpy(W2[k]))
        np.testing.assert_allclose(logits[:, k], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_topk_brute_force_with_ties():
    r = _rng(4)
    for _ in range(50):
        v = r.integers(0, 6, size=(3, 17)).astype(np.float64) * 0.25
        idx, val = oracle.topk(v, 5)
        for row in range(3):
            ref = sorted(range(17), key=lambda j: (-v[row, j], j))[:5]
            assert list(idx[row]) == ref
            assert list(val[row]) == [v[row, j] for j in ref]


def test_topk_decides_in_float32():
    # Two values that differ in float64 but round to the same float32 tie,
    # so the lower index wins.
    v = np.array([[1.0, 1.0 + 1e-12, 0.5]])
    idx, _ = oracle.topk(v, 2)
    assert list(idx[0]) == [0, 1]


def test_top2_by_top3_gives_six_candidates():
    # The tree section's example: top-2 of head 1 x top-3 of head 2.
    r = _rng(5)
    logits = r.normal(0, 1, (1, 2, 30))
    idx, _ = oracle.topk(logits, 3)
    t = mi.tiny_tree()
    parent, rank = t.arrays()
    node_tok, _, _ = oracle.build_tree(parent, rank, idx, np.array([7]), np.array([0]))
    leaves = [i for i in range(t.n) if t.depth[i] == 2]
    cands = {(int(node_tok[0, parent[i]]), int(node_tok[0, i])) for i in leaves}
    assert len(cands) == 6
    assert cands == {(int(a), int(b)) for a in idx[0, 0, :2] for b in idx[0, 1, :3]}
