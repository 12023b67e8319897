"""Pins of the oracle's whole-step composition (``oracle.medusa_step``) and of
its number formats (``oracle.widen``, ``oracle.round_bf16``) against
implementations that share nothing with it:

* the step is recomposed here from torch float64 operations, each step taken
  from the pages as this test reads them: the heads as ``F.linear`` + ``F.silu``
  + residual ("Medusa Heads", section on how the heads predict later tokens),
  the candidates as the Cartesian product of the heads' top guesses and the
  verification as one causal attention per root-to-leaf branch with
  ``F.scaled_dot_product_attention`` (section on tree attention and
  acceptance: a tree token sees the prefix and its ancestors, i.e. exactly the
  causal view of its own branch), the base choice as ``argmax`` of lm_head
  over the normalised row, the longest accepted branch by walking from the
  root, and the cache hand-off as the sequential append of that branch's
  keys/values after the prefix;
* bf16 <-> fp32 conversion against torch's own ``bfloat16`` casts, over every
  bf16 bit pattern and over rounding ties, overflow, subnormals and NaN.

A slip in the composition (compacting the cache before the tree's keys are
written, skipping the bf16 rounding of the attention output before the greedy
choice, taking the bonus from the wrong node, reading the wrong head's top-k)
makes one of these fail.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import medusa_inputs as mi
import oracle
from medusa_testlib import make_workload, widen_inputs


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def _torch_bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).to(torch.float64).numpy()


def _same(a, b):
    """Equal values, NaN where NaN, and the same sign of zero."""
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    m = ~np.isnan(a)
    assert np.array_equal(a[m], b[m])
    assert np.array_equal(np.signbit(a[m]), np.signbit(b[m]))


def test_widen_bf16_matches_torch_on_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    _same(oracle.widen(bits, "bf16"), _torch_bf16_bits_to_f64(bits))


def test_widen_f32_is_exact():
    r = np.random.default_rng(1)
    x = np.concatenate([(r.standard_normal(1000) * 10.0 ** r.integers(-30, 30, 1000)).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, 3.4028235e38], dtype=np.float32)])
    _same(oracle.widen(x, "f32"), torch.from_numpy(x).to(torch.float64).numpy())


def _ties_and_edges() -> np.ndarray:
    """float32 values at and around bf16 rounding boundaries."""
    vals = []
    for bf in (0x3F80, 0x3F81, 0x4049, 0x404A, 0xBF80, 0xBF81, 0x0001, 0x0080, 0x7F7F, 0xFF7F, 0x7F7E):
        hi = np.uint32(bf) << np.uint32(16)
        for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):   # below half, tie, above half
            vals.append(np.uint32(hi | np.uint32(low)))
    f = np.array(vals, dtype=np.uint32).view(np.float32)
    return np.concatenate([f, np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4028235e38, -3.4028235e38,
                                        1e-40, -1e-40, 1e-45], dtype=np.float32)])


def test_round_bf16_matches_torch_on_float32_values():
    r = np.random.default_rng(2)
    x = np.concatenate([_ties_and_edges(),
                        (r.standard_normal(20000) * 10.0 ** r.integers(-40, 38, 20000)).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    _same(oracle.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_rounds_float64_through_float32():
    # the boundary rounds a float64 value to float32 first, then to bf16 (both
    # nearest even): 1 + 2^-8 + 2^-30 rounds to float32 at 1 + 2^-8 (a bf16
    # tie), which goes to the even neighbour 1.0; a direct float64 -> bf16
    # rounding would give 1 + 2^-7
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 3 * 2.0 ** -8 - 2.0 ** -30])
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    _same(oracle.round_bf16(x), want)
    assert oracle.round_bf16(x)[0] == 1.0


def test_round_f32_matches_torch():
    r = np.random.default_rng(3)
    x = r.standard_normal(5000) * 10.0 ** r.integers(-50, 50, 5000)
    _same(oracle.round_f32(x), torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy())


# ----------------------------------------------------------------------------
# the whole step, recomposed from torch float64 operations
# ----------------------------------------------------------------------------

def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _independent_step(x, parent, rank, k, bf16, eps=1e-6):
    """The step from torch float64 ops; returns the same fields medusa_step does."""
    h = _t(x["h"])
    W1, b1, W2, lm = _t(x["W1"]), _t(x["b1"]), _t(x["W2"]), _t(x["lm_head"])
    B, H = h.shape
    K = W2.shape[0]
    # heads: z_k = h + SiLU(W1_k h + b1_k); logits_k = W2_k z_k
    z = torch.stack([h + F.silu(F.linear(h, W1[j], b1[j])) for j in range(K)], dim=1)   # [B][K][H]
    logits = torch.stack([F.linear(z[:, j], W2[j]) for j in range(K)], dim=1)          # [B][K][V]
    # top guesses, decided on float32 scores (no two within the generator's gap)
    top = torch.topk(logits.to(torch.float32), k, dim=-1).indices.numpy()
    # the tree: node i's token is head depth(i)'s rank[i]-th guess
    N = len(parent)
    depth = [0] * N
    for i in range(1, N):
        depth[i] = depth[parent[i]] + 1
    tok = np.array([[int(x["root_tok"][b]) if i == 0 else int(top[b, depth[i] - 1, rank[i]]) for i in range(N)]
                    for b in range(B)], dtype=np.int64)
    # verification: every root-to-leaf branch is one causal sequence after the prefix
    q, kt, vt = _t(x["q"]), _t(x["k_tree"]), _t(x["v_tree"])
    kc, vc = _t(x["k_cache"]), _t(x["v_cache"])
    _, _, nH, D = q.shape
    nKV = kt.shape[2]
    children = {i: [j for j in range(N) if j > 0 and parent[j] == i] for i in range(N)}
    leaves = [i for i in range(N) if not children[i]]
    o = torch.full((B, N, nH, D), float("nan"), dtype=torch.float64)
    for b in range(B):
        P = int(x["cache_len"][b])
        for leaf in leaves:
            path = []
            j = leaf
            while True:
                path.append(j)
                if j == 0:
                    break
                j = parent[j]
            path = path[::-1]
            T = P + len(path)
            for hh in range(nH):
                kv = hh // (nH // nKV)
                keys = torch.cat([kc[b, kv, :P], kt[b, path, kv]])             # [T][D]
                vals = torch.cat([vc[b, kv, :P], vt[b, path, kv]])
                qs = torch.zeros(T, D, dtype=torch.float64)
                qs[P:] = q[b, path, hh]
                mask = torch.ones(T, T, dtype=torch.bool).tril()                 # causal
                out = F.scaled_dot_product_attention(qs[None], keys[None], vals[None], attn_mask=mask[None],
                                                     scale=float(np.float32(1.0 / np.sqrt(D))))[0]
                o[b, path, hh] = out[P:]
    assert not torch.isnan(o).any()
    if bf16:
        o = o.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    # base choice after every node: argmax of lm_head . RMSNorm(o), float32 decision
    rows = o.reshape(B * N, nH * D)
    n = rows / torch.sqrt((rows * rows).mean(dim=-1, keepdim=True) + eps)
    node_logits = F.linear(n, lm)
    g = torch.argmax(node_logits.to(torch.float32), dim=-1).numpy().reshape(B, N)
    # the longest accepted branch: from the root, follow the child carrying the
    # base model's choice (siblings carry distinct tokens, so at most one)
    res = dict(z=z.numpy(), logits=logits.numpy(), topk_idx=top, node_tok=tok, o=o.numpy(), greedy=g,
               node_logits=node_logits.numpy().reshape(B, N, -1), accept_len=[], path=[], out_tokens=[],
               new_cache_len=[], k_prefix=[], v_prefix=[])
    for b in range(B):
        path = [0]
        while True:
            nxt = [c for c in children[path[-1]] if tok[b, c] == g[b, path[-1]]]
            assert len(nxt) <= 1
            if not nxt:
                break
            path.append(nxt[0])
        L = len(path) - 1
        P = int(x["cache_len"][b])
        # hand-off: the cache is the prefix followed by the accepted branch's
        # keys/values, appended one token at a time
        kseq = [kc[b, :, s] for s in range(P)] + [kt[b, p] for p in path]
        vseq = [vc[b, :, s] for s in range(P)] + [vt[b, p] for p in path]
        res["accept_len"].append(L)
        res["path"].append(path)
        res["out_tokens"].append([int(tok[b, p]) for p in path[1:]] + [int(g[b, path[-1]])])
        res["new_cache_len"].append(P + L + 1)
        res["k_prefix"].append(torch.stack(kseq, dim=1).numpy())                # [nKV][P+L+1][D]
        res["v_prefix"].append(torch.stack(vseq, dim=1).numpy())
    return res


def _compare(ref, ind, B):
    np.testing.assert_allclose(ref["z"], ind["z"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["logits"], ind["logits"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(ref["topk_idx"], ind["topk_idx"])
    assert np.array_equal(ref["node_tok"], ind["node_tok"])
    np.testing.assert_allclose(ref["o"], ind["o"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ref["node_logits"], ind["node_logits"], rtol=1e-10, atol=1e-12)
    assert np.array_equal(ref["greedy"], ind["greedy"])
    for b in range(B):
        L = ind["accept_len"][b]
        assert ref["accept_len"][b] == L
        assert list(ref["path"][b]) == ind["path"][b]
        assert list(ref["out_tokens"][b]) == ind["out_tokens"][b]
        assert ref["new_cache_len"][b] == ind["new_cache_len"][b]
        n = ind["new_cache_len"][b]
        assert np.array_equal(ref["k_cache"][b][:, :n], ind["k_prefix"][b])
        assert np.array_equal(ref["v_cache"][b][:, :n], ind["v_prefix"][b])


def _plant_two_deep(x, parent, rank, K, k, eps=1e-6):
    """Rewrite two lm_head rows so that the base model's choice after the root
    is head 1's rank-0 token and after that node head 2's rank-0 token: row
    t1 = 100 u0 / |u0|^2 with u0 the part of the root's normalised row
    orthogonal to node 1's (so lm_head[t1] . n_root = 100, . n_1 = 0), and row
    t2 likewise for node 1.  The accepted branch is then at least two deep."""
    logits, _ = oracle.medusa_heads(x["h"], x["W1"], x["b1"], x["W2"])
    top, _ = oracle.topk(logits, k)
    D = x["q"].shape[-1]
    o = oracle.tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"], x["cache_len"], parent,
                              float(np.float32(1.0 / np.sqrt(D))))
    B, N = o.shape[:2]
    c1 = next(i for i in range(1, N) if parent[i] == 0 and rank[i] == 0)
    c2 = next(i for i in range(1, N) if parent[i] == c1 and rank[i] == 0)
    lm = x["lm_head"].copy()
    for b in range(B):
        n = oracle.rmsnorm(o[b].reshape(N, -1), eps)
        n0, n1 = n[0], n[c1]
        u0 = n0 - (n0 @ n1) / (n1 @ n1) * n1
        u1 = n1 - (n1 @ n0) / (n0 @ n0) * n0
        t1, t2 = int(top[b, 0, 0]), int(top[b, 1, 0])
        assert t1 != t2
        lm[t1] = 100.0 * u0 / (u0 @ u0)
        lm[t2] = 100.0 * u1 / (u1 @ u1)
    y = dict(x)
    y["lm_head"] = lm
    return y


@pytest.mark.parametrize("planted", [False, True], ids=["as_generated", "planted_two_deep"])
def test_medusa_step_equals_independent_composition_f32(planted):
    cfg = mi.config(1)
    heads, att, root, _ = make_workload(cfg)
    x = widen_inputs(cfg, heads, att, root)
    parent, rank = cfg.tree.arrays()
    if planted:
        x = _plant_two_deep(x, parent, rank, cfg.K, cfg.topk)
    ref = oracle.medusa_step(x, parent, rank, cfg.topk, cfg.dtype)
    ind = _independent_step(x, parent, rank, cfg.topk, bf16=False)
    _compare(ref, ind, cfg.B)
    if planted:
        assert min(ind["accept_len"]) >= 2


def test_medusa_step_equals_independent_composition_bf16():
    # bf16 storage: the attention output is rounded to bf16 before the greedy
    # stage; two ragged sequences, a 4-deep sparse tree
    cfg = mi.custom_config("step_bf16", "bf16", 2, 256, 1200, 4, 3, mi.sparse_tree(20, max_depth=4), 4, 2, 64,
                           (37, 90), 77)
    heads, att, root, _ = make_workload(cfg)
    x = widen_inputs(cfg, heads, att, root)
    parent, rank = cfg.tree.arrays()
    x = _plant_two_deep(x, parent, rank, cfg.K, cfg.topk)
    ref = oracle.medusa_step(x, parent, rank, cfg.topk, cfg.dtype)
    ind = _independent_step(x, parent, rank, cfg.topk, bf16=True)
    _compare(ref, ind, cfg.B)
    assert min(ind["accept_len"]) >= 2
    # the rounding of o matters here: without it the node scores move by more
    # than the comparison's tolerance
    ind_unrounded = _independent_step(x, parent, rank, cfg.topk, bf16=False)
    assert np.abs(ind_unrounded["node_logits"] - ref["node_logits"]).max() > 1e-6
