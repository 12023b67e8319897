"""GPU parity: every C-ABI call against the float64 oracle on the same seeded
inputs.  Integers (top-k ids, tree tokens/positions/masks, greedy ids,
accepted lengths/paths/tokens, compacted caches) must match exactly; floats
within 1e-4 (float32 workloads) or 2e-2 (bf16 workloads, fp32 accumulation).
"""
import sys

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from medusa_testlib import (assert_bf16_close, dev, enforce_greedy_gap, enforce_heads_gap, host_f64, make_workload,
                            pv_atol, tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import speculative_decoding_medusa_amd as M
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return M


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _cfg(name, dtype, B, H, V, K, topk, tree, nH=4, nKV=4, D=64, P=(128,), seed=100):
    return mi.custom_config(name, dtype, B, H, V, K, topk, tree, nH, nKV, D, P, seed)


# (name, workload, layout of W2: row-major GEMV or packed MFMA product)
HEAD_CASES = [
    ("c1", lambda: mi.config(1), "rows"),
    ("bf16_h1024_v5003_b1", lambda: _cfg("m1", "bf16", 1, 1024, 5003, 3, 4, mi.tiny_tree(), seed=101), "rows"),
    ("bf16_h512_v3001_b3_k6", lambda: _cfg("m2", "bf16", 3, 512, 3001, 2, 6, mi.tiny_tree(), seed=102), "rows"),
    ("f32_h256_v777_b2_k5", lambda: _cfg("m3", "f32", 2, 256, 777, 3, 5, mi.tiny_tree(), seed=103), "rows"),
    ("bf16_h2048_v4000_b8", lambda: _cfg("m4", "bf16", 8, 2048, 4000, 2, 4, mi.tiny_tree(), seed=104), "rows"),
    # packed W2 (MFMA): 8, 3 and 1 sequences; vocabularies not a multiple of
    # the 256 rows of a workgroup; top-16
    ("packed_h2048_v4000_b8", lambda: _cfg("m4", "bf16", 8, 2048, 4000, 2, 4, mi.tiny_tree(), seed=104), "packed"),
    ("packed_h512_v3001_b3_k6", lambda: _cfg("m2", "bf16", 3, 512, 3001, 2, 6, mi.tiny_tree(), seed=102), "packed"),
    ("packed_h1024_v5003_b1_k16", lambda: _cfg("m5", "bf16", 1, 1024, 5003, 3, 16, mi.tiny_tree(), seed=106),
     "packed"),
]


@pytest.mark.parametrize("name,mk,layout", HEAD_CASES, ids=[c[0] for c in HEAD_CASES])
def test_heads_parity(M, name, mk, layout):
    cfg = mk()
    _say("heads", name, layout)
    heads = mi.gen_heads(cfg)
    ov = []
    logits_ref, z_ref = enforce_heads_gap(cfg, heads, ov)   # [K][V][B], [B][K][H]
    logits_ref = np.transpose(logits_ref, (2, 0, 1))
    idx_ref, val_ref = oracle.topk(logits_ref, cfg.topk)
    h, W1, b1, W2 = (dev(heads[k]) for k in ("h", "W1", "b1", "W2"))
    if layout == "packed":
        W1, W2 = M.pack_heads(W1), M.pack_heads(W2)
    B, K, V, H, k = cfg.B, cfg.K, cfg.V, cfg.H, cfg.topk
    z = torch.empty(B, K, H, device="cuda")
    M.medusa_resid_silu(h, W1, b1, z)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host_f64(z), z_ref, rtol=0, atol=tol(cfg.dtype))
    logits = torch.empty(B, K, V, device="cuda")
    ti = torch.empty(B, K, k, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, k, device="cuda")
    M.medusa_heads_forward(h, W1, b1, W2, k, ti, tv, logits=logits)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host_f64(logits), logits_ref, rtol=0, atol=tol(cfg.dtype))
    assert np.array_equal(ti.cpu().numpy(), idx_ref)
    np.testing.assert_allclose(host_f64(tv), val_ref, rtol=0, atol=tol(cfg.dtype))
    # the two-call form (a1 then a2) gives the same bits as the fused call
    ti2 = torch.empty_like(ti)
    tv2 = torch.empty_like(tv)
    M.medusa_vocab_topk(z, W2, k, ti2, tv2)
    torch.cuda.synchronize()
    assert torch.equal(ti, ti2) and torch.equal(tv, tv2)


# heads and tree build in one call (the merge workgroup of head k writes the
# nodes at depth k + 1): the same top-k bits as medusa_heads_forward and the
# same tree as medusa_build_tree on it; several sequences, both layouts, top-k
# up to 16
HEADS_TREE_CASES = [
    ("rows_b1_sparse64", "rows", 1, 1024, 5003, 5, 4, lambda: mi.sparse_tree(64)),
    ("rows_b3_dense256_k3", "rows", 3, 512, 3001, 5, 3, lambda: mi.dense_tree(256)),
    ("packed_b8_sparse64", "packed", 8, 1024, 4000, 5, 4, lambda: mi.sparse_tree(64)),
    ("packed_b4_tiny_k16", "packed", 4, 512, 2000, 3, 16, lambda: mi.tiny_tree()),
    ("rows_b2_tiny_k3", "rows", 2, 256, 777, 3, 3, lambda: mi.tiny_tree()),
]


@pytest.mark.parametrize("name,layout,B,H,V,K,k,tree_fn", HEADS_TREE_CASES, ids=[c[0] for c in HEADS_TREE_CASES])
def test_heads_forward_tree_matches_two_calls(M, name, layout, B, H, V, K, k, tree_fn):
    cfg = _cfg("ht", "bf16", B, H, V, K, k, tree_fn(), seed=261)
    _say("heads + tree in one call", name)
    heads = mi.gen_heads(cfg)
    h, W1, b1, W2 = (dev(heads[x]) for x in ("h", "W1", "b1", "W2"))
    if layout == "packed":
        W1, W2 = M.pack_heads(W1), M.pack_heads(W2)
    parent, rank = cfg.tree.arrays()
    t = M.Tree(parent, rank, K, k)
    g = np.random.default_rng(262)
    root = dev(g.integers(0, V, B).astype(np.int32))
    cache_len = dev(g.integers(0, 1000, B).astype(np.int32))
    N, W = t.N, (t.N + 63) // 64
    ti = torch.empty(B, K, k, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, k, device="cuda")
    M.medusa_heads_forward(h, W1, b1, W2, k, ti, tv)
    tok = torch.empty(B, N, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    mask = torch.zeros(N * W, dtype=torch.int64, device="cuda")
    M.medusa_build_tree(t, ti, root, cache_len, tok, pos, mask)
    ti2 = torch.full_like(ti, -7)
    tv2 = torch.full_like(tv, -7.0)
    tok2 = torch.full_like(tok, -7)
    pos2 = torch.full_like(pos, -7)
    mask2 = torch.full_like(mask, -7)
    M.medusa_heads_forward_tree(h, W1, b1, W2, k, ti2, tv2, t, root, cache_len, tok2, pos2, mask2)
    torch.cuda.synchronize()
    assert torch.equal(ti, ti2) and torch.equal(tv, tv2)
    assert torch.equal(tok, tok2) and torch.equal(pos, pos2) and torch.equal(mask, mask2)
    # and without the mask output
    tok3 = torch.full_like(tok, -7)
    M.medusa_heads_forward_tree(h, W1, b1, W2, k, ti2, tv2, t, root, cache_len, tok3, pos2)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok3)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "bf16_packed"])
def test_zero_init_heads_reproduce_lm_head_bitwise(M, dtype):
    # heads page sketch: W1 = 0, b1 = 0, W2 = copy of lm_head => every head's
    # logits equal lm_head(h) exactly
    _say("zero-init", dtype)
    packed = dtype.endswith("_packed")
    dtype = dtype.replace("_packed", "")
    H, V, K = (256, 1000, 3) if dtype == "f32" else (4096, 32000, 5)
    cfg = _cfg("zi", dtype, 1, H, V, K, 4, mi.tiny_tree(), seed=105)
    lm = mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, dtype)
    h = dev(mi.normal((1, H), cfg.seed, mi.S_H, 1.0, dtype))
    lm_d = dev(lm)
    W2 = lm_d.unsqueeze(0).repeat(K, 1, 1).contiguous()
    W1 = torch.zeros(K, H, H, dtype=lm_d.dtype, device="cuda")
    b1 = torch.zeros(K, H, dtype=lm_d.dtype, device="cuda")
    lg = torch.empty(1, K, V, device="cuda")
    ti = torch.empty(1, K, 4, dtype=torch.int32, device="cuda")
    tv = torch.empty(1, K, 4, device="cuda")
    lm_w2 = lm_d.unsqueeze(0).contiguous()
    if packed:
        W1, W2, lm_w2 = M.pack_heads(W1), M.pack_heads(W2), M.pack_heads(lm_w2)
    M.medusa_heads_forward(h, W1, b1, W2, 4, ti, tv, logits=lg)
    base = torch.empty(1, 1, V, device="cuda")
    bi = torch.empty(1, 1, 4, dtype=torch.int32, device="cuda")
    bv = torch.empty(1, 1, 4, device="cuda")
    M.medusa_heads_forward(h, None, None, lm_w2, 4, bi, bv, logits=base)
    torch.cuda.synchronize()
    assert [bool(torch.equal(lg[:, k], base[:, 0])) for k in range(K)] == [True] * K
    assert all(torch.equal(ti[:, k], bi[:, 0]) for k in range(K))


@pytest.mark.parametrize("tree,K,topk,B", [(mi.tiny_tree(), 3, 3, 1), (mi.sparse_tree(64), 5, 4, 8),
                                           (mi.dense_tree(256), 5, 3, 2), (mi.chain_tree(7), 7, 1, 3)])
def test_build_tree_exact(M, tree, K, topk, B):
    _say("build_tree", tree.name, B)
    r = np.random.default_rng(7)
    tk = np.stack([np.stack([r.choice(50000, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    root = r.integers(0, 50000, B).astype(np.int32)
    P = r.integers(0, 5000, B).astype(np.int32)
    parent, rank = tree.arrays()
    t = M.Tree(parent, rank, K, topk)
    tok = torch.empty(B, tree.n, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    mask = torch.zeros(tree.n, t.W, dtype=torch.int64, device="cuda")
    M.medusa_build_tree(t, dev(tk), dev(root), dev(P), tok, pos, anc_mask=mask)
    torch.cuda.synchronize()
    tok_ref, pos_ref, mask_ref = oracle.build_tree(parent, rank, tk, root, P)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
    assert np.array_equal(pos.cpu().numpy(), pos_ref)
    m = mask.cpu().numpy().view(np.uint64)
    bits = np.zeros((tree.n, tree.n), dtype=bool)
    for i in range(tree.n):
        for j in range(tree.n):
            bits[i, j] = (int(m[i, j // 64]) >> (j % 64)) & 1
    assert np.array_equal(bits, mask_ref)
    assert np.array_equal(t.mask_host(), m)


ATT_CASES = [
    ("c1", lambda: mi.config(1)),
    ("bf16_sparse64_h4_d128_p300", lambda: _cfg("a1", "bf16", 1, 512, 10, 5, 4, mi.sparse_tree(64), 4, 4, 128, (300,), 201)),
    ("bf16_tiny_gqa_d64_b2", lambda: _cfg("a2", "bf16", 2, 256, 10, 3, 3, mi.tiny_tree(), 4, 2, 64, (100, 257), 202)),
    ("f32_chain9_d128_p0", lambda: _cfg("a3", "f32", 1, 256, 10, 9, 1, mi.chain_tree(9), 2, 2, 128, (0,), 203)),
    ("bf16_dense256_h2_d128_p1000", lambda: _cfg("a4", "bf16", 1, 256, 10, 5, 3, mi.dense_tree(256), 2, 2, 128, (1000,), 204)),
    ("bf16_sparse64_b3_ragged", lambda: _cfg("a5", "bf16", 3, 256, 10, 5, 4, mi.sparse_tree(64), 2, 1, 128, (1, 777, 2049), 205)),
    # no prefix at all: the tree range is the only key range
    ("bf16_sparse64_p0", lambda: _cfg("a6", "bf16", 1, 256, 10, 5, 4, mi.sparse_tree(64), 4, 4, 128, (0,), 206)),
    # four query blocks of 64 at D = 64, GQA, two sequences
    ("bf16_dense256_d64_gqa_b2", lambda: _cfg("a7", "bf16", 2, 256, 10, 5, 3, mi.dense_tree(256), 4, 2, 64, (70, 513), 207)),
    # 65..128 nodes: one workgroup of 4 query groups x 2 key groups per head and range
    ("bf16_sparse100_gqa_d128_b2", lambda: _cfg("a8", "bf16", 2, 256, 10, 5, 4, mi.sparse_tree(100), 4, 2, 128, (333, 1500), 208)),
    # 129..256 nodes (padded queries): 8 query groups, every wave against whole tiles
    ("bf16_sparse200_d64_p2100", lambda: _cfg("a9", "bf16", 1, 256, 10, 5, 5, mi.sparse_tree(200), 8, 8, 64, (2100,), 209)),
    ("bf16_sparse129_d128_b2_p0", lambda: _cfg("a10", "bf16", 2, 256, 10, 5, 5, mi.sparse_tree(129), 2, 1, 128, (0, 64), 210)),
]


@pytest.mark.parametrize("name,mk", ATT_CASES, ids=[c[0] for c in ATT_CASES])
def test_tree_attention_parity(M, name, mk):
    cfg = mk()
    _say("attention", name)
    att = mi.gen_attention(cfg)
    parent, rank = cfg.tree.arrays()
    t = M.Tree(parent, rank, cfg.K, cfg.topk)
    q, kt, vt, kc, vc = (dev(att[k]) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache"))
    kc0, vc0 = kc.clone(), vc.clone()
    cl = dev(att["cache_len"])
    out = torch.empty_like(q)
    M.tree_attention_verify(q, kt, vt, kc, vc, cl, max(cfg.P), t, out)
    torch.cuda.synchronize()
    w = {k: oracle.widen(att[k], cfg.dtype) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    scale = float(np.float32(1.0 / np.sqrt(cfg.D)))
    ref = oracle.tree_attention(w["q"], w["k_tree"], w["v_tree"], w["k_cache"], w["v_cache"], att["cache_len"],
                                parent, scale)
    if cfg.dtype == "bf16":
        exact = assert_bf16_close(host_f64(out), ref, atol=pv_atol(w["v_cache"], w["v_tree"], att["cache_len"]),
                                  what=name)
        _say("exactly rounded fraction", round(exact, 5))
    else:
        np.testing.assert_allclose(host_f64(out), ref, rtol=0, atol=tol(cfg.dtype))
    # the tree's keys/values now sit at slots P..P+N-1; every other slot is untouched
    kc_ref = kc0.clone()
    vc_ref = vc0.clone()
    for b, P in enumerate(cfg.P):
        kc_ref[b, :, P:P + cfg.N] = kt[b].transpose(0, 1)
        vc_ref[b, :, P:P + cfg.N] = vt[b].transpose(0, 1)
    assert torch.equal(kc, kc_ref) and torch.equal(vc, vc_ref)


GREEDY_CASES = [
    ("f32_r9_v1000", "f32", 9, 256, 1000, "rows"),
    ("bf16_r64_h1024_v5000", "bf16", 64, 1024, 5000, "packed"),
    ("bf16_r64_h1024_v5000_gemv", "bf16", 64, 1024, 5000, "rows"),
    ("bf16_r13_h4096_v3001", "bf16", 13, 4096, 3001, "packed"),
    ("bf16_r100_h1024_v2000", "bf16", 100, 1024, 2000, "packed"),   # 128-node MFMA tiles
    ("bf16_r200_h512_v1537", "bf16", 200, 512, 1537, "packed"),     # 256-node MFMA tiles, ragged vocabulary
    ("bf16_r300_h256_v1000", "bf16", 300, 256, 1000, "packed"),     # two 256-node tiles, the second ragged
    ("bf16_r5_h520_v999_gemv", "bf16", 5, 520, 999, "rows"),        # H not a multiple of the MFMA k-chunk
]


@pytest.mark.parametrize("name,dtype,R,H,V,layout", GREEDY_CASES, ids=[c[0] for c in GREEDY_CASES])
def test_base_greedy_parity(M, name, dtype, R, H, V, layout):
    _say("base_greedy", name)
    cfg = _cfg("g", dtype, 1, H, V, 1, 1, mi.tiny_tree(), seed=300 + R)
    heads = {"lm_head": mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, dtype)}
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, dtype)
    xw = oracle.widen(x, dtype)
    ov = []
    enforce_greedy_gap(cfg, heads, xw, ov)
    g_ref, lg_ref = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], dtype), 1e-6)
    g = torch.empty(R, dtype=torch.int32, device="cuda")
    lg = torch.empty(R, V, device="cuda")
    lm = dev(heads["lm_head"])
    if layout == "packed":
        lm = M.pack(lm)
    M.medusa_base_greedy(dev(x), lm, g, eps=1e-6, logits=lg)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host_f64(lg), lg_ref, rtol=0, atol=tol(dtype))
    assert np.array_equal(g.cpu().numpy(), g_ref)


# Trees of more than 128 nodes without logits over a vocabulary too small to
# give the skinny product 256 workgroups take the 32 x 32 x 16 product with
# loader waves (256-node tiles, 128 weight rows a workgroup, 64-wide k-chunks,
# loader rings four chunks deep): one chunk, two, three, a whole ring round
# and two rounds; ragged node tiles, two node tiles, ragged row tiles and a
# vocabulary under one row tile.
WIDE_GREEDY_CASES = [
    ("r129_h64_v200", 129, 64, 200),        # one chunk, 2 row tiles (the second ragged), one node past 128
    ("r200_h512_v1537", 200, 512, 1537),    # two ring rounds, ragged node tile
    ("r256_h256_v5000", 256, 256, 5000),    # one ring round, the last chunk on its final slot
    ("r300_h128_v1000", 300, 128, 1000),    # two node tiles, the second ragged, two chunks
    ("r512_h1024_v4099", 512, 1024, 4099),  # two full node tiles
    ("r160_h192_v100", 160, 192, 100),      # three chunks, a vocabulary under one row tile
]


@pytest.mark.parametrize("name,R,H,V", WIDE_GREEDY_CASES, ids=[c[0] for c in WIDE_GREEDY_CASES])
def test_base_greedy_wide_tree_parity(M, name, R, H, V):
    _say("base_greedy wide", name)
    cfg = _cfg("gw", "bf16", 1, H, V, 1, 1, mi.tiny_tree(), seed=700 + R)
    heads = {"lm_head": mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, "bf16")}
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, "bf16")
    xw = oracle.widen(x, "bf16")
    enforce_greedy_gap(cfg, heads, xw, [])
    g_ref, _ = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], "bf16"), 1e-6)
    g = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    M.medusa_base_greedy(dev(x), M.pack(dev(heads["lm_head"])), g, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), g_ref)


# Node tiles whose vocabulary gives 256-row weight tiles at least 256
# workgroups take the 256-row variant (8 waves loading and multiplying,
# 64-wide chunks): two ragged node tiles, one full, and a vocabulary whose
# last row tile is ragged.
WIDE256_GREEDY_CASES = [
    ("r300_h128_v32513", 300, 128, 32513),   # two node tiles, 128 x 2 workgroups, ragged last row tile
    ("r256_h192_v65600", 256, 192, 65600),   # one node tile, 257 workgroups, three chunks
    ("r512_h64_v33000", 512, 64, 33000),     # two full node tiles, one chunk
]


@pytest.mark.parametrize("name,R,H,V", WIDE256_GREEDY_CASES, ids=[c[0] for c in WIDE256_GREEDY_CASES])
def test_base_greedy_wide256_parity(M, name, R, H, V):
    _say("base_greedy wide256", name)
    cfg = _cfg("gw2", "bf16", 1, H, V, 1, 1, mi.tiny_tree(), seed=800 + R)
    heads = {"lm_head": mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, "bf16")}
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, "bf16")
    xw = oracle.widen(x, "bf16")
    enforce_greedy_gap(cfg, heads, xw, [])
    g_ref, _ = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], "bf16"), 1e-6)
    g = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    M.medusa_base_greedy(dev(x), M.pack(dev(heads["lm_head"])), g, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), g_ref)


def test_base_greedy_wide_tree_tiny_vocabulary(M):
    """17 vocabulary rows (one packed block and one row of the next; every
    other weight block of the workgroup clamped) against 140 nodes.  Too few
    rows to enforce a gap between every node's best two scores, so: where the
    float64 scores' best two differ by more than the products' error bound
    the ids match; elsewhere the chosen row scores within that bound of the
    best."""
    R, H, V = 140, 64, 17
    _say("base_greedy wide tiny vocabulary", R, H, V)
    cfg = _cfg("gwt", "bf16", 1, H, V, 1, 1, mi.tiny_tree(), seed=913)
    lm = mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, "bf16")
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, "bf16")
    lmw, xw = oracle.widen(lm, "bf16"), oracle.widen(x, "bf16")
    g_ref, _ = oracle.base_greedy(xw, lmw, 1e-6)
    scores = xw @ lmw.T                     # unnormalised: same argmax (positive row factors)
    g = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    M.medusa_base_greedy(dev(x), M.pack(dev(lm)), g, eps=1e-6)
    torch.cuda.synchronize()
    got = g.cpu().numpy()
    bound = 1e-4 * np.abs(xw) @ np.abs(lmw).T  # fp32 accumulation of bf16 products, with margin
    top2 = np.sort(scores, axis=1)[:, -2:]
    clear = top2[:, 1] - top2[:, 0] > 2 * bound.max(axis=1)
    assert clear.sum() > R // 2
    assert np.array_equal(got[clear], g_ref[clear])
    rows = np.arange(R)
    assert np.all((got >= 0) & (got < V))
    assert np.all(scores[rows, got] >= scores[rows, g_ref] - 2 * bound[rows, g_ref])


def _random_wide_shapes(n, seed=4242):
    """n seeded (R, H, V): 129-512 node rows, H a multiple of 64 up to 512,
    ragged vocabularies up to 3000 rows."""
    r = np.random.default_rng(seed)
    return [(int(r.integers(129, 513)), 64 * int(r.integers(1, 9)), int(r.integers(100, 3001))) for _ in range(n)]


@pytest.mark.parametrize("R,H,V", _random_wide_shapes(10), ids=lambda v: str(v))
def test_base_greedy_wide_tree_random_shapes(M, R, H, V):
    _say("base_greedy wide random", R, H, V)
    cfg = _cfg("gwr", "bf16", 1, H, V, 1, 1, mi.tiny_tree(), seed=900 + R + H + V)
    heads = {"lm_head": mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, "bf16")}
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, "bf16")
    xw = oracle.widen(x, "bf16")
    enforce_greedy_gap(cfg, heads, xw, [])
    g_ref, _ = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], "bf16"), 1e-6)
    g = torch.full((R,), -1, dtype=torch.int32, device="cuda")
    M.medusa_base_greedy(dev(x), M.pack(dev(heads["lm_head"])), g, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), g_ref)


def _pack_layout(W):
    """Row r, column k of a [rows][K] matrix of NRB = ceil(rows / 16) row blocks
    -> element ((k // 32) * NRB + r // 16) * 512 + ((k % 32) // 8 * 16 + r % 16) * 8 + k % 8
    of the packed buffer (padding rows zero)."""
    rows, K = W.shape
    nrb = -(-rows // 16)
    out = np.zeros(nrb * 16 * K, dtype=W.dtype)
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    idx = ((k // 32) * nrb + r // 16) * 512 + ((k % 32) // 8 * 16 + r % 16) * 8 + k % 8
    out[idx.ravel()] = W.ravel()
    return out


@pytest.mark.parametrize("shapes,inter", [([(16, 32)], 1), ([(37, 64)], 1), ([(4096, 96), (1024, 96), (1024, 96)], 1),
                                          ([(5, 256), (3, 256)], 1), ([(64, 64), (64, 64)], 2),
                                          ([(32, 96), (32, 96), (32, 96)], 3)],
                         ids=["one_block", "ragged_rows", "stacked_qkv", "stacked_ragged", "gate_up_interleaved",
                              "three_interleaved"])
def test_pack_rows_layout(M, shapes, inter):
    _say("pack_rows", shapes, inter)
    r = np.random.default_rng(7)
    mats = [r.integers(0, 1 << 16, size=s, dtype=np.uint16) for s in shapes]
    if inter == 1:
        logical = np.concatenate(mats)
    else:  # 16-row blocks of the matrices alternate: A[0:16], B[0:16], .., A[16:32], ..
        logical = np.concatenate([m[j:j + 16] for j in range(0, shapes[0][0], 16) for m in mats])
    want = _pack_layout(logical)
    rows = sum(s[0] for s in shapes)
    dst = M.Packed(torch.full((M.packed_size(rows, shapes[0][1]) // 2,), -1, dtype=torch.int16, device="cuda"),
                   rows, shapes[0][1])
    r0 = 0
    for i, m in enumerate(mats):
        src = torch.from_numpy(m.view(np.int16)).cuda()
        if inter == 1:
            M.medusa_pack_rows(src, dst, r0)
            r0 += m.shape[0]
        else:
            M.medusa_pack_rows(src, dst, 16 * i, inter)
    torch.cuda.synchronize()
    assert np.array_equal(dst.data.cpu().numpy().view(np.uint16), want)


def _planted_greedy(tree, tk, tok, truth):
    """greedy[i] = head (d+1)'s token of the true rank at depth d+1 (or a
    token outside the top-k)."""
    parent, _ = tree.arrays()
    depth = np.asarray(tree.depth)
    B, N = tok.shape
    K, k = tk.shape[1], tk.shape[2]
    g = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            d = depth[i]
            if d < K:
                R = truth[b, d]
                g[b, i] = tk[b, d, R] if R < k else 999999
            else:
                g[b, i] = 123456 + i
    return g


@pytest.mark.parametrize("tree,K,topk", [(mi.tiny_tree(), 2, 3), (mi.sparse_tree(64), 5, 4),
                                         (mi.dense_tree(256), 5, 3), (mi.chain_tree(5), 5, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_accept_and_compaction_exact(M, tree, K, topk, dtype):
    _say("accept", tree.name, dtype)
    B, nKV, D, layers = 8, 2, 64, 3
    parent, rank = tree.arrays()
    r = np.random.default_rng(11)
    tk = np.stack([np.stack([r.choice(30000, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    root = r.integers(0, 30000, B).astype(np.int32)
    P = r.integers(0, 300, B).astype(np.int32)
    tok, _, _ = oracle.build_tree(parent, rank, tk, root, P)
    pr = np.array([mi.rank_prior(0.8, j) for j in range(topk)] + [0.0])
    pr[-1] = 1 - pr[:-1].sum()
    truth = r.choice(topk + 1, size=(B, K), p=pr)
    truth[0] = 0  # sequence 0 accepts its deepest rank-0 chain
    g = _planted_greedy(tree, tk, tok, truth)
    Lmax = int(P.max()) + tree.n + 5
    cache_k = mi.normal((layers, B, nKV, Lmax, D), 50, mi.S_TEST + 1, 1.0, dtype)
    cache_v = mi.normal((layers, B, nKV, Lmax, D), 50, mi.S_TEST + 2, 1.0, dtype)
    t = M.Tree(parent, rank, K, topk)
    kc, vc = dev(cache_k), dev(cache_v)
    Dm = t.max_depth
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")
    M.medusa_accept(t, dev(tok), dev(g), al, an, ot, dev(P), ncl, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    kc_h = kc.cpu()
    vc_h = vc.cpu()
    ck = torch.from_numpy(cache_k.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(cache_k)
    cv = torch.from_numpy(cache_v.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(cache_v)
    for b in range(B):
        L, path, toks = oracle.accept(parent, tok[b], g[b])
        assert al[b].item() == L
        assert an[b].cpu().numpy().tolist() == path.tolist() + [-1] * (Dm - L)
        assert ot[b].cpu().numpy().tolist() == toks.tolist() + [-1] * (Dm - L)
        assert ncl[b].item() == P[b] + L + 1
        for src, got in ((ck, kc_h), (cv, vc_h)):
            ref, _ = oracle.compact_kv(src[:, b].float().numpy(), int(P[b]), path)
            assert np.array_equal(got[:, b].float().numpy(), ref)
    assert al[0].item() == Dm if tree.name != "tiny_2x3" else al[0].item() == 2


def test_accept_without_caches(M):
    tree = mi.sparse_tree(64)
    parent, rank = tree.arrays()
    _say("accept-no-cache")
    t = M.Tree(parent, rank, 5, 4)
    tk = np.arange(5 * 4, dtype=np.int32).reshape(1, 5, 4) + 100
    tok, _, _ = oracle.build_tree(parent, rank, tk, np.array([1]), np.array([10]))
    g = _planted_greedy(tree, tk, tok, np.array([[1, 0, 2, 0, 0]]))
    al = torch.empty(1, dtype=torch.int32, device="cuda")
    an = torch.empty(1, 6, dtype=torch.int32, device="cuda")
    ot = torch.empty(1, 6, dtype=torch.int32, device="cuda")
    ncl = torch.empty(1, dtype=torch.int32, device="cuda")
    M.medusa_accept(t, dev(tok), dev(g), al, an, ot, dev(np.array([10], np.int32)), ncl)
    torch.cuda.synchronize()
    L, path, toks = oracle.accept(parent, tok[0], g[0])
    assert al.item() == L and ncl.item() == 10 + L + 1
    assert an[0, :L + 1].cpu().numpy().tolist() == path.tolist()
    assert ot[0, :L + 1].cpu().numpy().tolist() == toks.tolist()


# ---------------------------------------------------------------------------
# cache slots past the prefix never reach the output
# ---------------------------------------------------------------------------

NAN_CASES = [
    # ragged sequences under one host bound: every sequence but the longest has
    # slots in [P_b, max_cache_len) that the last tile of a prefix range loads
    ("bf16_sparse64_b3_ragged", lambda: _cfg("n1", "bf16", 3, 256, 10, 5, 4, mi.sparse_tree(64), 4, 2, 128,
                                             (1, 777, 1000), 221), 2300),
    ("bf16_dense256_d64_b2", lambda: _cfg("n2", "bf16", 2, 256, 10, 5, 3, mi.dense_tree(256), 2, 2, 64,
                                          (70, 513), 222), 600),
    # the 256-node kernel at head size 128 (two query blocks a wave): the
    # partial last tiles of both sequences' ranges get their V rows zeroed
    ("bf16_dense256_d128_b2", lambda: _cfg("n5", "bf16", 2, 256, 10, 5, 3, mi.dense_tree(256), 2, 2, 128,
                                           (70, 700), 225), 800),
    ("bf16_sparse100_b2", lambda: _cfg("n3", "bf16", 2, 256, 10, 5, 4, mi.sparse_tree(100), 4, 4, 128,
                                       (333, 100), 223), 700),
    ("f32_tiny_b2", lambda: _cfg("n4", "f32", 2, 256, 10, 3, 3, mi.tiny_tree(), 4, 4, 64, (30, 97), 224), 200),
]


@pytest.mark.parametrize("name,mk,maxP", NAN_CASES, ids=[c[0] for c in NAN_CASES])
def test_tree_attention_ignores_slots_past_prefix(M, name, mk, maxP):
    """Slots at and past cache_len[b] hold NaN and infinities; the result must
    equal the oracle's, which reads slots < cache_len[b] only."""
    cfg = mk()
    _say("attention, NaN past the prefix", name, "max_cache_len", maxP)
    att = mi.gen_attention(cfg)
    parent, rank = cfg.tree.arrays()
    t = M.Tree(parent, rank, cfg.K, cfg.topk)
    Lmax = maxP + cfg.N
    B, nKV, D = cfg.B, cfg.nKV, cfg.D
    kc_h = np.empty((B, nKV, Lmax, D), dtype=att["k_cache"].dtype)
    vc_h = np.empty_like(kc_h)
    nan, inf = (np.uint16(0x7FC0), np.uint16(0x7F80)) if cfg.dtype == "bf16" else (np.float32(np.nan),
                                                                                     np.float32(np.inf))
    kc_h[...] = nan
    vc_h[...] = nan
    vc_h[..., 1::3, :] = inf
    for b, P in enumerate(cfg.P):
        kc_h[b, :, :P] = att["k_cache"][b, :, :P]
        vc_h[b, :, :P] = att["v_cache"][b, :, :P]
    q, kt, vt = (dev(att[k]) for k in ("q", "k_tree", "v_tree"))
    kc, vc = dev(kc_h), dev(vc_h)
    out = torch.empty_like(q)
    M.tree_attention_verify(q, kt, vt, kc, vc, dev(att["cache_len"]), maxP, t, out)
    torch.cuda.synchronize()
    got = host_f64(out)
    assert np.isfinite(got).all()
    w = {k: oracle.widen(att[k], cfg.dtype) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    ref = oracle.tree_attention(w["q"], w["k_tree"], w["v_tree"], w["k_cache"], w["v_cache"], att["cache_len"],
                                parent, float(np.float32(1.0 / np.sqrt(cfg.D))))
    if cfg.dtype == "bf16":
        assert_bf16_close(got, ref, atol=pv_atol(w["v_cache"], w["v_tree"], att["cache_len"]), what=name)
    else:
        np.testing.assert_allclose(got, ref, rtol=0, atol=tol(cfg.dtype))
    assert t.status() == 0


# ---------------------------------------------------------------------------
# the tree's status word: invalid device-side lengths are reported
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_status_word_reports_clamped_cache_len(M, dtype):
    cfg = _cfg("s1", dtype, 2, 256, 10, 5, 4, mi.sparse_tree(64), 2, 2, 128, (100, 100), 231)
    _say("status: clamped cache_len", dtype)
    att = mi.gen_attention(cfg)
    parent, rank = cfg.tree.arrays()
    t = M.Tree(parent, rank, cfg.K, cfg.topk)
    maxP = 100
    q, kt, vt, kc, vc = (dev(att[k]) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache"))
    out = torch.empty_like(q)
    assert t.status() == 0
    M.tree_attention_verify(q, kt, vt, kc, vc, dev(np.array([100, 64], np.int32)), maxP, t, out)
    assert t.status() == 0
    # sequence 0 claims more than the host bound, sequence 1 a negative length:
    # both are clamped into [0, max_cache_len] (all accesses stay in bounds)
    M.tree_attention_verify(q, kt, vt, kc, vc, dev(np.array([maxP + 7, -5], np.int32)), maxP, t, out)
    assert t.status(clear=False) == M.STATUS_CACHE_LEN_CLAMPED
    assert t.status() == M.STATUS_CACHE_LEN_CLAMPED
    assert t.status() == 0
    # the clamped call computed attention at lengths maxP and 0
    w = {k: oracle.widen(att[k], cfg.dtype) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    ref = oracle.tree_attention(w["q"], w["k_tree"], w["v_tree"], w["k_cache"], w["v_cache"], [maxP, 0], parent,
                                float(np.float32(1.0 / np.sqrt(cfg.D))))
    np.testing.assert_allclose(host_f64(out), ref, rtol=0, atol=tol(cfg.dtype))


def test_status_word_reports_cache_overflow(M):
    tree = mi.sparse_tree(64)
    parent, rank = tree.arrays()
    _say("status: cache overflow in accept")
    B, nKV, D, K, topk = 2, 2, 64, 5, 4
    t = M.Tree(parent, rank, K, topk)
    tk = np.arange(B * K * topk, dtype=np.int32).reshape(B, K, topk) + 100
    Lmax = 200
    P = np.array([50, Lmax - tree.n + 1], dtype=np.int32)     # sequence 1's tree slots would pass Lmax
    tok, _, _ = oracle.build_tree(parent, rank, tk, np.array([1, 2]), P)
    g = _planted_greedy(tree, tk, tok, np.zeros((B, K), dtype=np.int64))   # both accept the rank-0 chain
    cache = mi.normal((1, B, nKV, Lmax, D), 60, mi.S_TEST + 7, 1.0, "bf16")
    kc, vc = dev(cache), dev(cache)
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, t.max_depth + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty_like(an)
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")
    M.medusa_accept(t, dev(tok), dev(g), al, an, ot, dev(P), ncl, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert t.status() == M.STATUS_CACHE_OVERFLOW
    assert al.cpu().numpy().tolist() == [t.max_depth, t.max_depth]
    # sequence 0 compacted and advanced; sequence 1 untouched and not advanced
    assert ncl.cpu().numpy().tolist() == [P[0] + t.max_depth + 1, P[1]]
    L0, path0, _ = oracle.accept(parent, tok[0], g[0])
    ref0, _ = oracle.compact_kv(cache[0, 0], int(P[0]), path0)
    got = kc.cpu().view(torch.int16).numpy().view(np.uint16)[0]
    assert np.array_equal(got[0], ref0)
    assert np.array_equal(got[1], cache[0, 1])
    # without caches nothing can overflow
    M.medusa_accept(t, dev(tok), dev(g), al, an, ot, dev(P), ncl)
    torch.cuda.synchronize()
    assert t.status() == 0
    assert ncl.cpu().numpy().tolist() == [P[0] + t.max_depth + 1, P[1] + t.max_depth + 1]


# ---------------------------------------------------------------------------
# the tie rule: among equal scores the lower vocabulary index ranks first
# ---------------------------------------------------------------------------

def _dup_positions(t, V, spread):
    """Rows to copy the winning row t to: within the same 16-row fragment
    ('near'), in other 16-row blocks tens of rows away, within one workgroup's
    weight rows but other waves' ('mid'), or hundreds of rows away, in other
    workgroups ('far').  Returns (rows holding a copy, expected order of the
    tied rows)."""
    if spread == "near":
        cands = [t - 1, t + 1, t + 5]
    elif spread == "mid":
        cands = [t - 37, t + 20, t + 45]
    else:
        cands = [t - 517, t - 1200, t + 733, t + 2100]
    rows = sorted(set(c for c in cands if 0 <= c < V and c != t))
    return rows, sorted(rows + [t])


@pytest.mark.parametrize("spread", ["near", "far"])
@pytest.mark.parametrize("layout", ["rows", "packed"])
def test_topk_ties_keep_lower_index(M, layout, spread):
    B = 1 if layout == "rows" else 4          # the step's layouts: GEMV at 1 sequence, MFMA from 4
    cfg = _cfg("tie", "bf16", B, 1024, 5003, 3, 4, mi.tiny_tree(), seed=241)
    _say("top-k ties", layout, spread)
    heads = mi.gen_heads(cfg)
    logits_ref, _ = enforce_heads_gap(cfg, heads, [])           # [K][V][B]
    # each head: copy sequence 0's winning row of W2 to other rows; a copy
    # scores exactly what the original scores, for every sequence
    order = []
    for k in range(cfg.K):
        tw = int(np.lexsort((np.arange(cfg.V), -oracle.round_f32(logits_ref[k, :, 0])))[0])
        rows, tied = _dup_positions(tw, cfg.V, spread)
        heads["W2"][k, rows] = heads["W2"][k, tw]
        logits_ref[k, rows] = logits_ref[k, tw]
        order.append(tied)
    idx_ref, _ = oracle.topk(np.transpose(logits_ref, (2, 0, 1)), cfg.topk)
    for k in range(cfg.K):                                       # the oracle's rule: tied rows by index
        n = min(len(order[k]), cfg.topk)
        assert idx_ref[0, k, :n].tolist() == order[k][:n]
    h, W1, b1, W2 = (dev(heads[k]) for k in ("h", "W1", "b1", "W2"))
    if layout == "packed":
        W1, W2 = M.pack_heads(W1), M.pack_heads(W2)
    ti = torch.empty(B, cfg.K, cfg.topk, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, cfg.K, cfg.topk, device="cuda")
    M.medusa_heads_forward(h, W1, b1, W2, cfg.topk, ti, tv)
    torch.cuda.synchronize()
    got, val = ti.cpu().numpy(), tv.cpu().numpy()
    for k in range(cfg.K):                                       # the copies scored bit for bit alike
        n = min(len(order[k]), cfg.topk)
        assert len(set(val[0, k, :n].tolist())) == 1, (k, val[0, k])
    assert np.array_equal(got, idx_ref)
    # the merge that also builds the tree keeps the same rule
    parent, rank = cfg.tree.arrays()
    t = M.Tree(parent, rank, cfg.K, cfg.topk)
    tok = torch.empty(B, t.N, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    zero = dev(np.zeros(B, np.int32))
    M.medusa_heads_forward_tree(h, W1, b1, W2, cfg.topk, ti, tv, t, zero, zero, tok, pos)
    torch.cuda.synchronize()
    assert np.array_equal(ti.cpu().numpy(), idx_ref)


@pytest.mark.parametrize("R", [64, 256, 512], ids=["r64", "r256", "r512"])  # 256, 512: 32 x 32 x 16 with loader waves
@pytest.mark.parametrize("spread", ["near", "mid", "far"])
@pytest.mark.parametrize("layout", ["rows", "packed"])
def test_greedy_ties_keep_lower_index(M, layout, spread, R):
    H, V = 1024, 5000
    cfg = _cfg("gtie", "bf16", 1, H, V, 1, 1, mi.tiny_tree(), seed=251)
    _say("argmax ties", layout, spread, R)
    tied = (0, 17, R // 2 + 3, R - 1)
    heads = {"lm_head": mi.normal((V, H), cfg.seed, mi.S_LM_HEAD, 0.02, "bf16")}
    x = mi.normal((R, H), cfg.seed, mi.S_TEST, 1.0, "bf16")
    xw = oracle.widen(x, "bf16")
    enforce_greedy_gap(cfg, heads, xw, [])
    g0, _ = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], "bf16"), 1e-6)
    # copy the winners of a few rows to other rows of lm_head
    for r in tied:
        rows, _ = _dup_positions(int(g0[r]), V, spread)
        heads["lm_head"][rows] = heads["lm_head"][int(g0[r])]
    g_ref, _ = oracle.base_greedy(xw, oracle.widen(heads["lm_head"], "bf16"), 1e-6)
    for r in tied:
        _, order = _dup_positions(int(g0[r]), V, spread)
        assert g_ref[r] == order[0]       # the oracle's rule: the lowest of the tied rows
    g = torch.empty(R, dtype=torch.int32, device="cuda")
    lm = dev(heads["lm_head"])
    if layout == "packed":
        lm = M.pack(lm)
    M.medusa_base_greedy(dev(x), lm, g, eps=1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), g_ref)


# ---------------------------------------------------------------------------
# compaction at the 32-layer workload's cache shape, deepest branches
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tree,K,topk,nKV,D,layers", [
    (mi.sparse_tree(64), 5, 4, 32, 128, 32),     # the 32-layer workload's caches: L = Dmax = 5, 640 elements a slice
    (mi.chain_tree(16), 16, 1, 4, 128, 4),       # the deepest tree: L = 16, 2048 elements a slice
    (mi.dense_tree(256), 5, 3, 8, 128, 6),
], ids=["sparse64_nkv32_d128_32layers", "chain16_d128", "dense256_d128"])
def test_deep_compaction_bench_shape(M, tree, K, topk, nKV, D, layers):
    _say("deep compaction", tree.name, "nKV", nKV, "D", D, "layers", layers)
    B = 2
    parent, rank = tree.arrays()
    r = np.random.default_rng(19)
    tk = np.stack([np.stack([r.choice(30000, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    root = r.integers(0, 30000, B).astype(np.int32)
    P = np.array([300, 7], dtype=np.int32)
    tok, _, _ = oracle.build_tree(parent, rank, tk, root, P)
    truth = np.zeros((B, K), dtype=np.int64)                   # the rank-0 chain all the way down
    if tree.name.startswith("dense"):
        truth[1] = [1, 1, 2, 0, 1]                             # a depth-5 branch under the second child (the
        #                                                        256-node cut keeps depth-5 tuples (0, ..) and (1, 0|1, ..))
    g = _planted_greedy(tree, tk, tok, truth)
    Lmax = int(P.max()) + tree.n + 3
    cache_k = mi.normal((layers, B, nKV, Lmax, D), 70, mi.S_TEST + 11, 1.0, "bf16")
    cache_v = mi.normal((layers, B, nKV, Lmax, D), 70, mi.S_TEST + 12, 1.0, "bf16")
    t = M.Tree(parent, rank, K, topk)
    kc, vc = dev(cache_k), dev(cache_v)
    Dm = t.max_depth
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")
    M.medusa_accept(t, dev(tok), dev(g), al, an, ot, dev(P), ncl, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert t.status() == 0
    kh = kc.cpu().view(torch.int16).numpy().view(np.uint16)
    vh = vc.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in range(B):
        L, path, toks = oracle.accept(parent, tok[b], g[b])
        assert L == Dm
        assert al[b].item() == L and ncl[b].item() == P[b] + L + 1
        assert an[b].cpu().numpy().tolist() == path.tolist()
        assert ot[b].cpu().numpy().tolist() == toks.tolist()
        for src, got in ((cache_k, kh), (cache_v, vh)):
            ref, _ = oracle.compact_kv(src[:, b], int(P[b]), path)     # bit patterns, every layer and head
            assert np.array_equal(got[:, b], ref)
