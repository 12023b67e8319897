"""GPU parity of the generate loop around the step: the hand-off call
(medusa_advance) against the oracle's, and rounds of MedusaLoop on a small
Llama-shaped decoder replayed round by round against the oracle.

Round replay.  Before every round the GPU state (h, root token, prefix
lengths, every layer's cache) is copied to the host; after it the oracle runs
the same round from that state and every result of the GPU round is checked:
the heads' top-k (indices exact unless two scores lie within 1e-3; the picked
scores must then match the oracle's by rank), the tree tokens (exact), the
greedy choices (exact unless the best two scores lie within the 2e-2 float
bound of the bf16 decoder pass, see test_gpu_decoder; the pick must then be
within that bound of the best), the decoder's hidden rows (the decoder test's
bound), the acceptance on the GPU's own choices (exact), the hand-off (exact:
root, h as the bf16 rounding of the GPU's hidden row, tokens, lengths) and the
caches (accepted slots within the float bound, the prefix untouched).  A
captured run of rounds must replay bit for bit like the eager rounds.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from medusa_testlib import dev, host_f64, planted_greedy_ref

pytestmark = pytest.mark.gpu

BF16_STEP = 2.0 ** -8
TOPK_TIE = 1e-3
GREEDY_TIE = 2e-2


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _close(got, ref):
    np.testing.assert_allclose(got, ref, rtol=2 * BF16_STEP, atol=4e-2)
    assert np.sqrt(np.mean((got - ref) ** 2)) <= 1e-2 * np.sqrt(np.mean(ref ** 2)) + 1e-12


# ---------------------------------------------------------------------------
# medusa_advance
# ---------------------------------------------------------------------------

def _paths(parent, depth, B, Dmax, seed):
    """One valid accepted path per sequence: L = 0, L = Dmax, then random depths."""
    r = np.random.default_rng(seed)
    out = []
    for b in range(B):
        L = 0 if b == 0 else Dmax if b == 1 else int(r.integers(0, Dmax + 1))
        ends = np.flatnonzero(depth == L)
        j = int(ends[r.integers(0, len(ends))])
        path = []
        while j >= 0:
            path.append(j)
            j = parent[j] if j > 0 else -1
        out.append((L, path[::-1]))
    return out


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_advance_parity(dt):
    import speculative_decoding_medusa_amd as M
    _say("advance", dt)
    spec = mi.sparse_tree(64)
    parent, rank = spec.arrays()
    tree = M.Tree(parent, rank, 5, 4)
    depth = oracle.tree_depths(parent)
    B, N, H, Dmax, cap = 4, tree.N, 320, tree.max_depth, 9
    paths = _paths(parent, depth, B, Dmax, 3)
    al = np.array([L for L, _ in paths], dtype=np.int32)
    an = np.full((B, Dmax + 1), -1, dtype=np.int32)
    ot = np.full((B, Dmax + 1), -1, dtype=np.int32)
    toks = mi.uniform_int((B, Dmax + 1), 71, mi.S_TEST + 11, 0, 31999)
    for b, (L, p) in enumerate(paths):
        an[b, :L + 1] = p
        ot[b, :L + 1] = toks[b, :L + 1]
    al[3] = -1  # not an acceptance result: the sequence must be left unchanged
    hidden = mi.normal((B, N, H), 71, mi.S_TEST + 12, 1.0, "f32")
    n0 = np.array([0, 2, cap - 1, 1], dtype=np.int32)   # sequence 2's round overruns the buffer
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    h = torch.full((B, H), 7.0, dtype=tdt, device="cuda")
    root = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    tokens = torch.full((B, cap), -1, dtype=torch.int32, device="cuda")
    n_tok = dev(n0)
    ncl = dev(np.array([100, 101, 102, 103], dtype=np.int32))
    cl = torch.zeros(B, dtype=torch.int32, device="cuda")
    M.medusa_advance(tree, dev(al), dev(an), dev(ot), dev(hidden), root, h, tokens=tokens, n_tokens=n_tok,
                     new_cache_len=ncl, cache_len=cl)
    torch.cuda.synchronize()
    h_got = h.float().cpu().numpy().astype(np.float64)
    want_tokens = np.full((B, cap), -1, dtype=np.int32)
    for b in range(B):
        if b == 3:
            assert root[b].item() == -5 and np.all(h_got[b] == 7.0) and n_tok[b].item() == n0[b]
            assert cl[b].item() == 0
            continue
        L, p = paths[b]
        r, hh, emitted = oracle.advance(L, np.array(p), ot[b, :L + 1], hidden[b].astype(np.float64), dt == "bf16")
        assert root[b].item() == r
        assert np.array_equal(h_got[b], hh)
        assert n_tok[b].item() == n0[b] + L + 1
        assert cl[b].item() == 100 + b
        for j, t in enumerate(emitted):
            if n0[b] + j < cap:
                want_tokens[b, n0[b] + j] = t
    assert np.array_equal(tokens.cpu().numpy(), want_tokens)


def test_advance_argument_errors():
    import speculative_decoding_medusa_amd as M
    parent, rank = mi.tiny_tree().arrays()
    tree = M.Tree(parent, rank, 3, 3)
    i = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    hid = torch.zeros(2, tree.N, 64, device="cuda")
    h = torch.zeros(2, 64, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MedusaError) as e:   # tokens without n_tokens
        M.medusa_advance(tree, r, i, i, hid, r, h, tokens=i)
    assert e.value.status == M.EINVAL
    with pytest.raises(M.MedusaError) as e:   # cache_len without new_cache_len
        M.medusa_advance(tree, r, i, i, hid, r, h, cache_len=r)
    assert e.value.status == M.EINVAL


# ---------------------------------------------------------------------------
# rounds of the loop on a small decoder
# ---------------------------------------------------------------------------

def _loop_setup(M, P_start, seed):
    # the config's P sizes the caches (Lmax = max P + N); the rounds start at P_start
    # an 8-token vocabulary: the heads' top-4 guesses are often right, so rounds accept candidates
    cfg = mi.custom_config("gen", "bf16", len(P_start), 256, 8, 5, 4, mi.sparse_tree(24), 4, 2, 64, (110,) * len(P_start),
                           seed, layers=2, ffn=384)
    heads = mi.gen_heads(cfg)
    layers = [mi.gen_layer(cfg, l) for l in range(cfg.layers)]
    caches = [mi.gen_layer_cache(cfg, l) for l in range(cfg.layers)]
    emb = mi.gen_embedding(cfg)
    root = mi.uniform_int((cfg.B,), seed, mi.S_TEST + 21, 0, cfg.V - 1).astype(np.int32)
    parent, rank = cfg.tree.arrays()
    tree = M.Tree(parent, rank, cfg.K, cfg.topk)
    g = dict(
        heads={"w1": dev(heads["W1"]), "b1": dev(heads["b1"]), "w2": dev(heads["W2"])},
        layers=[M.pack_layer({m: dev(W[m]) for m in W}) for W in layers],
        embedding=dev(emb), lm_head=M.pack(dev(heads["lm_head"])), tree=tree,
        k_cache=torch.stack([dev(c[0]) for c in caches]), v_cache=torch.stack([dev(c[1]) for c in caches]),
        cache_len=dev(np.asarray(P_start, dtype=np.int32)), h=dev(heads["h"]), root_tok=dev(root))
    o = dict(heads=dict(W1=oracle.widen(heads["W1"], "bf16"), b1=oracle.widen(heads["b1"], "bf16"),
                        W2=oracle.widen(heads["W2"], "bf16")),
             dec=dict(embedding=oracle.widen(emb, "bf16"), lm_head=oracle.widen(heads["lm_head"], "bf16"),
                      layers=[{m: oracle.widen(W[m], "bf16") for m in W} for W in layers], nH=cfg.nH, nKV=cfg.nKV))
    return cfg, g, o, parent, rank


def _make_loop(M, cfg, g, cap=64, planted=None):
    return M.MedusaLoop(g["heads"], g["layers"], g["embedding"], g["lm_head"], g["tree"], cfg.topk, g["k_cache"],
                        g["v_cache"], cfg.nH, g["cache_len"], g["h"], g["root_tok"], cap=cap, planted=planted,
                        plant_seed=99)


def _check_topk(gpu_idx, logits, k):
    """GPU top-k vs float64 scores: same indices unless scores tie within
    TOPK_TIE; the picked scores must match the oracle's by rank."""
    ref_idx, ref_val = oracle.topk(logits, k)
    B, K, _ = gpu_idx.shape
    for b in range(B):
        for j in range(K):
            got = gpu_idx[b, j]
            assert len(set(got.tolist())) == k
            if np.array_equal(got, ref_idx[b, j]):
                continue
            np.testing.assert_allclose(logits[b, j, got], ref_val[b, j], rtol=0, atol=TOPK_TIE)


@pytest.mark.parametrize("planted", [None, 0.8], ids=["model_choices", "planted_alpha0.8"])
def test_loop_rounds_replay_against_oracle(planted):
    import speculative_decoding_medusa_amd as M
    P_start = (40, 77)
    cfg, g, o, parent, rank = _loop_setup(M, P_start, 611)
    loop = _make_loop(M, cfg, g, planted=planted)
    B, N, Dmax = cfg.B, cfg.N, g["tree"].max_depth
    n_prev = np.zeros(B, dtype=np.int64)
    tokens_ref = [[] for _ in range(B)]
    accepted = 0
    for t in range(5):
        _say("round", t)
        s = dict(h=host_f64(loop.h), root_tok=loop.root_tok.cpu().numpy().astype(np.int64),
                 cache_len=loop.cache_len.cpu().numpy().astype(np.int64),
                 kc=host_f64(loop.k_cache), vc=host_f64(loop.v_cache))
        loop.round()
        torch.cuda.synchronize()
        # heads and tree
        logits, _ = oracle.medusa_heads(s["h"], o["heads"]["W1"], o["heads"]["b1"], o["heads"]["W2"])
        ti = loop.topk_idx.cpu().numpy()
        _check_topk(ti, logits, cfg.topk)
        node_tok, node_pos, _ = oracle.build_tree(parent, rank, ti, s["root_tok"], s["cache_len"])
        assert np.array_equal(loop.node_tok.cpu().numpy(), node_tok)
        assert np.array_equal(loop.node_pos.cpu().numpy(), node_pos)
        # the verify pass on the GPU's tree
        kcs = [s["kc"][l] for l in range(cfg.layers)]
        vcs = [s["vc"][l] for l in range(cfg.layers)]
        ref = oracle.decoder_verify(node_tok, s["cache_len"], parent, o["dec"]["embedding"], o["dec"]["layers"],
                                    o["dec"]["lm_head"], kcs, vcs, cfg.nH, cfg.nKV, bf16=True)
        hid = host_f64(loop.hidden)
        _close(hid, ref["hidden"])
        g_gpu = loop.greedy.cpu().numpy()
        if planted is None:
            lg = oracle.round_f32(ref["logits"])
            for b in range(B):
                for i in range(N):
                    best = lg[b, i].max()
                    if g_gpu[b, i] != ref["greedy"][b, i]:
                        assert lg[b, i, g_gpu[b, i]] >= best - GREEDY_TIE, (t, b, i)
        else:
            # the planted continuation, exactly as the host reference draws it
            assert np.array_equal(g_gpu, planted_greedy_ref(cfg.tree.depth, ti, s["cache_len"], planted, 99, cfg.V))
        # acceptance on the GPU's own choices, then the hand-off
        al, an, ot = loop.accept_len.cpu().numpy(), loop.accept_nodes.cpu().numpy(), loop.out_tokens.cpu().numpy()
        kh, vh = host_f64(loop.k_cache), host_f64(loop.v_cache)
        h_got = host_f64(loop.h)
        for b in range(B):
            L, path, toks = oracle.accept(parent, node_tok[b], g_gpu[b])
            accepted += L
            assert al[b] == L
            assert np.array_equal(an[b, :L + 1], path) and np.all(an[b, L + 1:] == -1)
            assert np.array_equal(ot[b, :L + 1], toks) and np.all(ot[b, L + 1:] == -1)
            r, hh, emitted = oracle.advance(L, path, toks, hid[b], True)
            assert loop.root_tok[b].item() == r
            assert np.array_equal(h_got[b], hh)
            P = int(s["cache_len"][b])
            assert loop.cache_len[b].item() == P + L + 1
            tokens_ref[b] += emitted
            for l in range(cfg.layers):
                # the prefix is untouched; slot P + d holds the tree keys/values of path[d]
                assert np.array_equal(kh[l, b, :, :P], s["kc"][l, b, :, :P])
                _close(kh[l, b, :, P:P + L + 1].transpose(1, 0, 2), ref["k_tree"][l][b][path])
                _close(vh[l, b, :, P:P + L + 1].transpose(1, 0, 2), ref["v_tree"][l][b][path])
        n_prev += np.array([L_ + 1 for L_ in al])
        assert np.array_equal(loop.n_tokens.cpu().numpy(), n_prev)
    got_tokens = loop.tokens.cpu().numpy()
    for b in range(B):
        assert got_tokens[b, :len(tokens_ref[b])].tolist() == tokens_ref[b]
    _say("ok, accepted candidates over the rounds:", accepted)
    assert accepted >= 1   # the accepted-path hand-off and compaction were exercised
    if planted is not None:
        assert accepted >= 10   # deep branches (about 2.9 per sequence and round under the prior)


def test_loop_graph_replays_match_eager():
    import speculative_decoding_medusa_amd as M
    _say("loop graph")
    P_start = (33, 61)
    cfg, g, _, _, _ = _loop_setup(M, P_start, 612)
    init = {k: g[k].clone() for k in ("k_cache", "v_cache", "cache_len", "h", "root_tok")}
    # eager reference: 3 x 2 rounds from the initial state
    eager = _make_loop(M, cfg, g)
    snaps = []
    for _ in range(3):
        eager.run(2)
        torch.cuda.synchronize()
        snaps.append({k: getattr(eager, k).clone() for k in ("k_cache", "v_cache", "cache_len", "h", "root_tok",
                                                               "tokens", "n_tokens")})
    # the same from the initial state, two rounds per captured graph
    g2 = dict(g)
    g2.update({k: v.clone() for k, v in init.items()})
    loop = _make_loop(M, cfg, g2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        # warm the launch paths on a scratch copy of the state, then restore it
        keep = {k: getattr(loop, k).clone() for k in ("k_cache", "v_cache", "cache_len", "h", "root_tok", "tokens",
                                                      "n_tokens")}
        loop.round()
        for k, v in keep.items():
            getattr(loop, k).copy_(v)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()   # no finalizer may free device memory while the graph is captured
    try:
        with torch.cuda.graph(graph):
            loop.run(2)
    finally:
        gc.enable()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1, device="cuda") * 2   # eager work between replays
        torch.cuda.synchronize()
        for k, v in snaps[rep].items():
            assert torch.equal(getattr(loop, k), v), (rep, k)
    _say("ok")


@pytest.mark.parametrize("alpha,tree_name", [(0.8, "sparse64"), (0.3, "sparse64"), (0.8, "dense256"),
                                              (1.0, "chain7")])
def test_plant_greedy_matches_host_reference(alpha, tree_name):
    import speculative_decoding_medusa_amd as M
    _say("plant_greedy", alpha, tree_name)
    tree = {"sparse64": mi.sparse_tree(64), "dense256": mi.dense_tree(256), "chain7": mi.chain_tree(7)}[tree_name]
    parent, rank = tree.arrays()
    K = max(tree.depth)
    topk = int(max(rank)) + 1
    B, V = 37, 32000
    r = np.random.default_rng(21)
    tk = np.stack([np.stack([r.choice(V, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
    P = r.integers(0, 1 << 20, B).astype(np.int32)
    t = M.Tree(parent, rank, K, topk)
    g = torch.full((B, tree.n), -7, dtype=torch.int32, device="cuda")
    M.medusa_plant_greedy(t, dev(tk), dev(P), g, V, alpha, seed=0xC0FFEE)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), planted_greedy_ref(tree.depth, tk, P, alpha, 0xC0FFEE, V))


@pytest.mark.parametrize("tree_name", ["sparse64", "dense256", "tiny"])
def test_accept_stats_matches_host_reference(tree_name):
    """medusa_accept_stats over three rounds of planted acceptance (per-depth
    alphas falling with depth) against the host count of what each round
    revealed."""
    import speculative_decoding_medusa_amd as M
    from medusa_testlib import accept_stats_ref
    _say("accept_stats", tree_name)
    tree = {"sparse64": mi.sparse_tree(64), "dense256": mi.dense_tree(256), "tiny": mi.tiny_tree()}[tree_name]
    parent, rank = tree.arrays()
    K = max(tree.depth) + (1 if tree_name == "tiny" else 0)    # tiny: a head beyond the tree's depth
    topk = int(max(rank)) + 1
    B, V = 29, 5000
    t = M.Tree(parent, rank, K, topk)
    counts = torch.zeros(K, topk + 1, dtype=torch.int32, device="cuda")
    want = np.zeros((K, topk + 1), dtype=np.int64)
    r = np.random.default_rng(31)
    Dm = t.max_depth
    for rnd in range(3):
        tk = np.stack([np.stack([r.choice(V, topk, replace=False) for _ in range(K)]) for _ in range(B)]).astype(np.int32)
        P = r.integers(0, 1 << 20, B).astype(np.int32)
        root = r.integers(0, V, B).astype(np.int32)
        tok, _, _ = oracle.build_tree(parent, rank, tk, root, P)
        g = torch.empty(B, tree.n, dtype=torch.int32, device="cuda")
        M.medusa_plant_greedy(t, dev(tk), dev(P), g, V, [0.9, 0.7, 0.5, 0.4, 0.3], seed=rnd)
        al = torch.empty(B, dtype=torch.int32, device="cuda")
        an = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
        ot = torch.empty(B, Dm + 1, dtype=torch.int32, device="cuda")
        ncl = torch.empty(B, dtype=torch.int32, device="cuda")
        M.medusa_accept(t, dev(tok), g, al, an, ot, dev(P), ncl)
        M.medusa_accept_stats(t, al, an, ot, dev(tk), counts)
        torch.cuda.synchronize()
        want += accept_stats_ref(rank, Dm, al.cpu().numpy(), an.cpu().numpy(), ot.cpu().numpy(), tk)
        assert np.array_equal(counts.cpu().numpy(), want), rnd
    assert want.sum() > 3 * B
