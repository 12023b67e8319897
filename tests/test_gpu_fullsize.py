"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: the Vicuna-7B-shaped single step with the sparse 64-node tree (2048-token
cache), the same shapes with the dense 256-node tree (4096-token cache), and the
batched workload (8 sequences, vocabulary 128256, cache lengths drawn from
[1024, 8192]).

Every top-k id and every tree token is compared with the float64 oracle; the
attention output, the base model's greedy choices, the accepted branches and
the compacted caches are compared for every sequence of the single-sequence
workloads and for the shortest- and longest-cache sequences of the batched one
(the oracle's attention is the expensive part).  Integers bit-exact; floats
within 2e-2 (bf16, fp32 accumulation).
"""
import sys

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from medusa_testlib import (assert_bf16_close, enforce_greedy_gap, enforce_heads_gap, oracle_attention_seqs,
                            pv_atol, run_step_gpu, tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import speculative_decoding_medusa_amd as M
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return M


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("c", [2, 3, 4], ids=["vicuna7b_sparse64", "vicuna7b_dense256", "batched8_v128k"])
def test_full_step(M, c):
    cfg = mi.config(c)
    _say("full step", cfg.name, "B", cfg.B, "V", cfg.V, "N", cfg.N, "P", cfg.P)
    heads = mi.gen_heads(cfg)
    att = mi.gen_attention(cfg)
    root = mi.gen_root_tokens(cfg)
    ov = []
    logits_ref, z_ref = enforce_heads_gap(cfg, heads, ov)             # [K][V][B], [B][K][H]
    idx_ref, val_ref = oracle.topk(np.transpose(logits_ref, (2, 0, 1)), cfg.topk)
    del logits_ref
    P = np.asarray(cfg.P)
    seqs = sorted({int(np.argmin(P)), int(np.argmax(P))}) if cfg.B > 1 else [0]
    o_ref = oracle_attention_seqs(cfg, att, seqs)
    rows = np.stack([o_ref[b] for b in seqs]).reshape(-1, cfg.H)
    enforce_greedy_gap(cfg, heads, rows, ov)
    _say("oracle inputs ready", len(ov), "gap overrides")

    got = run_step_gpu(M, cfg, heads, att, root)

    # the residual-SiLU block's float32 output, in the launch shape the step uses
    z_err = float(np.abs(got["z"] - z_ref).max())
    _say("z max abs error", z_err)
    np.testing.assert_allclose(got["z"], z_ref, rtol=0, atol=tol(cfg.dtype))
    assert np.array_equal(got["topk_idx"], idx_ref)
    np.testing.assert_allclose(got["topk_val"], val_ref, rtol=0, atol=tol(cfg.dtype))
    parent, rank = cfg.tree.arrays()
    tok_ref, pos_ref, _ = oracle.build_tree(parent, rank, idx_ref, root, P)
    assert np.array_equal(got["node_tok"], tok_ref)
    assert np.array_equal(got["node_pos"], pos_ref)
    lm = None
    for b in seqs:
        # o_ref is already rounded to bf16 (the boundary's output type)
        vw = oracle.widen(att["v_tree"][b:b + 1], cfg.dtype)
        vcw = oracle.widen(att["v_cache"][b:b + 1, :, :P[b]], cfg.dtype)
        exact = assert_bf16_close(got["o"][b], o_ref[b], atol=pv_atol(vcw, vw, [P[b]]),
                                  what=f"attention, sequence {b}")
        _say("attention exactly rounded fraction", b, round(exact, 5))
        if lm is None:
            lm = oracle.widen(heads["lm_head"], cfg.dtype)
        g_ref, _ = oracle.base_greedy(o_ref[b].reshape(cfg.N, cfg.H), lm, 1e-6)
        assert np.array_equal(got["greedy"][b], g_ref)
        L, path, toks = oracle.accept(parent, tok_ref[b], g_ref)
        Dm = got["accept_nodes"].shape[1] - 1
        assert got["accept_len"][b] == L
        assert got["accept_nodes"][b].tolist() == path.tolist() + [-1] * (Dm - L)
        assert got["out_tokens"][b].tolist() == toks.tolist() + [-1] * (Dm - L)
        assert got["new_cache_len"][b] == P[b] + L + 1
        # compaction: slots P..P+L hold the accepted branch's keys/values
        for name, tree_kv in (("k_cache", "k_tree"), ("v_cache", "v_tree")):
            cache = got[name][b].float().cpu().numpy()                      # [nKV][Lmax][D]
            src = att[tree_kv][b]                                            # [N][nKV][D]
            exp = oracle.widen(src[path], cfg.dtype).transpose(1, 0, 2)     # [nKV][L+1][D]
            assert np.array_equal(cache[:, P[b]:P[b] + L + 1].astype(np.float64), exp)
    _say("accept_len", got["accept_len"].tolist())
