"""Float64 oracle of the generate loop around the Medusa step -- TEST
INFRASTRUCTURE ONLY (imported by tests/ alone, never by the product path).

[MH-tree]: the longest accepted branch is kept and its final state feeds the
heads in the next round.  [SD-k+1]: a round yields its L accepted tokens plus
one more, the base model's own choice after the last accepted token; that
token starts the next round.

Readings taken (the pages print no loop):

* the heads' input of the next round is the final normalised hidden state at
  the deepest accepted node (the row lm_head scores for the extra token),
  stored in the heads' dtype (bf16: nearest even);
* the next tree's root is the extra token; after a round the cache holds the
  round's root and its L accepted tokens, so the prefix grows by L + 1;
* a prompt and its prefill lie outside the loop: a round starts from a cache,
  a root token and a hidden state; ``prefill`` produces that state from a
  prompt (every prompt token's keys/values in the cache, the greedy choice
  after the prompt as the first root, the row that chose it as the first h).

Pins (tests/test_oracle_generate.py): greedy speculative decoding is lossless
-- the rounds must emit exactly the tokens of plain autoregressive greedy
decoding (``greedy_decode``: one base-model pass per token), and their hidden
states and caches must be that decoding's; the prefix grows by the emitted
count.
"""
from __future__ import annotations

import numpy as np

from .decoder import decoder_verify
from .medusa import accept, build_tree, compact_kv, medusa_heads, round_bf16, topk, write_tree_kv

__all__ = ["advance", "medusa_round", "greedy_decode", "prefill"]


def advance(L, path, out_tokens, hidden_b, bf16):
    """Hand-off of one sequence's accepted branch [MH-tree], [SD-k+1].

    L, path [L+1], out_tokens [L+1] from ``accept``; hidden_b [N][H] the final
    normalised rows of the sequence's tree nodes.
    -> (next root token, next heads input [H], the round's emitted tokens)"""
    h = hidden_b[int(path[L])]
    return int(out_tokens[L]), (round_bf16(h) if bf16 else h.copy()), [int(t) for t in out_tokens[:L + 1]]


def medusa_round(state, heads, dec, parent, rank, topk_k, bf16=True, eps=1e-6, rope_base=10000.0):
    """One round: heads on h -> top-k -> candidate tree -> tree-verify pass
    through the decoder -> longest accepted branch -> every layer's cache
    compacted -> hand-off.

    state: dict(h [B][H], root_tok [B], cache_len [B], k_caches, v_caches:
    per layer [B][nKV][Lmax][D]); heads: dict(W1, b1, W2); dec: dict(embedding,
    layers, lm_head, nH, nKV).  All arrays float64 (bf16 values widened).
    -> (new state, record of the round's intermediate results)"""
    parent = np.asarray(parent)
    logits, _ = medusa_heads(state["h"], heads["W1"], heads["b1"], heads["W2"])
    tk_idx, tk_val = topk(logits, topk_k)
    node_tok, node_pos, _ = build_tree(parent, rank, tk_idx, state["root_tok"], state["cache_len"])
    r = decoder_verify(node_tok, state["cache_len"], parent, dec["embedding"], dec["layers"], dec["lm_head"],
                       state["k_caches"], state["v_caches"], dec["nH"], dec["nKV"], eps, rope_base, bf16)
    B = node_tok.shape[0]
    kcs, vcs = [], []
    for l in range(len(dec["layers"])):
        kc, vc = write_tree_kv(state["k_caches"][l], state["v_caches"][l], r["k_tree"][l], r["v_tree"][l],
                               state["cache_len"])
        kcs.append(kc)
        vcs.append(vc)
    new = dict(h=np.empty_like(state["h"]), root_tok=np.empty(B, dtype=np.int64),
               cache_len=np.empty(B, dtype=np.int64), k_caches=kcs, v_caches=vcs)
    rec = dict(logits=logits, topk_idx=tk_idx, topk_val=tk_val, node_tok=node_tok, node_pos=node_pos,
               greedy=r["greedy"], node_logits=r["logits"], hidden=r["hidden"], accept_len=[], path=[],
               out_tokens=[], emitted=[])
    for b in range(B):
        L, path, toks = accept(parent, node_tok[b], r["greedy"][b])
        P = int(state["cache_len"][b])
        for l in range(len(kcs)):
            kcs[l][b], newP = compact_kv(kcs[l][b], P, path)
            vcs[l][b], _ = compact_kv(vcs[l][b], P, path)
        new["cache_len"][b] = P + L + 1
        new["root_tok"][b], new["h"][b], emitted = advance(L, path, toks, r["hidden"][b], bf16)
        rec["accept_len"].append(L)
        rec["path"].append(path)
        rec["out_tokens"].append(toks)
        rec["emitted"].append(emitted)
    return new, rec


def greedy_decode(root_tok, cache_len, k_caches, v_caches, dec, n_tokens, bf16=True, eps=1e-6, rope_base=10000.0):
    """Plain autoregressive greedy decoding: one base-model pass per token (a
    one-node tree: the token sees the cache and itself), its keys/values
    appended to the cache, its argmax the next token.

    -> dict(tokens [B][n_tokens] (the tokens after root_tok), hidden
    [B][n_tokens][H] (the final normalised row of each pass: row t scored
    tokens[t]), k_caches, v_caches, cache_len)"""
    parent = np.array([-1])
    tok = np.asarray(root_tok, dtype=np.int64).copy()
    P = np.asarray(cache_len, dtype=np.int64).copy()
    kcs = [k.copy() for k in k_caches]
    vcs = [v.copy() for v in v_caches]
    toks, hid = [], []
    for _ in range(n_tokens):
        r = decoder_verify(tok[:, None], P, parent, dec["embedding"], dec["layers"], dec["lm_head"], kcs, vcs,
                           dec["nH"], dec["nKV"], eps, rope_base, bf16)
        for l in range(len(kcs)):
            kcs[l], vcs[l] = write_tree_kv(kcs[l], vcs[l], r["k_tree"][l], r["v_tree"][l], P)
        P = P + 1
        tok = r["greedy"][:, 0].astype(np.int64)
        toks.append(tok.copy())
        hid.append(r["hidden"][:, 0])
    return dict(tokens=np.stack(toks, axis=1), hidden=np.stack(hid, axis=1), k_caches=kcs, v_caches=vcs,
                cache_len=P)


def prefill(tokens, cache_len, k_caches, v_caches, dec, bf16=True, eps=1e-6, rope_base=10000.0):
    """The prompt before the first round, the plain causal way: one base-model
    pass per prompt token (a one-node tree: it sees the cache and itself),
    its keys/values appended to the cache.

    tokens [B][T] (every sequence's prompt), cache_len [B] (the prefix before
    it).  -> dict(next_tok [B] (the greedy choice after the last prompt
    token: the first round's root), hidden [B][H] (the final normalised row
    that chose it: the heads' first input), hidden_all [B][T][H], k_caches,
    v_caches, cache_len (+ T))"""
    parent = np.array([-1])
    tokens = np.asarray(tokens, dtype=np.int64)
    P = np.asarray(cache_len, dtype=np.int64).copy()
    kcs = [k.copy() for k in k_caches]
    vcs = [v.copy() for v in v_caches]
    hid = []
    for t in range(tokens.shape[1]):
        r = decoder_verify(tokens[:, t:t + 1], P, parent, dec["embedding"], dec["layers"], dec["lm_head"], kcs, vcs,
                           dec["nH"], dec["nKV"], eps, rope_base, bf16)
        for l in range(len(kcs)):
            kcs[l], vcs[l] = write_tree_kv(kcs[l], vcs[l], r["k_tree"][l], r["v_tree"][l], P)
        P = P + 1
        hid.append(r["hidden"][:, 0])
    return dict(next_tok=r["greedy"][:, 0].astype(np.int64), hidden=hid[-1], hidden_all=np.stack(hid, axis=1),
                k_caches=kcs, v_caches=vcs, cache_len=P)
