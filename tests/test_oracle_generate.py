"""Pins of the generate-loop oracle (oracle/generate.py).

Greedy speculative decoding is lossless: whatever the heads guess, the rounds
must emit exactly the tokens that plain autoregressive greedy decoding emits
from the same start (one base-model pass per token), leave the same keys and
values in every layer's cache, and hand each round the hidden state plain
decoding computes for the last token it emitted; the prefix grows by the
emitted count.  The heads decide only how many tokens a round yields.  A
mistake in the tree, the acceptance, the compaction or the hand-off (wrong
path, wrong bonus token, wrong slot, wrong hidden row) breaks one of these.

Checked in float64 without bf16 rounding, on a tiny decoder whose 8-token
vocabulary makes the heads' guesses often right, so that rounds accepting
one or more candidates occur (asserted).
"""
import numpy as np

import oracle
from oracle.generate import advance, greedy_decode, medusa_round

H, NH, NKV, D, F, V, LAYERS = 64, 2, 1, 32, 96, 8, 2
K, TOPK = 3, 3
# root; depth 1: ranks 0, 1, 2; depth 2: (0,0) (0,1) (0,2) (1,0); depth 3: (0,0,0) (0,0,1)
PARENT = [-1, 0, 0, 0, 1, 1, 1, 2, 4, 4]
RANK = [0, 0, 1, 2, 0, 1, 2, 0, 0, 1]


def _model(seed):
    r = np.random.default_rng(seed)
    layers = [dict(wq=r.normal(0, .2, (NH * D, H)), wk=r.normal(0, .2, (NKV * D, H)), wv=r.normal(0, .2, (NKV * D, H)),
                   wo=r.normal(0, .2, (H, NH * D)), w_gate=r.normal(0, .2, (F, H)), w_up=r.normal(0, .2, (F, H)),
                   w_down=r.normal(0, .2, (H, F))) for _ in range(LAYERS)]
    dec = dict(embedding=r.normal(0, 1, (V, H)), layers=layers, lm_head=r.normal(0, .4, (V, H)), nH=NH, nKV=NKV)
    heads = dict(W1=r.normal(0, .1, (K, H, H)), b1=r.normal(0, .1, (K, H)), W2=r.normal(0, .4, (K, V, H)))
    B, Lmax = 2, 96
    P0 = np.array([5, 9])
    kc = [np.zeros((B, NKV, Lmax, D)) for _ in range(LAYERS)]
    vc = [np.zeros((B, NKV, Lmax, D)) for _ in range(LAYERS)]
    for l in range(LAYERS):
        for b in range(B):
            kc[l][b, :, :P0[b]] = r.normal(0, 1, (NKV, P0[b], D))
            vc[l][b, :, :P0[b]] = r.normal(0, 1, (NKV, P0[b], D))
    state = dict(h=r.normal(0, 1, (B, H)), root_tok=r.integers(0, V, B), cache_len=P0.copy(), k_caches=kc,
                 v_caches=vc)
    return dec, heads, state


def _run_rounds(dec, heads, state, rounds):
    B = state["h"].shape[0]
    emitted = [[] for _ in range(B)]
    per_round = []
    for _ in range(rounds):
        state, rec = medusa_round(state, heads, dec, PARENT, RANK, TOPK, bf16=False)
        for b in range(B):
            emitted[b] += rec["emitted"][b]
        per_round.append((state, rec, [len(e) for e in emitted]))
    return emitted, per_round


def test_rounds_emit_exactly_the_greedy_decoding():
    dec, heads, s0 = _model(11)
    emitted, per_round = _run_rounds(dec, heads, s0, rounds=6)
    n = max(len(e) for e in emitted)
    ref = greedy_decode(s0["root_tok"], s0["cache_len"], s0["k_caches"], s0["v_caches"], dec, n, bf16=False)
    # some round accepted candidates, so the tree, the path and the compaction were exercised
    assert max(max(rec["accept_len"]) for _, rec, _ in per_round) >= 1
    for b in range(len(emitted)):
        assert emitted[b] == [int(t) for t in ref["tokens"][b, :len(emitted[b])]]
    for state, rec, counts in per_round:
        for b, c in enumerate(counts):
            # prefix length: start + tokens emitted so far
            assert state["cache_len"][b] == s0["cache_len"][b] + c
            # next heads input: the hidden state that scored the last emitted token
            np.testing.assert_allclose(state["h"][b], ref["hidden"][b, c - 1], rtol=0, atol=1e-9)
            # next root: that token
            assert state["root_tok"][b] == emitted[b][c - 1]
    last = per_round[-1][0]
    for l in range(LAYERS):
        for b in range(len(emitted)):
            P = last["cache_len"][b]
            np.testing.assert_allclose(last["k_caches"][l][b, :, :P], ref["k_caches"][l][b, :, :P], rtol=0, atol=1e-9)
            np.testing.assert_allclose(last["v_caches"][l][b, :, :P], ref["v_caches"][l][b, :, :P], rtol=0, atol=1e-9)


def test_heads_change_only_the_pace():
    """Other heads, same base model: the same tokens come out (possibly over a
    different number of rounds)."""
    dec, heads, s0 = _model(11)
    _, heads2, _ = _model(12)
    a, _ = _run_rounds(dec, heads, s0, rounds=4)
    b, _ = _run_rounds(dec, heads2, s0, rounds=4)
    for x, y in zip(a, b):
        m = min(len(x), len(y))
        assert x[:m] == y[:m]


def test_advance_takes_the_deepest_accepted_row_and_the_bonus():
    """Worked example: accepted path 0 -> 2 -> 5 (L = 2), out_tokens = the two
    accepted candidates then the bonus token."""
    hidden = np.arange(6 * 4, dtype=np.float64).reshape(6, 4) + 0.5
    root, h, toks = advance(2, np.array([0, 2, 5]), np.array([17, 3, 29]), hidden, bf16=False)
    assert root == 29 and toks == [17, 3, 29]
    assert np.array_equal(h, [20.5, 21.5, 22.5, 23.5])
    # L = 0: the root alone was kept; the bonus is the model's choice after it
    root, h, toks = advance(0, np.array([0]), np.array([4]), hidden, bf16=False)
    assert root == 4 and toks == [4] and np.array_equal(h, hidden[0])
    # bf16: nearest-even rounding of the row (1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins)
    _, h, _ = advance(0, np.array([0]), np.array([0]), np.array([[1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]]), bf16=True)
    assert np.array_equal(h, [1.0, 1 + 2.0 ** -6])


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def test_prefill_equals_one_chain_tree_pass():
    # the causal token-by-token prefill equals one verify pass over the whole
    # prompt as a chain tree (every token sees the prefix and its earlier tokens)
    from oracle.decoder import decoder_verify
    from oracle.generate import prefill
    dec, _, state = _model(31)
    T = 7
    r = np.random.default_rng(5)
    prompt = r.integers(0, V, (2, T))
    pre = prefill(prompt, state["cache_len"], state["k_caches"], state["v_caches"], dec, bf16=False)
    chain = np.arange(-1, T - 1)
    one = decoder_verify(prompt, state["cache_len"], chain, dec["embedding"], dec["layers"], dec["lm_head"],
                         state["k_caches"], state["v_caches"], NH, NKV, bf16=False)
    np.testing.assert_allclose(pre["hidden_all"], one["hidden"], rtol=1e-11, atol=1e-11)
    assert np.array_equal(pre["next_tok"], one["greedy"][:, -1])
    for b in range(2):
        P = int(state["cache_len"][b])
        for l in range(LAYERS):
            np.testing.assert_allclose(pre["k_caches"][l][b, :, P:P + T], one["k_tree"][l][b].transpose(1, 0, 2),
                                       rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(pre["v_caches"][l][b, :, P:P + T], one["v_tree"][l][b].transpose(1, 0, 2),
                                       rtol=1e-11, atol=1e-11)
            assert np.array_equal(pre["k_caches"][l][b, :, :P], state["k_caches"][l][b, :, :P])
    assert np.array_equal(pre["cache_len"], state["cache_len"] + T)


def test_prefill_hands_greedy_decoding_the_same_state():
    # prefilling the whole prompt gives the token and caches that prefilling
    # all but its last token and then taking one greedy step from that token
    # gives
    from oracle.generate import greedy_decode, prefill
    dec, _, state = _model(32)
    r = np.random.default_rng(6)
    prompt = r.integers(0, V, (2, 6))
    full = prefill(prompt, state["cache_len"], state["k_caches"], state["v_caches"], dec, bf16=False)
    part = prefill(prompt[:, :-1], state["cache_len"], state["k_caches"], state["v_caches"], dec, bf16=False)
    step = greedy_decode(prompt[:, -1], part["cache_len"], part["k_caches"], part["v_caches"], dec, 1, bf16=False)
    assert np.array_equal(full["next_tok"], step["tokens"][:, 0])
    np.testing.assert_allclose(full["hidden"], step["hidden"][:, 0], rtol=1e-12, atol=1e-12)
    assert np.array_equal(full["cache_len"], step["cache_len"])
    for l in range(LAYERS):
        np.testing.assert_allclose(full["k_caches"][l], step["k_caches"][l], rtol=1e-12, atol=1e-12)
