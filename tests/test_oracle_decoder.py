"""Pins of the decoder oracle (the tree-verify forward pass of the 32-layer
workload).

* Every root-to-leaf branch of the tree pass must equal running that branch as
  an ordinary causal sequence through an independent Llama implementation
  (Hugging Face transformers' LlamaModel, float64, CPU) whose KV cache holds
  the same prefix: this pins the layer structure, RMSNorm, the rotary
  pairing and positions (cache length + depth), SwiGLU, the residuals and the
  ancestor mask at once.
* RoPE against closed forms and invariants.
"""
import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from oracle.decoder import decoder_verify, rope


def _weights(L, H, F, V, seed):
    r = np.random.default_rng(seed)
    layers = []
    for _ in range(L):
        layers.append(dict(wq=r.normal(0, .15, (H, H)), wk=r.normal(0, .15, (H, H)), wv=r.normal(0, .15, (H, H)),
                           wo=r.normal(0, .15, (H, H)), w_gate=r.normal(0, .15, (F, H)),
                           w_up=r.normal(0, .15, (F, H)), w_down=r.normal(0, .15, (H, F))))
    return layers, r.normal(0, 1, (V, H)), r.normal(0, .1, (V, H))


@pytest.fixture
def hf_float64(monkeypatch):
    """The library deliberately keeps RMSNorm's mean square and the attention
    softmax in float32 (and builds float32 rotary tables); for a float64
    reference those three are switched to float64 for the test's duration.
    The formulas are unchanged."""
    import transformers.models.llama.modeling_llama as ml

    def rms(self, x):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.variance_epsilon) * self.weight

    softmax = torch.nn.functional.softmax
    monkeypatch.setattr(ml.LlamaRMSNorm, "forward", rms)
    monkeypatch.setattr(ml.nn.functional, "softmax", lambda x, dim=None, dtype=None, **kw: softmax(x, dim=dim))
    return ml


def _hf_model(layers, emb, H, nH, nKV, F, V):
    from transformers import LlamaConfig, LlamaModel
    cfg = LlamaConfig(vocab_size=V, hidden_size=H, intermediate_size=F, num_hidden_layers=len(layers),
                      num_attention_heads=nH, num_key_value_heads=nKV, rms_norm_eps=1e-6, rope_theta=10000.0,
                      max_position_embeddings=512, attn_implementation="eager")
    m = LlamaModel(cfg).double().eval()
    with torch.no_grad():
        m.embed_tokens.weight.copy_(torch.from_numpy(emb))
        for l, W in enumerate(layers):
            lay = m.layers[l]
            lay.self_attn.q_proj.weight.copy_(torch.from_numpy(W["wq"]))
            lay.self_attn.k_proj.weight.copy_(torch.from_numpy(W["wk"][:nKV * (H // nH)]))
            lay.self_attn.v_proj.weight.copy_(torch.from_numpy(W["wv"][:nKV * (H // nH)]))
            lay.self_attn.o_proj.weight.copy_(torch.from_numpy(W["wo"]))
            lay.mlp.gate_proj.weight.copy_(torch.from_numpy(W["w_gate"]))
            lay.mlp.up_proj.weight.copy_(torch.from_numpy(W["w_up"]))
            lay.mlp.down_proj.weight.copy_(torch.from_numpy(W["w_down"]))
            lay.input_layernorm.weight.fill_(1.0)
            lay.post_attention_layernorm.weight.fill_(1.0)
        m.norm.weight.fill_(1.0)
    # float64 rotary tables (frequency base^(-2i/D), pinned separately below)
    m.rotary_emb = _Rotary64(H // nH, 10000.0)
    return m


class _Rotary64(torch.nn.Module):
    def __init__(self, D, base):
        super().__init__()
        self.inv = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)

    def forward(self, x, position_ids):
        f = position_ids[..., None].double() * self.inv
        e = torch.cat((f, f), dim=-1)
        return e.cos().to(x.dtype), e.sin().to(x.dtype)


@pytest.mark.parametrize("tree,nH,nKV,P", [(mi.tiny_tree(), 4, 4, (5, 0)), (mi.sparse_tree(24), 4, 2, (7,)),
                                           (mi.chain_tree(4), 2, 2, (3,))])
def test_every_branch_equals_hf_llama_causal(hf_float64, tree, nH, nKV, P):
    from transformers import DynamicCache
    L, H, F, V = 2, 64, 96, 40
    D = H // nH
    layers, emb, lm_head = _weights(L, H, F, V, 11)
    for W in layers:  # GQA: the oracle reads only the first nKV heads' rows of wk / wv
        W["wk"] = W["wk"][:nKV * D]
        W["wv"] = W["wv"][:nKV * D]
    r = np.random.default_rng(12)
    B, N = len(P), tree.n
    Lmax = max(P) + N + 2
    kc = [r.normal(0, 1, (B, nKV, Lmax, D)) for _ in range(L)]
    vc = [r.normal(0, 1, (B, nKV, Lmax, D)) for _ in range(L)]
    tok = r.integers(0, V, (B, N))
    parent, _ = tree.arrays()
    res = decoder_verify(tok, np.asarray(P), parent, emb, layers, lm_head, kc, vc, nH, nKV, bf16=False)
    model = _hf_model(layers, emb, H, nH, nKV, F, V)
    leaves = [i for i in range(N) if i not in set(parent.tolist())]
    for b in range(B):
        for leaf in leaves:
            path = []
            j = leaf
            while j >= 0:
                path.append(j)
                j = parent[j] if j > 0 else -1
            path = path[::-1]
            cache = DynamicCache()
            for l in range(L):
                cache.update(torch.from_numpy(kc[l][b:b + 1, :, :P[b]].copy()),
                             torch.from_numpy(vc[l][b:b + 1, :, :P[b]].copy()), l)
            ids = torch.from_numpy(tok[b, path][None].astype(np.int64))
            pos = torch.arange(P[b], P[b] + len(path))[None]
            with torch.no_grad():
                out = model(input_ids=ids, position_ids=pos, past_key_values=cache, use_cache=True)
            np.testing.assert_allclose(res["hidden"][b, path], out.last_hidden_state[0].numpy(), rtol=0, atol=1e-11)
    # greedy = argmax of lm_head . hidden, lower index first
    lg = res["hidden"] @ lm_head.T
    assert np.array_equal(res["greedy"], lg.astype(np.float32).argmax(-1))


def test_rope_closed_forms():
    # D = 2: a plain rotation of (x0, x1) by pos radians (base^0 = 1)
    x = np.array([[[[1.0, 0.0]]]])
    for p in (0, 1, 2.5):
        y = rope(x, np.array([[p]]))
        np.testing.assert_allclose(y[0, 0, 0], [np.cos(p), np.sin(p)], rtol=0, atol=1e-15)
    # position 0 is the identity; norms are preserved
    r = np.random.default_rng(0)
    q = r.normal(0, 1, (1, 3, 2, 16))
    np.testing.assert_array_equal(rope(q, np.zeros((1, 3))), q)
    pos = np.array([[5, 17, 300]])
    np.testing.assert_allclose(np.linalg.norm(rope(q, pos), axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # pair (i, i + D/2) at frequency base^(-2i/D): i = 1, D = 16 -> angle pos * 10000^(-1/8)
    e = np.zeros((1, 1, 1, 16)); e[..., 1] = 1.0
    y = rope(e, np.array([[7]]))
    a = 7 * 10000.0 ** (-1 / 8)
    np.testing.assert_allclose([y[0, 0, 0, 1], y[0, 0, 0, 9]], [np.cos(a), np.sin(a)], rtol=0, atol=1e-15)


def test_rope_scores_depend_on_relative_position_only():
    r = np.random.default_rng(1)
    q, k = r.normal(0, 1, (1, 1, 1, 32)), r.normal(0, 1, (1, 1, 1, 32))
    s = lambda m, n: float((rope(q, np.array([[m]])) * rope(k, np.array([[n]]))).sum())
    for m, n, shift in ((3, 1, 10), (100, 40, 2048), (0, 0, 77)):
        assert abs(s(m, n) - s(m + shift, n + shift)) < 1e-10


def test_bf16_mirror_changes_only_rounding():
    # with bf16 rounding the hidden rows move by bf16-sized amounts, not more
    L, H, F, V, nH = 1, 64, 96, 40, 4
    layers, emb, lm_head = _weights(L, H, F, V, 21)
    r = np.random.default_rng(22)
    tree = mi.tiny_tree()
    parent, _ = tree.arrays()
    kc = [r.normal(0, 1, (1, nH, 12, H // nH))]
    vc = [r.normal(0, 1, (1, nH, 12, H // nH))]
    tok = r.integers(0, V, (1, tree.n))
    a = decoder_verify(tok, np.array([3]), parent, emb, layers, lm_head, kc, vc, nH, nH, bf16=False)["hidden"]
    b = decoder_verify(tok, np.array([3]), parent, emb, layers, lm_head, kc, vc, nH, nH, bf16=True)["hidden"]
    assert 0 < np.abs(a - b).max() < 0.05
