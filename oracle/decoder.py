"""Float64 oracle of the tree-verify forward pass through a Llama-shaped
decoder (test infrastructure only).

[MH-tree]: in the next forward pass every candidate is appended to the input
at once and the attention mask lets each token see only its tree ancestors;
the base model scores all branches in parallel.  That forward pass is a whole
decoder, so the verify step of the 32-layer workload runs every tree token
through every layer with the tree-masked attention of ``tree_attention``.

The pages fix no decoder internals; the layer is the standard Llama shape the
workload names (readings taken):

* pre-norm residual blocks: x += Wo . Attn(RoPE(Wq n), RoPE(Wk n), Wv n) with
  n = RMSNorm(x); then x += Wdown . (SiLU(Wgate n') * (Wup n')) with
  n' = RMSNorm(x); a final RMSNorm before lm_head;
* RMSNorm with unit weight and eps 1e-6 (the weights drawn N(0, 0.02) are the
  linear and embedding matrices);
* rotary embedding with base 10000 that rotates the pair (i, i + D/2) of each
  head by the angle pos * base^(-2i/D) ("rotate-half" pairing);
* a tree token at depth d has position cache_len + d;
* attention scale 1/sqrt(D); the embedding and lm_head are separate matrices.

With ``bf16=True`` the values the GPU path stores in bfloat16 are rounded
here too (nearest even): the normalised rows fed to every product, the
rotated q/k and v fed to attention, the attention output, and the SwiGLU
product.  The residual stream stays unrounded (float64 here, float32 there).
With ``bf16=False`` nothing is rounded (used by the pins).
"""
from __future__ import annotations

import numpy as np

from .medusa import ancestor_matrix, rmsnorm, round_bf16, silu, tree_attention, tree_depths

__all__ = ["rope", "decoder_layer", "decoder_verify"]


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding over the last axis (length D, even).

    Pair (i, i + D/2) is rotated by angle pos * base^(-2i/D):
      out[i]       = x[i] cos - x[i + D/2] sin
      out[i + D/2] = x[i + D/2] cos + x[i] sin
    x [..., T, nHeads, D] with pos [..., T] broadcast over the heads."""
    D = x.shape[-1]
    half = D // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / D)          # [half]
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv        # [..., T, 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def decoder_layer(x, W, k_cache, v_cache, cache_len, parent, node_pos, nH, nKV, eps, rope_base, bf16):
    """One pre-norm decoder layer over the tree tokens.

    x [B][N][H] residual stream; W dict of wq, wk, wv, wo [H][H], w_gate, w_up
    [F][H], w_down [H][F] (float64, [out][in]); k_cache, v_cache [B][nKV][Lmax][D]
    (the prefix, already rotated); node_pos [B][N].
    -> new x, the layer's tree keys (rotated) and values [B][N][nKV][D]."""
    rnd = round_bf16 if bf16 else (lambda a: a)
    B, N, H = x.shape
    D = H // nH
    n = rnd(rmsnorm(x, eps))
    q = (n @ W["wq"].T).reshape(B, N, nH, D)
    k = (n @ W["wk"].T).reshape(B, N, nKV, D)
    v = (n @ W["wv"].T).reshape(B, N, nKV, D)
    q = rnd(rope(q, node_pos, rope_base))
    k = rnd(rope(k, node_pos, rope_base))
    v = rnd(v)
    o = tree_attention(q, k, v, k_cache, v_cache, cache_len, parent, 1.0 / np.sqrt(D))
    o = rnd(o).reshape(B, N, H)
    x = x + o @ W["wo"].T
    n2 = rnd(rmsnorm(x, eps))
    a = rnd(silu(n2 @ W["w_gate"].T) * (n2 @ W["w_up"].T))
    x = x + a @ W["w_down"].T
    return x, k, v


def decoder_verify(node_tok, cache_len, parent, embedding, layers, lm_head, k_caches, v_caches, nH, nKV,
                   eps=1e-6, rope_base=10000.0, bf16=True):
    """The tree-verify forward pass: embed the tree tokens, run every layer
    with tree-masked attention over that layer's prefix cache, normalise, and
    take the base model's greedy choice after every node ([MH-tree]: greedy
    acceptance compares each candidate with the model's top choice).

    node_tok [B][N]; cache_len [B]; embedding, lm_head [V][H]; layers: list of
    weight dicts; k_caches, v_caches: per layer [B][nKV][Lmax][D].
    -> dict(greedy [B][N] int32, logits [B][N][V], hidden [B][N][H] (the final
    normalised rows), x (residual stream before the final norm), k_tree,
    v_tree (per layer, [B][N][nKV][D]))."""
    rnd = round_bf16 if bf16 else (lambda a: a)
    node_tok = np.asarray(node_tok)
    B, N = node_tok.shape
    depth = tree_depths(parent)
    node_pos = np.asarray(cache_len)[:, None] + depth[None, :]
    x = embedding[node_tok]                                   # [B][N][H]
    k_tree, v_tree = [], []
    for l, W in enumerate(layers):
        x, k, v = decoder_layer(x, W, k_caches[l], v_caches[l], cache_len, parent, node_pos, nH, nKV, eps,
                                rope_base, bf16)
        k_tree.append(k)
        v_tree.append(v)
    hidden = rnd(rmsnorm(x, eps))
    logits = hidden @ lm_head.T
    lg = logits.astype(np.float32).astype(np.float64)
    greedy = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            greedy[b, i] = int(np.flatnonzero(lg[b, i] == lg[b, i].max())[0])
    return dict(greedy=greedy, logits=logits, hidden=hidden, x=x, k_tree=k_tree, v_tree=v_tree,
                mask=ancestor_matrix(parent))
