"""Float64 oracle of the Medusa step (test infrastructure only).

Conventions shared with the inputs: bfloat16 tensors arrive as uint16 bit
patterns and are widened exactly; float32 tensors are widened exactly.  Every
floating-point result is float64 unless a function says it mirrors a rounding
point of the boundary (bf16 operands, fp32 decisions).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "widen", "round_f32", "round_bf16", "silu", "medusa_heads", "lm_head_logits", "topk",
    "ancestor_matrix", "tree_depths", "build_tree", "tree_attention", "write_tree_kv",
    "rmsnorm", "base_greedy", "accept", "compact_kv", "medusa_step",
]


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor ('f32' float32, 'bf16' uint16 bits)."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Value after rounding to float32 (nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Value after rounding to float32 and then to bfloat16 (both nearest-even)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    u = u.astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# a1/a2: Medusa heads and per-head top-k  [MH-heads], [MH-tree]
# ----------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)), the activation of the
    heads' feed-forward layer [MH-heads]."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def medusa_heads(h, W1, b1, W2):
    """Logits of every Medusa head [MH-heads].

    Head k is one feed-forward layer with SiLU and a residual connection,
    followed by a projection to the vocabulary; all heads read the same last
    hidden state h:  z_k = h + SiLU(W1_k h + b1_k),  logits_k = W2_k z_k.
    Weights use the [out][in] layout of a linear layer; W2 has no bias.

    h [B][H], W1 [K][H][H], b1 [K][H], W2 [K][V][H] (float64)
    -> logits [B][K][V], z [B][K][H]
    """
    B, H = h.shape
    K = W2.shape[0]
    z = np.empty((B, K, H))
    logits = np.empty((B, K, W2.shape[1]))
    for k in range(K):
        pre = h @ W1[k].T + b1[k]          # [B][H]
        z[:, k, :] = h + silu(pre)
        logits[:, k, :] = z[:, k, :] @ W2[k].T
    return logits, z


def lm_head_logits(h, lm_head):
    """The base model's next-token scores: lm_head applied to h [MH-heads]."""
    return h @ lm_head.T


def topk(logits: np.ndarray, k: int):
    """Per-row top-k in descending order; among equal values the lower index
    ranks first [MH-tree: the heads' top guesses].

    The decision is taken on the values rounded to float32 (the precision the
    GPU accumulates in); returned values are those rounded values.
    logits [..., V] -> idx [..., k] int32, val [..., k] float64
    """
    lg = round_f32(logits)
    flat = lg.reshape(-1, lg.shape[-1])
    idx = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        order = np.lexsort((np.arange(flat.shape[1]), -flat[r]))  # key: (-value, index)
        idx[r] = order[:k]
    val = np.take_along_axis(flat, idx.astype(np.int64), axis=1)
    return idx.reshape(lg.shape[:-1] + (k,)), val.reshape(lg.shape[:-1] + (k,))


# ----------------------------------------------------------------------------
# a3: the candidate tree  [MH-tree]
# ----------------------------------------------------------------------------

def tree_depths(parent) -> np.ndarray:
    parent = np.asarray(parent)
    d = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def ancestor_matrix(parent) -> np.ndarray:
    """mask[i][j] is True iff node j is node i or one of its ancestors.

    A tree token may attend only to its ancestors in the tree [MH-tree]; the
    reading taken is that a node also sees itself, as in causal attention."""
    n = len(parent)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            m[i, j] = True
            j = parent[j] if j > 0 else -1
    return m


def build_tree(parent, rank, topk_idx, root_tok, cache_len):
    """Cartesian candidate tree [MH-tree].

    The heads' top guesses combine into candidate continuations that share
    prefixes: a node at depth d with rank r carries head d's rank-r token;
    the root carries the token the base model already chose.  Position of a
    node = cache length + depth.

    parent, rank [N]; topk_idx [B][K][k]; root_tok [B]; cache_len [B]
    -> node_tok [B][N], node_pos [B][N], mask [N][N] (bool)
    """
    depth = tree_depths(parent)
    B = topk_idx.shape[0]
    N = len(parent)
    node_tok = np.empty((B, N), dtype=np.int32)
    node_pos = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            node_tok[b, i] = root_tok[b] if i == 0 else topk_idx[b, depth[i] - 1, rank[i]]
            node_pos[b, i] = cache_len[b] + depth[i]
    return node_tok, node_pos, ancestor_matrix(parent)


# ----------------------------------------------------------------------------
# a4: tree-masked attention  [MH-tree]
# ----------------------------------------------------------------------------

def tree_attention(q, k_tree, v_tree, k_cache, v_cache, cache_len, parent, scale):
    """All candidates are scored in one pass; each sees the KV-cache prefix
    and its own tree ancestors (and itself) only [MH-tree].

    q [B][N][nH][D]; k_tree, v_tree [B][N][nKV][D];
    k_cache, v_cache [B][nKV][Lmax][D] (only slots < cache_len[b] are read);
    query head h reads KV head h // (nH / nKV).  Softmax is max-subtracted.
    -> o [B][N][nH][D] float64
    """
    B, N, nH, D = q.shape
    nKV = k_tree.shape[2]
    grp = nH // nKV
    anc = ancestor_matrix(parent)
    o = np.zeros((B, N, nH, D))
    for b in range(B):
        P = int(cache_len[b])
        for h in range(nH):
            kv = h // grp
            for i in range(N):
                vis = np.nonzero(anc[i])[0]
                keys = np.concatenate([k_cache[b, kv, :P], k_tree[b, vis, kv]], axis=0)
                vals = np.concatenate([v_cache[b, kv, :P], v_tree[b, vis, kv]], axis=0)
                s = (keys @ q[b, i, h]) * scale
                p = np.exp(s - s.max())
                o[b, i, h] = (p @ vals) / p.sum()
    return o


def write_tree_kv(k_cache, v_cache, k_tree, v_tree, cache_len):
    """The tree tokens' keys/values occupy cache slots P..P+N-1 (copies)."""
    kc, vc = k_cache.copy(), v_cache.copy()
    N = k_tree.shape[1]
    for b in range(k_cache.shape[0]):
        P = int(cache_len[b])
        kc[b, :, P:P + N] = np.transpose(k_tree[b], (1, 0, 2))
        vc[b, :, P:P + N] = np.transpose(v_tree[b], (1, 0, 2))
    return kc, vc


# ----------------------------------------------------------------------------
# a5: the base model's greedy choice at every tree node  [MH-tree]
# ----------------------------------------------------------------------------

def rmsnorm(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis (unit weight)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def base_greedy(o_rows, lm_head, eps):
    """Greedy decoding accepts a candidate when it equals the base model's top
    choice [MH-tree]; this is that top choice after each tree node.

    Reading: with synthetic attention outputs standing in for the backbone,
    the node's hidden state is RMSNorm(o) (unit weight) and its scores are
    lm_head . RMSNorm(o); the normalised row is not rounded (RMSNorm with unit
    weight is a positive factor per row, so the top choice is that of
    lm_head . o).  The argmax is taken on the float32-rounded scores, lower
    index first among equal values.

    o_rows [R][H]; lm_head [V][H] -> greedy [R] int32, logits [R][V]
    """
    n = rmsnorm(o_rows, eps)
    logits = n @ lm_head.T
    lg = round_f32(logits)
    g = np.empty(lg.shape[0], dtype=np.int32)
    for r in range(lg.shape[0]):
        g[r] = int(np.flatnonzero(lg[r] == lg[r].max())[0])
    return g, logits


# ----------------------------------------------------------------------------
# a6: greedy longest-branch acceptance  [MH-tree], [SD-k+1]
# ----------------------------------------------------------------------------

def accept(parent, node_tok, greedy):
    """Keep the longest branch the base model agrees with [MH-tree].

    A candidate at node i is accepted when its parent was accepted and its
    token equals the base model's top choice after the parent; the root is
    always kept.  L = depth of the deepest accepted node; the path is that
    node's root-to-node chain (lowest index if several, which distinct sibling
    tokens rule out).  The round yields L accepted tokens plus one more: the
    base model's choice after the last accepted node, a correction or a bonus
    token [SD-k+1].

    parent [N]; node_tok [N]; greedy [N]
    -> L, path [L+1] (node ids, path[0] = 0), out_tokens [L+1]
    """
    N = len(parent)
    depth = tree_depths(parent)
    acc = np.zeros(N, dtype=bool)
    acc[0] = True
    for i in range(1, N):
        p = parent[i]
        acc[i] = acc[p] and node_tok[i] == greedy[p]
    L = int(depth[acc].max())
    deepest = int(np.flatnonzero(acc & (depth == L))[0])
    path = []
    j = deepest
    while j >= 0:
        path.append(j)
        j = parent[j] if j > 0 else -1
    path = path[::-1]
    tokens = [int(node_tok[n]) for n in path[1:]] + [int(greedy[deepest])]
    return L, np.asarray(path, dtype=np.int32), np.asarray(tokens, dtype=np.int32)


# ----------------------------------------------------------------------------
# a7: accepted-path KV hand-off
# ----------------------------------------------------------------------------

def compact_kv(cache, P, path):
    """The accepted branch's final state feeds the next round [MH-tree]; its
    keys/values must therefore persist as ordinary cache entries.  For
    d = 0..L, slot P+d receives what slot P+path[d] held (every source is read
    before any slot is written); the new cache length is P + L + 1.

    cache [..., Lmax, D] (any leading axes); returns (new cache, new length).
    """
    out = cache.copy()
    src = cache[..., [P + int(p) for p in path], :].copy()
    out[..., P:P + len(path), :] = src
    return out, P + len(path)


# ----------------------------------------------------------------------------
# One whole step (synthetic tree q/k/v), chaining the above
# ----------------------------------------------------------------------------

def medusa_step(x: dict, parent, rank, topk_k: int, dtype: str, eps: float = 1e-6):
    """The whole step on widened inputs: heads -> top-k -> tree -> tree
    attention -> base greedy per node -> accept -> compaction.

    In bf16 workloads the attention output is stored in bf16 (the boundary's
    output type), so it is rounded before the greedy stage.
    """
    bf = dtype == "bf16"
    logits, z = medusa_heads(x["h"], x["W1"], x["b1"], x["W2"])
    tk_idx, tk_val = topk(logits, topk_k)
    node_tok, node_pos, mask = build_tree(parent, rank, tk_idx, x["root_tok"], x["cache_len"])
    D = x["q"].shape[-1]
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o = tree_attention(x["q"], x["k_tree"], x["v_tree"], x["k_cache"], x["v_cache"],
                       x["cache_len"], parent, scale)
    if bf:
        o = round_bf16(o)
    B, N = node_tok.shape
    g, node_logits = base_greedy(o.reshape(B * N, -1), x["lm_head"], eps)
    g = g.reshape(B, N)
    kc, vc = write_tree_kv(x["k_cache"], x["v_cache"], x["k_tree"], x["v_tree"], x["cache_len"])
    res = dict(logits=logits, z=z, topk_idx=tk_idx, topk_val=tk_val, node_tok=node_tok,
               node_pos=node_pos, mask=mask, o=o, greedy=g, node_logits=node_logits.reshape(B, N, -1),
               accept_len=[], path=[], out_tokens=[], new_cache_len=[], k_cache=kc, v_cache=vc)
    for b in range(B):
        L, path, toks = accept(parent, node_tok[b], g[b])
        P = int(x["cache_len"][b])
        res["k_cache"][b], newP = compact_kv(res["k_cache"][b], P, path)
        res["v_cache"][b], _ = compact_kv(res["v_cache"][b], P, path)
        res["accept_len"].append(L)
        res["path"].append(path)
        res["out_tokens"].append(toks)
        res["new_cache_len"].append(newP)
    return res
