"""Helpers shared by the tests and the golden-value script.

* ``enforce_gaps``: make every integer decision of a workload robust: the
  oracle's consecutive gaps among each head's top-(k+1) logits, and between
  each node's best two base logits, must be at least ``gap``.  Violations are
  removed by redrawing the lower-ranked row of W2 (or lm_head) from its own
  stream (an "override"), which changes no other input.
* ``widen_inputs``: the float64 view of generated inputs the oracle consumes.
* device helpers (only used by GPU tests).
"""
from __future__ import annotations

import numpy as np

import medusa_inputs as mi
import oracle

GAP = 1e-2


def widen_inputs(cfg, heads, att, root_tok):
    dt = cfg.dtype
    x = {k: oracle.widen(v, dt) for k, v in heads.items()}
    for k in ("k_cache", "v_cache", "q", "k_tree", "v_tree"):
        x[k] = oracle.widen(att[k], dt)
    x["cache_len"] = np.asarray(att["cache_len"])
    x["root_tok"] = np.asarray(root_tok)
    return x


def _oracle_z(cfg, heads):
    dt = cfg.dtype
    h = oracle.widen(heads["h"], dt)
    z = np.empty((cfg.B, cfg.K, cfg.H))
    for k in range(cfg.K):
        W1 = oracle.widen(heads["W1"][k], dt)
        b1 = oracle.widen(heads["b1"][k], dt)
        z[:, k] = h + oracle.silu(h @ W1.T + b1)
    return z


def _row_logits(W, rows, z, dt):
    return oracle.widen(W[rows], dt) @ z.T  # [rows][B]


def _top(lg, n):
    order = np.lexsort((np.arange(lg.shape[0]), -oracle.round_f32(lg)))
    return order[:n]


def enforce_heads_gap(cfg, heads, overrides, gap=GAP, max_iter=200):
    """Redraw W2 rows until every (b, head) has top-(k+1) gaps >= gap."""
    dt = cfg.dtype
    z = _oracle_z(cfg, heads)
    logits = np.empty((cfg.K, cfg.V, cfg.B))
    for k in range(cfg.K):
        for r0 in range(0, cfg.V, 8192):
            logits[k, r0:r0 + 8192] = _row_logits(heads["W2"][k], slice(r0, r0 + 8192), z[:, k], dt)
    for _ in range(max_iter):
        bad = []
        for k in range(cfg.K):
            for b in range(cfg.B):
                lg = logits[k, :, b]
                top = _top(lg, cfg.topk + 1)
                for j in range(cfg.topk):
                    if lg[top[j]] - lg[top[j + 1]] < gap:
                        bad.append((k, int(top[j + 1])))
                        break
        if not bad:
            return logits, z
        for k, row in sorted(set(bad)):
            o = {"tensor": "W2", "head": k, "row": row, "serial": len(overrides)}
            overrides.append(o)
            mi.apply_overrides(cfg, heads, [o])
            logits[k, row] = _row_logits(heads["W2"][k], [row], z[:, k], dt)[0]
    raise RuntimeError("heads gap enforcement did not converge")


def node_hidden(cfg, att):
    """Oracle attention output per node, rounded like the boundary's output
    type, flattened to [B*N][nH*D]."""
    dt = cfg.dtype
    parent, _ = cfg.tree.arrays()
    w = {k: oracle.widen(att[k], dt) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    scale = float(np.float32(1.0 / np.sqrt(cfg.D)))
    o = oracle.tree_attention(w["q"], w["k_tree"], w["v_tree"], w["k_cache"], w["v_cache"], att["cache_len"],
                              parent, scale)
    if dt == "bf16":
        o = oracle.round_bf16(o)
    return o


def enforce_greedy_gap(cfg, heads, o, overrides, eps=1e-6, gap=GAP, max_iter=200):
    """Redraw lm_head rows until every node's best two base logits differ by >= gap.
    ``o``: node hidden rows (any shape ending in H)."""
    dt = cfg.dtype
    rows = o.reshape(-1, cfg.H)
    n = oracle.rmsnorm(rows, eps)
    logits = np.empty((cfg.V, n.shape[0]))
    for r0 in range(0, cfg.V, 8192):
        logits[r0:r0 + 8192] = oracle.widen(heads["lm_head"][r0:r0 + 8192], dt) @ n.T
    for _ in range(max_iter):
        bad = set()
        for r in range(n.shape[0]):
            top = _top(logits[:, r], 2)
            if logits[top[0], r] - logits[top[1], r] < gap:
                bad.add(int(top[1]))
        if not bad:
            return logits.T
        for row in sorted(bad):
            ov = {"tensor": "lm_head", "row": row, "serial": len(overrides)}
            overrides.append(ov)
            mi.apply_overrides(cfg, heads, [ov])
            logits[row] = oracle.widen(heads["lm_head"][row], dt) @ n.T
    raise RuntimeError("greedy gap enforcement did not converge")


def make_workload(cfg, overrides=None, enforce=True):
    """Generate every input of a workload; apply (or compute) gap overrides."""
    heads = mi.gen_heads(cfg)
    att = mi.gen_attention(cfg)
    root = mi.gen_root_tokens(cfg)
    if overrides is not None:
        mi.apply_overrides(cfg, heads, overrides)
        return heads, att, root, list(overrides)
    ov = []
    if enforce:
        enforce_heads_gap(cfg, heads, ov)
        o = node_hidden(cfg, att)
        enforce_greedy_gap(cfg, heads, o, ov)
    return heads, att, root, ov


# ---------------------------------------------------------------------------
# device helpers
# ---------------------------------------------------------------------------

def dev(arr, dtype_str=None):
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host_f64(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.detach().cpu().numpy().astype(np.float64)


def tol(dtype_str):
    return 1e-4 if dtype_str == "f32" else 2e-2


def bf16_step(x):
    """One bf16 step (unit in the last place) at the magnitude of x."""
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


def pv_atol(v_cache, v_tree, cache_len):
    """Absolute accuracy of the bf16 attention path before its output is
    rounded: each probability enters the P.V product with 17 significant bits
    (a bf16 head plus a bf16 remainder), so an output, a convex combination of
    values, is off by at most 2^-17 max|v| (plus float32 accumulation, far
    smaller); twice that.  Matters only for outputs near 0, where one bf16
    step is smaller still."""
    m = float(np.abs(v_tree).max())
    for b, P in enumerate(np.asarray(cache_len)):
        if P > 0:
            m = max(m, float(np.abs(v_cache[b, :, :P]).max()))
    return 2.0 ** -16 * m


def assert_bf16_close(got, ref, min_exact=0.99, atol=1e-6, what=""):
    """bf16 outputs against float64 oracle values: every element within one
    bf16 step of the oracle value rounded to bf16 (a rounding flip at most;
    atol covers values near 0), and at least ``min_exact`` of them equal to it.
    Well inside 2e-2 everywhere, and tight enough that a wrong mask or scale
    (moves of a few 1e-3 on outputs of size 0.04) fails."""
    rb = oracle.round_bf16(ref)
    err = np.abs(np.asarray(got, dtype=np.float64) - rb)
    lim = bf16_step(ref) + atol
    bad = err > lim
    exact = float(np.mean(err == 0))
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements beyond one bf16 step; "
                           f"worst {float((err - lim).max()):.3g} past it")
    assert exact >= min_exact, f"{what}: only {exact:.4f} of the elements equal the rounded oracle"
    return exact


# ---------------------------------------------------------------------------
# one whole step on the GPU, in the call sequence and launch shapes bench.py
# times (the same C-ABI calls with the same arguments)
# ---------------------------------------------------------------------------

def lm_head_arg(M, lm_head):
    """The lm_head argument of medusa_base_greedy as a step passes it: bf16
    weights packed for the MFMA product when H allows it (H % 64 == 0), else
    the row-major tensor (vector GEMV).  Returns (argument, layout)."""
    import torch
    if lm_head.dtype == torch.bfloat16 and lm_head.shape[1] % 64 == 0:
        return M.pack(lm_head), M.PACKED
    return lm_head, M.ROW_MAJOR


def head_weights_arg(M, W1, W2, B):
    """The heads' W1 and W2 as a step passes them: packed for the MFMA
    products from 4 sequences on (bf16, H % 128 == 0), else the row-major
    tensors (vector-ALU GEMVs)."""
    import torch
    if B >= 4 and W2.dtype == torch.bfloat16 and W2.shape[2] % 128 == 0:
        return M.pack_heads(W1), M.pack_heads(W2)
    return W1, W2


def run_step_gpu(M, cfg, heads, att, root):
    """Upload the workload, run the heads with the tree build (the one call
    bench.py times) -> tree_attention_verify -> base_greedy -> accept (with
    compaction) once and return host copies of every output; z comes from a
    separate medusa_resid_silu call on the same inputs."""
    import torch
    d = {k: dev(v) for k, v in {**heads, **att}.items()}
    B, K, H, V, N, topk = cfg.B, cfg.K, cfg.H, cfg.V, cfg.N, cfg.topk
    parent, rank = cfg.tree.arrays()
    tree = M.Tree(parent, rank, K, topk)
    wdt = M.BF16 if cfg.dtype == "bf16" else M.F32
    z = torch.empty(B, K, H, device="cuda")
    ti = torch.empty(B, K, topk, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, topk, device="cuda")
    w1, w2 = head_weights_arg(M, d["W1"], d["W2"], B)
    w2_layout = M.PACKED if isinstance(w2, M.Packed) else M.ROW_MAJOR
    ws_h = torch.empty(M.heads_workspace_size(B, H, V, K, topk, wdt, w2_layout), dtype=torch.uint8, device="cuda")
    tok = torch.empty(B, N, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    o = torch.empty_like(d["q"])
    maxP = max(cfg.P)
    ws_a = torch.empty(M.tree_attention_workspace_size(tree, B, cfg.nH, cfg.D, maxP, wdt), dtype=torch.uint8,
                       device="cuda")
    g = torch.empty(B * N, dtype=torch.int32, device="cuda")
    lm, layout = lm_head_arg(M, d["lm_head"])
    ws_g = torch.empty(M.base_greedy_workspace_size(B * N, H, V, wdt, layout), dtype=torch.uint8, device="cuda")
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, tree.max_depth + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty_like(an)
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")
    M.medusa_resid_silu(d["h"], w1, d["b1"], z)
    M.medusa_heads_forward_tree(d["h"], w1, d["b1"], w2, topk, ti, tv, tree, dev(root), d["cache_len"], tok, pos,
                                ws=ws_h)
    M.tree_attention_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"], d["cache_len"], maxP, tree, o,
                            ws=ws_a)
    M.medusa_base_greedy(o, lm, g, ws=ws_g)
    M.medusa_accept(tree, tok, g.view(B, N), al, an, ot, d["cache_len"], ncl, k_cache=d["k_cache"],
                    v_cache=d["v_cache"])
    torch.cuda.synchronize()
    out = dict(z=host_f64(z), topk_idx=ti.cpu().numpy(), topk_val=host_f64(tv), node_tok=tok.cpu().numpy(),
               node_pos=pos.cpu().numpy(), o=host_f64(o), greedy=g.view(B, N).cpu().numpy(),
               accept_len=al.cpu().numpy(), accept_nodes=an.cpu().numpy(), out_tokens=ot.cpu().numpy(),
               new_cache_len=ncl.cpu().numpy(), k_cache=d["k_cache"], v_cache=d["v_cache"])
    del d, lm, w1, w2
    return out


def oracle_attention_seqs(cfg, att, seqs):
    """Oracle tree attention for every node and head of the listed sequences,
    rounded like the boundary's output type: {b: o[N][nH][D]}."""
    dt = cfg.dtype
    parent, _ = cfg.tree.arrays()
    scale = float(np.float32(1.0 / np.sqrt(cfg.D)))
    res = {}
    for b in seqs:
        sl = slice(b, b + 1)
        w = {k: oracle.widen(att[k][sl], dt) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
        o = oracle.tree_attention(w["q"], w["k_tree"], w["v_tree"], w["k_cache"], w["v_cache"],
                                  np.asarray(att["cache_len"])[sl], parent, scale)[0]
        res[b] = oracle.round_bf16(o) if dt == "bf16" else o
    return res


# ---------------------------------------------------------------------------
# host reference of medusa_plant_greedy (a measurement aid: the planted
# continuation drawn from the rank prior with a counter hash)
# ---------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def mix64(z: int) -> int:
    """The 64-bit finaliser of SplitMix64 (Steele, Lea and Flood, OOPSLA'14)."""
    z = (z + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def planted_next_tokens(topk_idx_b, K, topk, P, max_depth, alpha, seed, b, V):
    """Token after a node of depth d = 0..max_depth for one sequence."""
    out = []
    for d in range(max_depth + 1):
        z = mix64(mix64(mix64((seed ^ b) & _M64) ^ (P & 0xFFFFFFFF)) ^ d)
        u = np.float32(z >> 40) * np.float32(1.0 / 16777216.0)
        cand = [int(x) for x in topk_idx_b[min(d, K - 1)]]
        a = alpha[min(d, len(alpha) - 1, 15)] if hasattr(alpha, "__len__") else alpha
        r = topk
        if d < K:
            cum, pr = np.float32(0), np.float32(a)
            for j in range(topk):
                cum = np.float32(cum + pr)
                if u < cum:
                    r = j
                    break
                pr = np.float32(pr * np.float32(1.0 - np.float32(a)))
        if r < topk:
            tok = cand[r]
        else:
            tok = (mix64(z) >> 33) % V
            if d < K:
                for _ in range(topk + 1):
                    if tok not in cand:
                        break
                    tok = tok + 1 if tok + 1 < V else 0
        out.append(int(tok))
    return out


def planted_greedy_ref(depth, topk_idx, cache_len, alpha, seed, V):
    """greedy [B][N] as medusa_plant_greedy writes it."""
    depth = np.asarray(depth)
    B, K, topk = topk_idx.shape
    g = np.empty((B, len(depth)), dtype=np.int32)
    for b in range(B):
        nxt = planted_next_tokens(topk_idx[b], K, topk, int(cache_len[b]), int(depth.max()), alpha, seed, b, V)
        g[b] = [nxt[d] for d in depth]
    return g


def accept_stats_ref(rank, Dmax, accept_len, accept_nodes, out_tokens, topk_idx):
    """counts [K][topk + 1] that one round of medusa_accept_stats adds."""
    B, K, topk = topk_idx.shape
    c = np.zeros((K, topk + 1), dtype=np.int64)
    for b in range(B):
        L = int(accept_len[b])
        for d in range(1, L + 1):
            c[d - 1, rank[accept_nodes[b, d]]] += 1
        if L + 1 <= K:
            cand = list(topk_idx[b, L])
            tok = int(out_tokens[b, L])
            c[L, cand.index(tok) if tok in cand else topk] += 1
    return c
