"""Device-resident generate loop around the Medusa step on the Llama-shaped
decoder.

A round runs the heads on h, builds the candidate tree from their top-k,
verifies every candidate in one pass through the decoder, keeps the longest
branch the base model agrees with (compacting every layer's cache) and hands
that branch to the next round: the bonus token becomes the root and the
hidden state at the deepest accepted node becomes h ("Medusa Heads" glossary,
section on tree attention and acceptance; the speculative-decoding e-book,
section on why a round yields the accepted tokens plus one).  Every round is
a fixed sequence of library calls on one stream that never waits for the
host, so a run of rounds can be captured in a HIP graph and replayed.

Only argument marshalling happens here; every step runs in libmedusa.
"""
from __future__ import annotations

import torch

from . import (Packed, Tree, _ws, chain_tree, decoder_workspace_size, heads_workspace_size, medusa_accept,
               medusa_accept_stats, medusa_advance, medusa_decoder_verify, medusa_heads_forward_tree,
               medusa_plant_greedy, medusa_prefill, ROW_MAJOR, PACKED, BF16, F32)


class MedusaLoop:
    """State and buffers of the loop for B sequences.

    heads: dict(w1, b1, w2) as medusa_heads_forward takes them (row-major
    tensors or pack_heads results); layers: pack_layer() dicts; embedding
    [V][H] bf16; lm_head: Packed [V][H]; k_cache, v_cache [layers][B][nKV][Lmax][D]
    bf16 holding each sequence's prefix; cache_len [B] int32 (device);
    h [B][H] (the heads' dtype) and root_tok [B] int32: the state the first
    round starts from.  max_cache_len bounds every prefix length the rounds
    reach (default Lmax - N: any state the caches can hold).  tokens [B][cap]
    collects every round's output; n_tokens [B] counts it.

    Capacity: a round grows a prefix by at most Dmax + 1 tokens (Dmax = the
    tree's depth), so from the longest starting prefix P0 (start_len, or read
    from cache_len once here) the loop can run (max_cache_len - P0) // (Dmax +
    1) rounds before a prefix could pass max_cache_len.  round() and run()
    refuse to enqueue a round beyond that (ValueError), since the device would
    otherwise only clamp the length and flag it in the tree's status word.

    planted (measurement aid): None, or the alpha of a rank prior; then after
    the verify pass the base model's choices are replaced by a continuation
    drawn from that prior (medusa_plant_greedy, keyed by plant_seed and each
    sequence's prefix length), so that random weights accept candidates the
    way a trained model would and the rounds compact deep branches."""

    def __init__(self, heads, layers, embedding, lm_head: Packed, tree: Tree, topk: int, k_cache, v_cache, nH: int,
                 cache_len, h, root_tok, max_cache_len: int | None = None, cap: int = 1024, rms_eps: float = 1e-6,
                 rope_base: float = 10000.0, start_len: int | None = None, planted: float | None = None,
                 plant_seed: int = 0):
        dev = h.device
        self.heads, self.layers, self.embedding, self.lm_head, self.tree = heads, layers, embedding, lm_head, tree
        self.topk, self.nH, self.rms_eps, self.rope_base = topk, nH, rms_eps, rope_base
        self.planted, self.plant_seed = planted, plant_seed
        self.stats = None   # counts [K][topk + 1] of medusa_accept_stats, when gathered
        self.k_cache, self.v_cache = k_cache, v_cache
        self.cache_len, self.h, self.root_tok = cache_len, h, root_tok
        n_layers, B, nKV, Lmax, D = k_cache.shape
        N, Dmax = tree.N, tree.max_depth
        V, H = embedding.shape
        w2 = heads["w2"]
        K = w2.heads if isinstance(w2, Packed) else w2.shape[0]
        self.B, self.N, self.K, self.V = B, N, K, V
        self.max_cache_len = Lmax - N if max_cache_len is None else int(max_cache_len)
        if self.max_cache_len + N > Lmax:
            raise ValueError(f"max_cache_len + N = {self.max_cache_len + N} exceeds Lmax = {Lmax}")
        self.restart(int(cache_len.max().item()) if start_len is None else int(start_len))
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_idx = torch.empty(B, K, topk, **i32)
        self.topk_val = torch.empty(B, K, topk, dtype=torch.float32, device=dev)
        self.node_tok = torch.empty(B, N, **i32)
        self.node_pos = torch.empty(B, N, **i32)
        self.greedy = torch.empty(B, N, **i32)
        self.hidden = torch.empty(B, N, H, dtype=torch.float32, device=dev)
        self.accept_len = torch.empty(B, **i32)
        self.accept_nodes = torch.empty(B, Dmax + 1, **i32)
        self.out_tokens = torch.empty(B, Dmax + 1, **i32)
        self.new_cache_len = torch.empty(B, **i32)
        self.tokens = torch.full((B, cap), -1, **i32)
        self.n_tokens = torch.zeros(B, **i32)
        layout = PACKED if isinstance(w2, Packed) else ROW_MAJOR
        dt = BF16 if h.dtype == torch.bfloat16 else F32
        self.ws_heads = _ws(heads_workspace_size(B, H, V, K, topk, dt, layout), dev, None)
        F = layers[0]["w_gate_up"].rows // 2
        self.ws_dec = _ws(decoder_workspace_size(tree, B, H, nH, nKV, D, F, V, self.max_cache_len), dev, None)

    def prefill(self, tokens, start_len: int, chunk: int = 0, stream=None):
        """Run the prompts tokens [B][T] (int32, device) through the decoder
        from the current caches (medusa_prefill): afterwards the caches hold
        their keys/values, root_tok is the greedy choice after each prompt and
        h the row that chose it -- the state the first round starts from.
        start_len: the longest prefix before the prompts (host bound).  chunk:
        tokens per pass (default: as many as 256 rows allow)."""
        B, T = tokens.shape
        C = chunk or max(1, min(256 // B, T))
        key = ("chain", C)
        if getattr(self, "_chain", None) is None or self._chain[0] != key:
            self._chain = (key, chain_tree(C))
        passes = -(-T // C)
        if start_len + passes * C > self.k_cache.shape[3]:
            raise ValueError(f"prompts of {T} tokens in passes of {C} do not fit the caches after {start_len}")
        medusa_prefill(self.layers, self.embedding, self.lm_head, self._chain[1], tokens, self.cache_len, start_len,
                       self.k_cache, self.v_cache, self.nH, self.root_tok, self.h, rms_eps=self.rms_eps,
                       rope_base=self.rope_base, stream=stream)
        self.restart(start_len + T)

    def set_tree(self, tree: Tree):
        """Use another candidate tree from the next round on (a host call
        between rounds; buffers that depend on the tree are reallocated when
        its size or depth differs)."""
        dev = self.h.device
        B, H = self.h.shape
        i32 = dict(dtype=torch.int32, device=dev)
        if tree.N != self.N:
            self.node_tok = torch.empty(B, tree.N, **i32)
            self.node_pos = torch.empty(B, tree.N, **i32)
            self.greedy = torch.empty(B, tree.N, **i32)
            self.hidden = torch.empty(B, tree.N, H, dtype=torch.float32, device=dev)
            n_layers, _, nKV, Lmax, D = self.k_cache.shape
            V = self.embedding.shape[0]
            F = self.layers[0]["w_gate_up"].rows // 2
            self.ws_dec = _ws(decoder_workspace_size(tree, B, H, self.nH, nKV, D, F, V, self.max_cache_len), dev, None)
        if tree.max_depth != self.tree.max_depth:
            self.accept_nodes = torch.empty(B, tree.max_depth + 1, **i32)
            self.out_tokens = torch.empty(B, tree.max_depth + 1, **i32)
        self.tree, self.N = tree, tree.N

    def restart(self, start_len: int):
        """Set the round budget from start_len, the longest prefix the
        sequences now hold (after the caller restored or replaced the state)."""
        if start_len > self.max_cache_len:
            raise ValueError(f"a starting prefix of {start_len} tokens exceeds max_cache_len = {self.max_cache_len}")
        self.rounds_left = (self.max_cache_len - int(start_len)) // (self.tree.max_depth + 1)

    def _reserve(self, rounds: int):
        if rounds > self.rounds_left:
            raise ValueError(f"{rounds} more rounds could grow a prefix past max_cache_len = {self.max_cache_len}: "
                             f"{self.rounds_left} fit")
        self.rounds_left -= rounds

    def round(self, stream=None):
        """One round on `stream` (torch's current stream if None)."""
        self._reserve(1)
        self._enqueue(stream)

    def _enqueue(self, stream):
        hd = self.heads
        medusa_heads_forward_tree(self.h, hd.get("w1"), hd.get("b1"), hd["w2"], self.topk, self.topk_idx,
                                  self.topk_val, self.tree, self.root_tok, self.cache_len, self.node_tok, self.node_pos,
                                  ws=self.ws_heads, stream=stream)
        medusa_decoder_verify(self.layers, self.embedding, self.lm_head, self.tree, self.node_tok, self.node_pos,
                              self.cache_len, self.max_cache_len, self.k_cache, self.v_cache, self.nH, self.greedy,
                              hidden=self.hidden, rms_eps=self.rms_eps, rope_base=self.rope_base, ws=self.ws_dec,
                              stream=stream)
        if self.planted is not None:
            medusa_plant_greedy(self.tree, self.topk_idx, self.cache_len, self.greedy, self.V, self.planted,
                                self.plant_seed, stream=stream)
        medusa_accept(self.tree, self.node_tok, self.greedy, self.accept_len, self.accept_nodes, self.out_tokens,
                      self.cache_len, self.new_cache_len, k_cache=self.k_cache, v_cache=self.v_cache, stream=stream)
        if self.stats is not None:
            medusa_accept_stats(self.tree, self.accept_len, self.accept_nodes, self.out_tokens, self.topk_idx,
                                self.stats, stream=stream)
        medusa_advance(self.tree, self.accept_len, self.accept_nodes, self.out_tokens, self.hidden, self.root_tok,
                       self.h, tokens=self.tokens, n_tokens=self.n_tokens, new_cache_len=self.new_cache_len,
                       cache_len=self.cache_len, stream=stream)

    def run(self, rounds: int, stream=None):
        self._reserve(rounds)
        for _ in range(rounds):
            self._enqueue(stream)
