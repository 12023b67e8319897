"""Python binding of libmedusa.so, the HIP (gfx950) implementation of one
Medusa decoding step.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the path runs in the library's kernels.  The
functions carry the names of the C entry points declared in
include/medusa.h.  There is no fallback: if the library is missing, importing
this package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_medusa_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
STATUS_CACHE_LEN_CLAMPED, STATUS_CACHE_OVERFLOW = 1, 2
F32, BF16 = 0, 1
ROW_MAJOR, PACKED = 0, 1

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "medusa_last_error": ([], ctypes.c_char_p),
    "medusa_version": ([], ctypes.c_char_p),
    "medusa_resid_silu": ([_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp], _i32),
    "medusa_vocab_topk_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "medusa_vocab_topk": ([_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "medusa_heads_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "medusa_heads_forward": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                              _vp], _i32),
    "medusa_heads_forward_static": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                     _vp], _i32),
    "medusa_tree_create": ([_vp, _vp, _i32, _i32, _i32, ctypes.POINTER(_vp)], _i32),
    "medusa_tree_destroy": ([_vp], None),
    "medusa_tree_num_nodes": ([_vp], _i32),
    "medusa_tree_max_depth": ([_vp], _i32),
    "medusa_tree_mask_host": ([_vp, _vp, _sz], _i32),
    "medusa_tree_status": ([_vp, ctypes.POINTER(ctypes.c_int32), _i32, _vp], _i32),
    "medusa_build_tree": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp], _i32),
    "medusa_heads_forward_tree": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "tree_attention_workspace_size": ([_vp, _i32, _i32, _i32, _i32, _i32], _sz),
    "tree_attention_verify": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                               _vp, _vp, _sz, _vp], _i32),
    "medusa_packed_size": ([_i32, _i32], _sz),
    "medusa_pack_rows": ([_vp, _i32, _i32, _vp, _i32, _i32, _i32, _vp], _i32),
    "medusa_base_greedy_workspace_size": ([_i32, _i32, _i32, _i32, _i32], _sz),
    "medusa_base_greedy": ([_vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "medusa_accept": ([_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32,
                       _vp], _i32),
    "medusa_typical_accept_workspace_size": ([_vp, _i32], _sz),
    "medusa_typical_accept": ([_vp, _vp, _vp, _i32, _i32, _f32, _f32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _i32, _i64, _i32, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "medusa_speculative_sample": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "medusa_advance": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp], _i32),
    "medusa_plant_greedy": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, ctypes.c_uint64, _vp, _vp], _i32),
    "medusa_accept_stats": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp], _i32),
    "medusa_tree_select": ([_vp, _i32, _i32, _i32, _vp, _vp], _i32),
    "medusa_decoder_workspace_size": ([_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "medusa_decoder_verify": ([_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, _i32, _f32, _f32, _vp, _vp, _vp, _sz, _vp], _i32),
    "medusa_prefill_workspace_size": ([_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "medusa_prefill": ([_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32,
                        _i32, _i32, _i32, _f32, _f32, _vp, _vp, _i32, _vp, _sz, _vp], _i32),
    "medusa_gemm_skinny_workspace_size": ([_i32, _i32, _i32], _sz),
    "medusa_gemm_skinny": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp], _i32),
    "medusa_rmsnorm": ([_vp, _i32, _i32, _f32, _vp, _vp], _i32),
    "medusa_rope_workspace_size": ([_i32, _i32], _sz),
    "medusa_rope": ([_vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "medusa_swiglu": ([_vp, _i32, _i32, _vp, _vp], _i32),
    "medusa_embed": ([_vp, _vp, _i32, _i32, _i32, _vp, _vp], _i32),
    "medusa_stream_read": ([_vp, _sz, _vp, _i32, _vp], _i32),
    "medusa_read_mix": ([_vp, _sz, _vp, _sz, _i32, _i32, _i32, _vp, _i32, _vp], _i32),
    "medusa_mfma_rate": ([_i32, _i32, _vp, _i32, _vp], _i32),
    "medusa_profiler_enable": ([_i32], _i32),
    "medusa_profiler_reset": ([], _i32),
    "medusa_profiler_collect": ([], _i32),
    "medusa_profiler_stat": ([_i32, ctypes.c_char_p, _sz, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)],
                             _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class MedusaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {_lib.medusa_last_error().decode()}")


def _check(fn, st):
    if st != OK:
        raise MedusaError(fn, st)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ws(nbytes: int, device, ws):
    if ws is None:
        ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert ws.numel() * ws.element_size() >= nbytes, "workspace too small"
    return ws


def version() -> str:
    return _lib.medusa_version().decode()


# ---------------------------------------------------------------------------
# a1 / a2
# ---------------------------------------------------------------------------

def medusa_resid_silu(h, w1, b1, z, stream=None):
    """w1: [K][H][H] (row-major) or the result of pack_heads (packed, MFMA)."""
    K, H, _ = w1.shape
    B = h.shape[0]
    layout, dt = _w_args(w1)
    _check("medusa_resid_silu", _lib.medusa_resid_silu(_p(h), _p(w1), layout, _p(b1), B, H, K, dt, _p(z),
                                                       _stream(stream)))
    return z


def vocab_topk_workspace_size(B, H, V, K, topk, dt, layout=ROW_MAJOR):
    return _lib.medusa_vocab_topk_workspace_size(B, H, V, K, topk, dt, layout)


def _w_args(w):
    """(layout, dtype) of a head weight: a [K][rows][H] tensor or the packed
    heads of pack_heads."""
    if isinstance(w, Packed):
        return PACKED, BF16
    return ROW_MAJOR, _dt(w)


def medusa_vocab_topk(z, w2, topk, topk_idx, topk_val, logits=None, ws=None, stream=None):
    """w2: [K][V][H] (row-major) or the result of pack_heads (packed, MFMA)."""
    K, V, H = w2.shape
    B = z.shape[0]
    layout, dt = _w_args(w2)
    need = vocab_topk_workspace_size(B, H, V, K, topk, dt, layout)
    ws = _ws(need, z.device, ws)
    _check("medusa_vocab_topk", _lib.medusa_vocab_topk(_p(z), _p(w2), layout, B, H, V, K, topk, dt, _p(logits),
                                                       _p(topk_idx), _p(topk_val), _p(ws),
                                                       ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_val


def heads_workspace_size(B, H, V, K, topk, dt, layout=ROW_MAJOR):
    return _lib.medusa_heads_workspace_size(B, H, V, K, topk, dt, layout)


def medusa_heads_forward(h, w1, b1, w2, topk, topk_idx, topk_val, logits=None, ws=None, stream=None):
    """w1, w2: [K][H][H], [K][V][H] (row-major), or both the results of
    pack_heads (packed, MFMA; w1 may be None either way)."""
    K, V, H = w2.shape
    B = h.shape[0]
    if w1 is not None:
        assert isinstance(w1, Packed) == isinstance(w2, Packed), "w1 and w2 must share one layout"
    layout, dt = _w_args(w2)
    need = heads_workspace_size(B, H, V, K, topk, dt, layout)
    ws = _ws(need, h.device, ws)
    _check("medusa_heads_forward", _lib.medusa_heads_forward(
        _p(h), _p(w1), _p(b1), _p(w2), layout, B, H, V, K, topk, dt, _p(logits), _p(topk_idx), _p(topk_val),
        _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_val


STATIC_SCRATCH_BYTES = 8 << 20


def medusa_heads_forward_static(h, w1, b1, w2, topk, topk_idx, topk_val, logits=None, stream=None):
    """medusa_heads_forward without a workspace: the library's static device
    scratch array holds z and the top-k partials (nothing is allocated)."""
    K, V, H = w2.shape
    B = h.shape[0]
    if w1 is not None:
        assert isinstance(w1, Packed) == isinstance(w2, Packed), "w1 and w2 must share one layout"
    layout, dt = _w_args(w2)
    _check("medusa_heads_forward_static", _lib.medusa_heads_forward_static(
        _p(h), _p(w1), _p(b1), _p(w2), layout, B, H, V, K, topk, dt, _p(logits), _p(topk_idx), _p(topk_val),
        _stream(stream)))
    return topk_idx, topk_val


# ---------------------------------------------------------------------------
# a3
# ---------------------------------------------------------------------------

class Tree:
    """Owner of a medusa_tree handle (topology uploaded to the current device)."""

    def __init__(self, parent, rank, K: int, topk: int):
        import numpy as np
        self._parent = np.ascontiguousarray(parent, dtype=np.int32)
        self._rank = np.ascontiguousarray(rank, dtype=np.int32)
        h = ctypes.c_void_p()
        _check("medusa_tree_create", _lib.medusa_tree_create(
            self._parent.ctypes.data, self._rank.ctypes.data, len(self._parent), K, topk, ctypes.byref(h)))
        self.handle = h
        self.N = _lib.medusa_tree_num_nodes(h)
        self.max_depth = _lib.medusa_tree_max_depth(h)
        self.W = (self.N + 63) // 64

    def status(self, clear: bool = True, stream=None) -> int:
        """The tree's device status word (STATUS_* bits set by kernels that
        met an invalid cache length); waits for `stream` and, by default,
        resets the word."""
        v = ctypes.c_int32()
        _check("medusa_tree_status", _lib.medusa_tree_status(self.handle, ctypes.byref(v), 1 if clear else 0,
                                                             _stream(stream)))
        return v.value

    def mask_host(self):
        import numpy as np
        m = np.zeros((self.N, self.W), dtype=np.uint64)
        _check("medusa_tree_mask_host", _lib.medusa_tree_mask_host(self.handle, m.ctypes.data, m.size))
        return m

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:  # _lib is gone at interpreter shutdown
            self.handle = None
            # medusa_tree_destroy frees device memory, which would invalidate a
            # HIP graph being captured on this thread (a collection can run a
            # finalizer at any allocation): free it after the capture instead
            if torch.cuda.is_available() and torch.cuda.is_current_stream_capturing():
                _deferred_trees.append(h)
                return
            _lib.medusa_tree_destroy(h)
            while _deferred_trees:
                _lib.medusa_tree_destroy(_deferred_trees.pop())


_deferred_trees = []  # tree handles released during a graph capture, freed at the next release outside one


def medusa_heads_forward_tree(h, w1, b1, w2, topk, topk_idx, topk_val, tree: Tree, root_tok, cache_len, node_tok,
                              node_pos, anc_mask=None, logits=None, ws=None, stream=None):
    """medusa_heads_forward and medusa_build_tree in one call (the tree built by
    the top-k merge's workgroups); arguments as those two."""
    K, V, H = w2.shape
    B = h.shape[0]
    if w1 is not None:
        assert isinstance(w1, Packed) == isinstance(w2, Packed), "w1 and w2 must share one layout"
    layout, dt = _w_args(w2)
    need = heads_workspace_size(B, H, V, K, topk, dt, layout)
    ws = _ws(need, h.device, ws)
    _check("medusa_heads_forward_tree", _lib.medusa_heads_forward_tree(
        _p(h), _p(w1), _p(b1), _p(w2), layout, B, H, V, K, topk, dt, _p(logits), _p(topk_idx), _p(topk_val),
        tree.handle, _p(root_tok), _p(cache_len), _p(node_tok), _p(node_pos), _p(anc_mask), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return node_tok, node_pos


def medusa_build_tree(tree: Tree, topk_idx, root_tok, cache_len, node_tok, node_pos, anc_mask=None, stream=None):
    B, K, topk = topk_idx.shape
    _check("medusa_build_tree", _lib.medusa_build_tree(
        tree.handle, _p(topk_idx), _p(root_tok), _p(cache_len), B, K, topk, _p(node_tok), _p(node_pos),
        _p(anc_mask), _stream(stream)))
    return node_tok, node_pos


# ---------------------------------------------------------------------------
# a4
# ---------------------------------------------------------------------------

def tree_attention_workspace_size(tree: Tree, B, nH, D, max_cache_len, dt):
    return _lib.tree_attention_workspace_size(tree.handle, B, nH, D, max_cache_len, dt)


def tree_attention_verify(q, k_tree, v_tree, k_cache, v_cache, cache_len, max_cache_len: int, tree: Tree, out,
                          scale=None, ws=None, stream=None):
    B, N, nH, D = q.shape
    nKV = k_tree.shape[2]
    Lmax = k_cache.shape[2]
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    need = tree_attention_workspace_size(tree, B, nH, D, max_cache_len, dt)
    ws = _ws(need, q.device, ws)
    _check("tree_attention_verify", _lib.tree_attention_verify(
        _p(q), _p(k_tree), _p(v_tree), _p(k_cache), _p(v_cache), _p(cache_len), int(max_cache_len), tree.handle,
        B, nH, nKV, D, Lmax, float(scale), dt, _p(out), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# weight packing (the MFMA products' layout)
# ---------------------------------------------------------------------------

class Packed:
    """A bf16 matrix [rows][cols] in the packed fragment order of
    medusa_pack_rows; `data` is the device buffer (bf16, padded rows).  With
    heads = K, K such matrices back to back (shape (K, rows, cols))."""

    def __init__(self, data, rows: int, cols: int, heads: int = 0):
        self.data, self.rows, self.cols, self.heads = data, rows, cols, heads

    @property
    def shape(self):
        return (self.heads, self.rows, self.cols) if self.heads else (self.rows, self.cols)

    def data_ptr(self):
        return self.data.data_ptr()


def packed_size(rows: int, cols: int) -> int:
    return _lib.medusa_packed_size(rows, cols)


def medusa_pack_rows(src, dst: Packed, dst_row0: int = 0, interleave: int = 1, stream=None):
    rows, cols = src.shape
    _check("medusa_pack_rows", _lib.medusa_pack_rows(_p(src), rows, cols, _p(dst.data), int(dst_row0), dst.rows,
                                                     int(interleave), _stream(stream)))
    return dst


def pack(*mats, interleave: bool = False, stream=None) -> Packed:
    """Pack bf16 [rows_i][cols] matrices into one packed matrix: stacked in the
    given order, or (interleave) alternating in blocks of 16 rows (equal row
    counts, multiples of 16)."""
    cols = mats[0].shape[1]
    rows = sum(m.shape[0] for m in mats)
    nbytes = packed_size(rows, cols)
    if nbytes == 0:
        raise MedusaError("medusa_packed_size", EUNSUPPORTED)
    dst = Packed(torch.empty(nbytes // 2, dtype=torch.bfloat16, device=mats[0].device), rows, cols)
    r0 = 0
    for i, m in enumerate(mats):
        assert m.shape[1] == cols and m.dtype == torch.bfloat16 and m.is_contiguous()
        if interleave:
            medusa_pack_rows(m, dst, 16 * i, len(mats), stream)
        else:
            medusa_pack_rows(m, dst, r0, 1, stream)
            r0 += m.shape[0]
    return dst


def pack_heads(w2, stream=None) -> Packed:
    """Pack per-head matrices [K][rows][H] (bf16; the heads' W2 [K][V][H] or
    W1 [K][H][H]) for medusa_vocab_topk / medusa_resid_silu /
    medusa_heads_forward: head k's packed matrix at byte offset
    k * medusa_packed_size(rows, H)."""
    K, V, H = w2.shape
    assert w2.dtype == torch.bfloat16 and w2.is_contiguous()
    one = packed_size(V, H)
    if one == 0:
        raise MedusaError("medusa_packed_size", EUNSUPPORTED)
    data = torch.empty(K * one // 2, dtype=torch.bfloat16, device=w2.device)
    for k in range(K):
        dst = Packed(data[k * one // 2:(k + 1) * one // 2], V, H)
        medusa_pack_rows(w2[k], dst, 0, 1, stream)
    return Packed(data, V, H, heads=K)


# ---------------------------------------------------------------------------
# a5
# ---------------------------------------------------------------------------

def base_greedy_workspace_size(R, H, V, dt, layout=ROW_MAJOR):
    return _lib.medusa_base_greedy_workspace_size(R, H, V, dt, layout)


def medusa_base_greedy(x, lm_head, greedy, eps=1e-6, logits=None, ws=None, stream=None):
    """lm_head: a row-major [V][H] tensor (vector GEMV) or a Packed bf16
    matrix (MFMA product)."""
    layout = PACKED if isinstance(lm_head, Packed) else ROW_MAJOR
    V, H = lm_head.shape
    R = x.numel() // H
    dt = BF16 if layout == PACKED else _dt(lm_head)
    need = base_greedy_workspace_size(R, H, V, dt, layout)
    ws = _ws(need, x.device, ws)
    _check("medusa_base_greedy", _lib.medusa_base_greedy(
        _p(x), ctypes.c_void_p(lm_head.data_ptr()), layout, R, H, V, float(eps), dt, _p(greedy), _p(logits), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return greedy


# ---------------------------------------------------------------------------
# a6 + a7
# ---------------------------------------------------------------------------

def medusa_accept(tree: Tree, node_tok, greedy, accept_len, accept_nodes, out_tokens, cache_len, new_cache_len,
                  k_cache=None, v_cache=None, stream=None):
    """k_cache / v_cache: None, or [layers][B][nKV][Lmax][D] / [B][nKV][Lmax][D] tensors."""
    B = node_tok.shape[0]
    n_layers, nKV, D, Lmax, stride, dt = 0, 0, 0, 0, 0, F32
    if k_cache is not None:
        kc = k_cache if k_cache.dim() == 5 else k_cache.unsqueeze(0)
        n_layers, _, nKV, Lmax, D = kc.shape
        stride = kc.stride(0)
        dt = _dt(kc)
    _check("medusa_accept", _lib.medusa_accept(
        tree.handle, _p(node_tok), _p(greedy), B, _p(accept_len), _p(accept_nodes), _p(out_tokens), _p(cache_len),
        _p(new_cache_len), _p(k_cache), _p(v_cache), n_layers, stride, nKV, D, Lmax, dt, _stream(stream)))
    return accept_len


def medusa_typical_accept(tree: Tree, node_tok, logits, uniform, accept_len, accept_nodes, out_tokens, cache_len,
                          new_cache_len, temperature=0.7, epsilon=0.09, delta=0.3, k_cache=None, v_cache=None, ws=None,
                          stream=None):
    """Typical acceptance (sampling mode).  logits [B][N][V] float32 (the base
    model's scores after every node); uniform [B] float32 in [0, 1).
    k_cache / v_cache as medusa_accept."""
    B, N, V = logits.shape
    n_layers, nKV, D, Lmax, stride, dt = 0, 0, 0, 0, 0, F32
    if k_cache is not None:
        kc = k_cache if k_cache.dim() == 5 else k_cache.unsqueeze(0)
        n_layers, _, nKV, Lmax, D = kc.shape
        stride = kc.stride(0)
        dt = _dt(kc)
    need = _lib.medusa_typical_accept_workspace_size(tree.handle, B)
    ws = _ws(need, logits.device, ws)
    _check("medusa_typical_accept", _lib.medusa_typical_accept(
        tree.handle, _p(node_tok), _p(logits), B, V, float(temperature), float(epsilon), float(delta), _p(uniform),
        _p(accept_len), _p(accept_nodes), _p(out_tokens), _p(cache_len), _p(new_cache_len), _p(k_cache), _p(v_cache),
        n_layers, stride, nKV, D, Lmax, dt, _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return accept_len


def medusa_speculative_sample(p, q, drafts, u_accept, u_resample, n_accepted, out_tokens, stream=None):
    """p [B][gamma+1][V], q [B][gamma][V] float32; drafts [B][gamma] int32;
    u_accept [B][gamma], u_resample [B][gamma+1] float32."""
    B, g1, V = p.shape
    _check("medusa_speculative_sample", _lib.medusa_speculative_sample(
        _p(p), _p(q), _p(drafts), _p(u_accept), _p(u_resample), B, g1 - 1, V, _p(n_accepted), _p(out_tokens),
        _stream(stream)))
    return n_accepted


def medusa_advance(tree: Tree, accept_len, accept_nodes, out_tokens, hidden, root_tok, h, tokens=None,
                   n_tokens=None, new_cache_len=None, cache_len=None, stream=None):
    """Hand the accepted branch to the next round: root_tok <- the bonus token,
    h <- hidden at the deepest accepted node (in h's dtype), optionally append
    the round's tokens to tokens [B][cap] at n_tokens and copy new_cache_len
    into cache_len."""
    B, H = h.shape
    cap = tokens.shape[1] if tokens is not None else 0
    _check("medusa_advance", _lib.medusa_advance(
        tree.handle, _p(accept_len), _p(accept_nodes), _p(out_tokens), _p(hidden), B, H, _dt(h), _p(root_tok),
        _p(h), _p(tokens), _p(n_tokens), cap, _p(new_cache_len), _p(cache_len), _stream(stream)))
    return root_tok


def medusa_plant_greedy(tree: Tree, topk_idx, cache_len, greedy, V: int, alpha=0.8, seed: int = 0,
                        stream=None):
    """Measurement aid: overwrite greedy [B][N] with a continuation drawn
    from the rank prior a (1 - a)^r (see include/medusa.h); alpha: one value
    or one per depth."""
    B, K, topk = topk_idx.shape
    a = (ctypes.c_float * 16)(*([float(x) for x in alpha] if hasattr(alpha, "__len__") else [float(alpha)]))
    n = len(alpha) if hasattr(alpha, "__len__") else 1
    _check("medusa_plant_greedy", _lib.medusa_plant_greedy(
        tree.handle, _p(topk_idx), _p(cache_len), B, K, topk, int(V), ctypes.cast(a, ctypes.c_void_p), n,
        ctypes.c_uint64(seed), _p(greedy), _stream(stream)))
    return greedy


def medusa_accept_stats(tree: Tree, accept_len, accept_nodes, out_tokens, topk_idx, counts, stream=None):
    """Add one round's acceptance observations to counts [K][topk + 1] (int32)."""
    B, K, topk = topk_idx.shape
    _check("medusa_accept_stats", _lib.medusa_accept_stats(
        tree.handle, _p(accept_len), _p(accept_nodes), _p(out_tokens), _p(topk_idx), B, K, topk, _p(counts),
        _stream(stream)))
    return counts


def tree_select(acc, N: int):
    """(parent, rank) of the N-node tree chosen best-first under acc
    [K][topk] (per-depth probability that each rank's guess is right)."""
    import numpy as np
    a = np.ascontiguousarray(acc, dtype=np.float64)
    K, topk = a.shape
    parent = np.empty(N, dtype=np.int32)
    rank = np.empty(N, dtype=np.int32)
    _check("medusa_tree_select", _lib.medusa_tree_select(a.ctypes.data, K, topk, N, parent.ctypes.data,
                                                         rank.ctypes.data))
    return parent, rank


# ---------------------------------------------------------------------------
# a8
# ---------------------------------------------------------------------------

LAYER_MATRICES = ("wqkv", "wo", "w_gate_up", "w_down")


class LayerWeights(ctypes.Structure):
    """medusa_layer_weights: device pointers of one decoder layer's packed matrices."""
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_MATRICES]


def pack_layer(W, stream=None):
    """Row-major bf16 layer weights {wq, wk, wv, wo, w_gate, w_up, w_down}
    -> the packed matrices medusa_decoder_verify reads."""
    return {"wqkv": pack(W["wq"], W["wk"], W["wv"], stream=stream), "wo": pack(W["wo"], stream=stream),
            "w_gate_up": pack(W["w_gate"], W["w_up"], interleave=True, stream=stream),
            "w_down": pack(W["w_down"], stream=stream)}


def decoder_workspace_size(tree: Tree, B, H, nH, nKV, D, F, V, max_cache_len):
    return _lib.medusa_decoder_workspace_size(tree.handle, B, H, nH, nKV, D, F, V, max_cache_len)


def medusa_decoder_verify(layers, embedding, lm_head: Packed, tree: Tree, node_tok, node_pos, cache_len,
                          max_cache_len: int, k_cache, v_cache, nH: int, greedy, hidden=None, rms_eps=1e-6,
                          rope_base=10000.0, ws=None, stream=None):
    """layers: list of pack_layer() dicts; embedding [V][H] bf16 row-major;
    lm_head Packed [V][H]; k_cache / v_cache: [layers][B][nKV][Lmax][D] bf16."""
    n_layers, B, nKV, Lmax, D = k_cache.shape
    V, H = embedding.shape
    F = layers[0]["w_gate_up"].rows // 2
    arr = (LayerWeights * len(layers))()
    for i, W in enumerate(layers):
        arr[i] = LayerWeights(*[W[n].data_ptr() for n in LAYER_MATRICES])
    need = decoder_workspace_size(tree, B, H, nH, nKV, D, F, V, max_cache_len)
    ws = _ws(need, embedding.device, ws)
    _check("medusa_decoder_verify", _lib.medusa_decoder_verify(
        ctypes.cast(arr, ctypes.c_void_p), len(layers), _p(embedding), ctypes.c_void_p(lm_head.data_ptr()),
        tree.handle, _p(node_tok), _p(node_pos), _p(cache_len), int(max_cache_len), _p(k_cache), _p(v_cache),
        k_cache.stride(0), B, H, nH, nKV, D, F, V, Lmax, float(rms_eps), float(rope_base), _p(greedy), _p(hidden),
        _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return greedy


def chain_tree(C: int) -> Tree:
    """A chain of C nodes (each node's parent is the previous one): the tree
    medusa_prefill runs its passes on."""
    import numpy as np
    return Tree(np.arange(-1, C - 1, dtype=np.int32), np.zeros(C, dtype=np.int32), max(C - 1, 1), 1)


def medusa_prefill(layers, embedding, lm_head: Packed, chain: Tree, tokens, cache_len, max_cache_len: int, k_cache,
                   v_cache, nH: int, next_tok, hidden, rms_eps=1e-6, rope_base=10000.0, ws=None, stream=None):
    """Prefill the prompt tokens [B][T] (int32) in passes of chain.N tokens:
    their keys/values go to the caches at cache_len.., cache_len grows by T,
    next_tok [B] gets the greedy choice after the prompt and hidden [B][H]
    (float32 or bf16) its final normalised row."""
    n_layers, B, nKV, Lmax, D = k_cache.shape
    V, H = embedding.shape
    T = tokens.shape[1]
    F = layers[0]["w_gate_up"].rows // 2
    arr = (LayerWeights * len(layers))()
    for i, W in enumerate(layers):
        arr[i] = LayerWeights(*[W[n].data_ptr() for n in LAYER_MATRICES])
    need = _lib.medusa_prefill_workspace_size(chain.handle, B, H, nH, nKV, D, F, V, T, int(max_cache_len))
    ws = _ws(need, embedding.device, ws)
    _check("medusa_prefill", _lib.medusa_prefill(
        ctypes.cast(arr, ctypes.c_void_p), len(layers), _p(embedding), ctypes.c_void_p(lm_head.data_ptr()),
        chain.handle, _p(tokens), T, _p(cache_len), int(max_cache_len), _p(k_cache), _p(v_cache), k_cache.stride(0),
        B, H, nH, nKV, D, F, V, Lmax, float(rms_eps), float(rope_base), _p(next_tok), _p(hidden), _dt(hidden), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return next_tok


# ---------------------------------------------------------------------------
# kernel timing
# ---------------------------------------------------------------------------

def medusa_gemm_skinny(n, w: Packed, out, ws=None, stream=None):
    """out [R][ncols] float32 = n [R][K] (bf16) times the packed W [ncols][K]^T."""
    R, K = n.shape
    need = _lib.medusa_gemm_skinny_workspace_size(R, K, w.rows)
    ws = _ws(need, n.device, ws) if need else ws
    _check("medusa_gemm_skinny", _lib.medusa_gemm_skinny(
        _p(n), ctypes.c_void_p(w.data_ptr()), R, K, w.rows, _p(out), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return out


def medusa_rmsnorm(x, n, eps: float = 1e-6, stream=None):
    """n [R][H] bf16 = RMSNorm(x [R][H] float32), unit weight."""
    R, H = x.shape
    _check("medusa_rmsnorm", _lib.medusa_rmsnorm(_p(x), R, H, float(eps), _p(n), _stream(stream)))
    return n


def medusa_rope(qkv, pos, nH: int, nKV: int, D: int, q, k, v, rope_base: float = 10000.0, ws=None, stream=None):
    """qkv [R][(nH + 2 nKV) D] float32, pos [R] int32 -> q [R][nH][D], k, v
    [R][nKV][D] bf16 (q and k rotated)."""
    R = qkv.shape[0]
    ws = _ws(_lib.medusa_rope_workspace_size(R, D), qkv.device, ws)
    _check("medusa_rope", _lib.medusa_rope(_p(qkv), _p(pos), R, nH, nKV, D, float(rope_base), _p(q), _p(k), _p(v),
                                           _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return q, k, v


def medusa_swiglu(gate_up, a, stream=None):
    """a [R][F] bf16 = SiLU(gate) * up from gate_up [R][2F] float32 (gate and
    up columns alternating in blocks of 16)."""
    R, F2 = gate_up.shape
    _check("medusa_swiglu", _lib.medusa_swiglu(_p(gate_up), R, F2 // 2, _p(a), _stream(stream)))
    return a


def medusa_embed(tok, embedding, x, stream=None):
    """x [R][H] float32 = embedding [V][H] (bf16) rows tok [R] (ids outside
    [0, V) read row 0)."""
    V, H = embedding.shape
    _check("medusa_embed", _lib.medusa_embed(_p(tok), _p(embedding), tok.numel(), H, V, _p(x), _stream(stream)))
    return x


def medusa_stream_read(src, sink, n_wg: int = 16384, stream=None):
    """Measurement aid: read src (a device tensor) once as the weight streams
    read (see include/medusa.h); sink: [n_wg] int32 device tensor."""
    nbytes = src.numel() * src.element_size()
    _check("medusa_stream_read", _lib.medusa_stream_read(_p(src), nbytes, _p(sink), int(n_wg), _stream(stream)))
    return sink


def medusa_read_mix(window, src, window_parts: int, stream_parts: int, rounds: int, sink, n_wg: int = 256,
                    stream=None):
    """Measurement aid: per-CU read rate from a shared L2-resident window and
    private HBM slices (see include/medusa.h).  window / src: device tensors
    (or None where their part is 0); sink: [n_wg] int32 device tensor."""
    wb = 0 if window is None else window.numel() * window.element_size()
    sb = 0 if src is None else src.numel() * src.element_size()
    _check("medusa_read_mix", _lib.medusa_read_mix(_p(window), wb, _p(src), sb, int(window_parts), int(stream_parts),
                                                   int(rounds), _p(sink), int(n_wg), _stream(stream)))
    return sink


def medusa_mfma_rate(random_operands: bool, iters: int, out, n_wg: int = 256, stream=None):
    """Measurement aid: the wide lm_head's matrix loop alone (see
    include/medusa.h); out: [n_wg * 256] float32 device tensor."""
    _check("medusa_mfma_rate", _lib.medusa_mfma_rate(int(bool(random_operands)), int(iters), _p(out), int(n_wg),
                                                     _stream(stream)))
    return out


def profiler_enable(on: bool = True):
    _lib.medusa_profiler_enable(1 if on else 0)


def profiler_reset():
    _lib.medusa_profiler_reset()


def profiler_collect() -> dict:
    """{kernel name: (launches, total milliseconds)} since the last reset."""
    n = _lib.medusa_profiler_collect()
    if n < 0:
        raise MedusaError("medusa_profiler_collect", EHIP)
    out = {}
    for i in range(n):
        name = ctypes.create_string_buffer(128)
        calls = ctypes.c_int64()
        ms = ctypes.c_double()
        _check("medusa_profiler_stat", _lib.medusa_profiler_stat(i, name, 128, ctypes.byref(calls), ctypes.byref(ms)))
        out[name.value.decode()] = (calls.value, ms.value)
    return out


from .generate import MedusaLoop  # noqa: E402  (the loop helper builds on the calls above)
