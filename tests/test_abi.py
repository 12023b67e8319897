"""The C-ABI library loads on a machine without a GPU, exports every function
include/medusa.h declares, and rejects bad arguments on the host before any
GPU work (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "medusa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


@pytest.fixture(scope="module")
def M():
    import speculative_decoding_medusa_amd as M
    return M


def test_header_declares_the_step_calls():
    names = _declared()
    for n in ["medusa_heads_forward", "medusa_build_tree", "tree_attention_verify", "medusa_accept",
              "medusa_resid_silu", "medusa_vocab_topk", "medusa_base_greedy", "medusa_tree_create"]:
        assert n in names


def test_library_exports_every_declared_symbol(M):
    for n in _declared():
        assert hasattr(M._lib, n), f"libmedusa.so does not export {n}"


def test_binding_names_match_the_abi(M):
    for n in ["medusa_resid_silu", "medusa_vocab_topk", "medusa_heads_forward", "medusa_build_tree",
              "tree_attention_verify", "medusa_base_greedy", "medusa_accept", "medusa_pack_rows",
              "medusa_decoder_verify", "medusa_advance", "medusa_typical_accept", "medusa_speculative_sample",
              "medusa_gemm_skinny", "medusa_rmsnorm", "medusa_rope", "medusa_swiglu", "medusa_embed"]:
        assert callable(getattr(M, n))


def _tree(M, parent, rank, N=None, K=5, topk=4):
    p = np.asarray(parent, dtype=np.int32)
    r = np.asarray(rank, dtype=np.int32)
    h = ctypes.c_void_p()
    st = M._lib.medusa_tree_create(p.ctypes.data, r.ctypes.data, len(p) if N is None else N, K, topk,
                                   ctypes.byref(h))
    return st, M._lib.medusa_last_error().decode()


@pytest.mark.parametrize("parent,rank,kw,err", [
    ([0, 0], [0, 0], {}, "parent[0]"),
    ([-1, 1], [0, 0], {}, "parent"),
    ([-1, 0, 0], [0, 1, 1], {}, "repeats rank"),
    ([-1, 0], [0, 4], {}, "rank"),
    ([-1, 0, 1, 2], [0, 0, 0, 0], {"K": 2}, "depth"),
    ([-1], [0], {"N": 0}, "N must be"),
])
def test_tree_spec_errors(M, parent, rank, kw, err):
    st, msg = _tree(M, parent, rank, **kw)
    assert st == M.EINVAL and err in msg


def test_tree_too_large_is_unsupported(M):
    parent = [-1] + [0] * 300
    st, msg = _tree(M, parent, list(range(301)), topk=16)
    assert st in (M.EUNSUPPORTED, M.EINVAL)


def test_heads_argument_errors(M):
    L = M._lib
    st = L.medusa_heads_forward(None, None, None, None, M.ROW_MAJOR, 1, 4096, 32000, 5, 4, M.BF16, None, None, None, None, 0, None)
    assert st == M.EINVAL and "null" in L.medusa_last_error().decode()
    d = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    st = L.medusa_vocab_topk(d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 0, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EINVAL and "topk" in L.medusa_last_error().decode()
    st = L.medusa_vocab_topk(d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 17, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED
    st = L.medusa_vocab_topk(d, d, M.ROW_MAJOR, 9, 4096, 32000, 5, 4, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED
    st = L.medusa_vocab_topk(d, d, M.ROW_MAJOR, 1, 4100, 32000, 5, 4, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED
    st = L.medusa_vocab_topk(d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 4, M.BF16, None, d, d, d, 10, None)
    assert st == M.EINVAL and "workspace" in L.medusa_last_error().decode()
    st = L.medusa_heads_forward(d, d, None, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 4, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EINVAL and "both" in L.medusa_last_error().decode()
    # the heads with the tree build: the tree and its outputs are required,
    # and the heads' checks come first
    st = L.medusa_heads_forward_tree(d, d, d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 4, M.BF16, None, d, d, None, d, d,
                                     d, d, None, d, 1 << 30, None)
    assert st == M.EINVAL and "null" in L.medusa_last_error().decode()
    st = L.medusa_heads_forward_tree(d, d, d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 4, M.BF16, None, d, d, d, d, d,
                                     None, d, None, d, 1 << 30, None)
    assert st == M.EINVAL and "null" in L.medusa_last_error().decode()
    st = L.medusa_heads_forward_tree(d, d, d, d, M.ROW_MAJOR, 1, 4096, 32000, 5, 17, M.BF16, None, d, d, d, d, d,
                                     d, d, None, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED
    st = L.medusa_resid_silu(d, d, M.ROW_MAJOR, d, 1, 4096, 5, 7, d, None)
    assert st == M.EINVAL
    st = L.medusa_resid_silu(d, d, M.PACKED, d, 8, 4104, 5, M.BF16, d, None)
    assert st == M.EUNSUPPORTED and "multiple" in L.medusa_last_error().decode()
    st = L.medusa_resid_silu(d, d, M.PACKED, d, 8, 4096, 5, M.F32, d, None)
    assert st == M.EUNSUPPORTED and "bf16" in L.medusa_last_error().decode()
    # packed w2: bf16 only, H a multiple of 128, a known layout
    st = L.medusa_vocab_topk(d, d, M.PACKED, 8, 256, 1000, 5, 4, M.F32, None, d, d, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED and "bf16" in L.medusa_last_error().decode()
    st = L.medusa_vocab_topk(d, d, M.PACKED, 8, 4104, 1000, 5, 4, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EUNSUPPORTED and "multiple" in L.medusa_last_error().decode()
    st = L.medusa_vocab_topk(d, d, 7, 8, 4096, 1000, 5, 4, M.BF16, None, d, d, d, 1 << 30, None)
    assert st == M.EINVAL and "layout" in L.medusa_last_error().decode()


def test_sampling_and_handoff_argument_errors(M):
    """The sampling-mode and hand-off calls reject bad arguments on the host."""
    L = M._lib
    d = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    ss = L.medusa_speculative_sample
    assert ss(None, d, d, d, d, 1, 4, 100, d, d, None) == M.EINVAL                  # no target rows
    assert ss(d, None, d, d, d, 1, 4, 100, d, d, None) == M.EINVAL                  # drafts without q
    assert "draft" in L.medusa_last_error().decode()
    assert ss(d, d, d, d, d, 0, 4, 100, d, d, None) == M.EINVAL                     # B = 0
    assert ss(d, d, d, d, d, 1, -1, 100, d, d, None) == M.EINVAL                    # gamma < 0
    assert ss(d, d, d, d, d, 1, 65, 100, d, d, None) == M.EUNSUPPORTED              # gamma > 64
    assert ss(d, d, d, d, d, 1, 4, 262145, d, d, None) == M.EUNSUPPORTED            # V over the draw's limit
    ta = L.medusa_typical_accept
    assert ta(None, d, d, 1, 100, 0.7, 0.09, 0.3, d, d, d, d, d, d, None, None, 0, 0, 0, 0, 0, M.BF16, d, 1 << 20,
              None) == M.EINVAL and "null" in L.medusa_last_error().decode()
    assert L.medusa_typical_accept_workspace_size(None, 1) == 0
    adv = L.medusa_advance
    assert adv(None, d, d, d, d, 1, 4096, M.BF16, d, d, None, None, 0, None, None, None) == M.EINVAL


def test_layer_block_argument_errors(M):
    """The decoder layer's building blocks reject bad shapes and misaligned
    pointers on the host."""
    L = M._lib
    d = ctypes.c_void_p(256)   # aligned; never dereferenced: validation fails first
    m = ctypes.c_void_p(264)   # 8-byte but not 16-byte aligned
    assert L.medusa_gemm_skinny(None, d, 64, 4096, 4096, d, d, 1 << 30, None) == M.EINVAL
    assert L.medusa_gemm_skinny(d, d, 64, 100, 4096, d, d, 1 << 30, None) == M.EUNSUPPORTED     # K % 64
    assert L.medusa_gemm_skinny(d, d, 300, 4096, 4096, d, d, 1 << 30, None) == M.EUNSUPPORTED   # R > 256
    assert L.medusa_gemm_skinny(m, d, 64, 4096, 4096, d, d, 1 << 30, None) == M.EINVAL          # alignment
    assert L.medusa_gemm_skinny(d, d, 64, 4096, 4096, d, d, 16, None) == M.EINVAL               # workspace
    assert "workspace" in L.medusa_last_error().decode()
    assert L.medusa_gemm_skinny_workspace_size(64, 100, 4096) == 0
    assert L.medusa_rmsnorm(d, 4, 6, 1e-6, d, None) == M.EUNSUPPORTED                           # H % 4
    assert L.medusa_rmsnorm(d, 4, 8, -1.0, d, None) == M.EINVAL                                 # eps < 0
    assert L.medusa_rope(d, d, 4, 2, 1, 130, 10000.0, d, d, d, d, 1 << 20, None) == M.EUNSUPPORTED  # D > 128
    assert L.medusa_rope(d, d, 4, 2, 1, 64, 1.0, d, d, d, d, 1 << 20, None) == M.EINVAL             # base
    assert L.medusa_rope(d, d, 4, 2, 1, 64, 10000.0, d, d, d, d, 8, None) == M.EINVAL               # workspace
    assert L.medusa_swiglu(d, 4, 20, d, None) == M.EUNSUPPORTED                                 # F % 16
    assert L.medusa_embed(d, d, 4, 12, 100, d, None) == M.EUNSUPPORTED                          # H % 8
    assert L.medusa_embed(d, m, 4, 16, 100, d, None) == M.EINVAL                                # alignment


def test_workspace_sizes_are_positive(M):
    L = M._lib
    assert L.medusa_heads_workspace_size(1, 4096, 32000, 5, 4, M.BF16, M.ROW_MAJOR) >= 5 * 4096 * 4
    assert L.medusa_vocab_topk_workspace_size(8, 4096, 128256, 5, 4, M.BF16, M.ROW_MAJOR) > 0
    # packed: the bf16 head/remainder rows of every head + the top-k candidates
    # of every 256-row workgroup (501 of them per head)
    assert (L.medusa_vocab_topk_workspace_size(8, 4096, 128256, 5, 4, M.BF16, M.PACKED)
            >= 5 * 16 * 4096 * 2 + 2 * 8 * 5 * 501 * 4 * 4)
    # packed: per-workgroup (value, index) candidates of every row
    assert L.medusa_base_greedy_workspace_size(64, 4096, 32000, M.BF16, M.PACKED) >= 2 * 64 * 250 * 4
    assert L.medusa_base_greedy_workspace_size(9, 256, 1000, M.F32, M.ROW_MAJOR) >= 9 * 256 * 4
    assert L.medusa_heads_workspace_size(0, 4096, 32000, 5, 4, M.BF16, M.ROW_MAJOR) == 0


def test_packed_size(M):
    # rows round up to whole 16-row fragments; cols must be a multiple of 32
    assert M.packed_size(16, 32) == 16 * 32 * 2
    assert M.packed_size(17, 64) == 32 * 64 * 2
    assert M.packed_size(32000, 4096) == 32000 * 4096 * 2
    assert M.packed_size(16, 48) == 0
    assert M.packed_size(0, 64) == 0


def test_pack_rows_argument_errors(M):
    L = M._lib
    d = ctypes.c_void_p(16)
    assert L.medusa_pack_rows(d, 16, 48, d, 0, 16, 1, None) == M.EUNSUPPORTED    # cols % 32
    assert L.medusa_pack_rows(d, 16, 64, d, 8, 16, 1, None) == M.EINVAL          # rows do not fit
    assert L.medusa_pack_rows(None, 16, 64, d, 0, 16, 1, None) == M.EINVAL
    assert L.medusa_pack_rows(d, 24, 64, d, 0, 48, 2, None) == M.EINVAL          # interleave: rows % 16
    assert L.medusa_pack_rows(d, 32, 64, d, 32, 64, 2, None) == M.EINVAL         # interleave: dst_row0 < 32
    assert L.medusa_pack_rows(d, 32, 64, d, 16, 48, 2, None) == M.EINVAL         # interleave: rows do not fit
    assert L.medusa_base_greedy(d, d, M.PACKED, 4, 256, 100, 1e-6, M.F32, d, None, d, 1 << 30, None) == \
        M.EUNSUPPORTED                                                           # packed needs bf16
    assert L.medusa_base_greedy(d, d, M.PACKED, 4, 264, 100, 1e-6, M.BF16, d, None, d, 1 << 30, None) == \
        M.EUNSUPPORTED                                                           # H % 64


def test_profiler_without_launches(M):
    M.profiler_enable(True)
    M.profiler_reset()
    assert M.profiler_collect() == {}
    M.profiler_enable(False)


def test_tree_status_argument_errors(M):
    L = M._lib
    v = ctypes.c_int32(-1)
    assert L.medusa_tree_status(None, ctypes.byref(v), 1, None) == M.EINVAL
    assert "null" in L.medusa_last_error().decode()
    assert v.value == -1            # nothing written on an error


def test_status_bits_match_the_header(M):
    src = open(HEADER).read()
    bits = dict(re.findall(r"#define\s+MEDUSA_(STATUS_\w+)\s+(\d+)", src))
    assert int(bits["STATUS_CACHE_LEN_CLAMPED"]) == M.STATUS_CACHE_LEN_CLAMPED
    assert int(bits["STATUS_CACHE_OVERFLOW"]) == M.STATUS_CACHE_OVERFLOW


class _StubTree:
    def __init__(self, max_depth):
        self.max_depth = max_depth


def _loop_budget(M, max_cache_len, start_len, max_depth):
    loop = M.MedusaLoop.__new__(M.MedusaLoop)     # the host-side budget only; no device buffers
    loop.max_cache_len = max_cache_len
    loop.tree = _StubTree(max_depth)
    loop.restart(start_len)
    return loop


def test_loop_refuses_rounds_past_the_cache(M):
    # a round grows a prefix by at most Dmax + 1 = 6 tokens: from 4000 under a
    # bound of 4096, 16 rounds fit (4096 = 4000 + 16 * 6), the 17th could overrun
    loop = _loop_budget(M, 4096, 4000, 5)
    assert loop.rounds_left == 16
    with pytest.raises(ValueError):
        loop.run(17)
    assert loop.rounds_left == 16        # a refused run reserves nothing
    loop._reserve(10)
    loop._reserve(6)
    with pytest.raises(ValueError):
        loop._reserve(1)
    loop.restart(4096 - 6)
    assert loop.rounds_left == 1
    with pytest.raises(ValueError):
        _loop_budget(M, 4096, 4097, 5)   # a start past the bound
    assert _loop_budget(M, 100, 100, 5).rounds_left == 0


def test_measurement_aid_argument_errors(M):
    L = M._lib
    d = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    st = L.medusa_read_mix(d, 4096, d, 1 << 20, 3, 1, 1, d, 1, None)
    assert st == M.EINVAL and "window_parts" in L.medusa_last_error().decode()
    st = L.medusa_read_mix(d, 4096, d, 4096, 0, 8, 1, d, 1, None)      # needs 8 x 4096 bytes of src
    assert st == M.EINVAL and "src_bytes" in L.medusa_last_error().decode()
    st = L.medusa_read_mix(ctypes.c_void_p(24), 8 * 4096, None, 0, 8, 0, 1, d, 1, None)
    assert st == M.EINVAL and "aligned" in L.medusa_last_error().decode()
    st = L.medusa_read_mix(d, 4096, None, 0, 8, 0, 1, d, 1, None)      # not a whole round of 8 x 4 KB
    assert st == M.EINVAL and "window_bytes" in L.medusa_last_error().decode()
    st = L.medusa_mfma_rate(2, 10, d, 1, None)
    assert st == M.EINVAL and "random_operands" in L.medusa_last_error().decode()
    st = L.medusa_mfma_rate(0, 0, d, 1, None)
    assert st == M.EINVAL and "iters" in L.medusa_last_error().decode()
