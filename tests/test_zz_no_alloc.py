"""medusa_heads_forward_static (no workspace, no allocation) against
medusa_heads_forward on the same inputs: two calls in a row, the second with
smaller sizes, each equal bit for bit to the workspace entry point (the same
kernels), and both within the oracle's bar (top-k ids exact)."""
import sys

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from medusa_testlib import dev, enforce_heads_gap

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _run(M, cfg, layout, static):
    heads = mi.gen_heads(cfg)
    logits_ref, _ = enforce_heads_gap(cfg, heads, [])
    idx_ref, _ = oracle.topk(np.transpose(logits_ref, (2, 0, 1)), cfg.topk)
    h, W1, b1, W2 = (dev(heads[k]) for k in ("h", "W1", "b1", "W2"))
    if layout == "packed":
        W1, W2 = M.pack_heads(W1), M.pack_heads(W2)
    B, K, V, k = cfg.B, cfg.K, cfg.V, cfg.topk
    out = {}
    for name in ("ws", "static"):
        lg = torch.full((B, K, V), float("nan"), device="cuda")
        ti = torch.full((B, K, k), -1, dtype=torch.int32, device="cuda")
        tv = torch.full((B, K, k), float("nan"), device="cuda")
        if name == "ws":
            M.medusa_heads_forward(h, W1, b1, W2, k, ti, tv, logits=lg)
        else:
            static(h, W1, b1, W2, k, ti, tv, logits=lg)
        torch.cuda.synchronize()
        out[name] = (lg, ti, tv)
    for a, b in zip(out["ws"], out["static"]):
        assert torch.equal(a, b)
    assert np.array_equal(out["static"][1].cpu().numpy(), idx_ref)


@pytest.mark.parametrize("layout", ["rows", "packed"])
def test_static_scratch_matches_workspace_call(layout):
    import speculative_decoding_medusa_amd as M
    big = mi.custom_config("ns1", "bf16", 4, 2048, 9001, 5, 4, mi.tiny_tree(), 4, 4, 64, (16,), 801)
    small = mi.custom_config("ns2", "bf16", 1, 512, 1003, 2, 3, mi.tiny_tree(), 4, 4, 64, (16,), 802)
    for cfg in (big, small):
        _say("static scratch", layout, "B", cfg.B, "H", cfg.H, "V", cfg.V, "K", cfg.K)
        _run(M, cfg, layout, M.medusa_heads_forward_static)


def test_static_scratch_rejects_sizes_past_its_limit():
    import speculative_decoding_medusa_amd as M
    B, K, H, V = 8, 64, 4096, 1000       # z alone is 8 MiB
    assert M.heads_workspace_size(B, H, V, K, 4, M.BF16) > M.STATIC_SCRATCH_BYTES
    h = torch.zeros(B, H, dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros(K, V, H, dtype=torch.bfloat16, device="cuda")
    ti = torch.empty(B, K, 4, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, 4, device="cuda")
    with pytest.raises(M.MedusaError) as e:
        M.medusa_heads_forward_static(h, None, None, W2, 4, ti, tv)
    assert e.value.status == M.EUNSUPPORTED and "static array" in str(e.value)
