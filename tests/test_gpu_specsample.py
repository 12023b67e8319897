"""GPU parity of the speculative-sampling rule on a chain of drafts
(medusa_speculative_sample) against the oracle (oracle/specsample.py).

* Random target/draft rows (softmax of seeded scores), drafts drawn from q:
  the accepted counts and every output token exact.  The uniforms keep each
  acceptance test (u q(x) against p(x)) at least 1e-4 relative and each draw
  at least 1e-4 of probability away from a boundary, as the oracle computes
  them; the GPU decides in float32.
* The e-book's toy pair on 4096 sequences whose draft, acceptance and
  resample uniforms sweep grids: the GPU's output frequencies at the first
  position equal p (the rule's exactness, on the GPU's own draws).
"""
import sys

import numpy as np
import pytest
import torch

import medusa_inputs as mi
import oracle
from medusa_testlib import dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _safe_u(r, cdf_row, margin=1e-4):
    c = np.cumsum(cdf_row)
    for _ in range(1000):
        u = float(np.float32(r.random()))
        j = int(np.searchsorted(c, u, side="right"))
        lo = c[j - 1] if j > 0 else 0.0
        if j < len(c) and min(c[j] - u, u - lo) >= margin * c[-1]:
            return u
    raise RuntimeError("no uniform away from the boundaries")


@pytest.mark.parametrize("B,gamma,V,seed", [(4, 4, 1000, 901), (2, 5, 32000, 902), (3, 0, 777, 903), (2, 3, 5, 904)],
                         ids=["b4_g4_v1000", "b2_g5_v32000", "b3_g0_v777", "b2_g3_v5"])
def test_speculative_sample_parity(B, gamma, V, seed):
    import speculative_decoding_medusa_amd as M
    _say("speculative sample", B, gamma, V)
    r = np.random.default_rng(seed)
    lp = mi.normal((B, gamma + 1, V), seed, mi.S_TEST + 51, 1.5, "f32").astype(np.float64)
    lq = lp[:, :gamma] + mi.normal((B, max(gamma, 1), V), seed, mi.S_TEST + 52, 0.7, "f32")[:, :gamma]
    p = _softmax(lp).astype(np.float32)
    q = _softmax(lq).astype(np.float32) if gamma else np.zeros((B, 0, V), dtype=np.float32)
    p64, q64 = p.astype(np.float64), q.astype(np.float64)
    drafts = np.zeros((B, gamma), dtype=np.int32)
    ua = np.zeros((B, gamma), dtype=np.float32)
    ur = np.zeros((B, gamma + 1), dtype=np.float32)
    want = []
    for b in range(B):
        for i in range(gamma):
            drafts[b, i] = oracle.sample_token(q64[b, i], float(r.random()))
            x = drafts[b, i]
            for _ in range(1000):   # the acceptance test away from its boundary
                u = np.float32(r.random())
                if abs(float(u) * q64[b, i, x] - p64[b, i, x]) >= 1e-4 * max(p64[b, i, x], q64[b, i, x]):
                    break
            ua[b, i] = u
        n, _ = oracle.speculative_sample_chain(p64[b], q64[b], drafts[b], ua[b].astype(np.float64), [0.5] * (gamma + 1))
        row = oracle.residual(p64[b, n], q64[b, n]) if n < gamma else p64[b, gamma]
        ur[b] = 0.5
        ur[b, n] = _safe_u(r, row)
        want.append(oracle.speculative_sample_chain(p64[b], q64[b], drafts[b], ua[b].astype(np.float64),
                                                    ur[b].astype(np.float64)))
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, gamma + 1, dtype=torch.int32, device="cuda")
    qd = dev(q) if gamma else None
    M.medusa_speculative_sample(dev(p), qd, dev(drafts) if gamma else None, dev(ua) if gamma else None, dev(ur),
                                n_acc, out)
    torch.cuda.synchronize()
    n_got, out_got = n_acc.cpu().numpy(), out.cpu().numpy()
    for b, (n, toks) in enumerate(want):
        assert n_got[b] == n, (b, n_got[b], n)
        assert out_got[b, :n + 1].tolist() == toks and np.all(out_got[b, n + 1:] == -1)
    _say("ok, accepted:", [w[0] for w in want])


def test_speculative_sample_output_distribution_is_the_target():
    import speculative_decoding_medusa_amd as M
    _say("speculative sample toy distribution")
    p, q = oracle.TOY_P, oracle.TOY_Q
    G = 16   # grid per uniform: G^3 = 4096 sequences
    B = G ** 3
    P = np.tile(np.stack([p, p]).astype(np.float32), (B, 1, 1))
    Q = np.tile(q.astype(np.float32)[None], (B, 1, 1))
    drafts = np.zeros((B, 1), dtype=np.int32)
    ua = np.zeros((B, 1), dtype=np.float32)
    ur = np.zeros((B, 2), dtype=np.float32)
    k = 0
    for a in range(G):
        x = oracle.sample_token(q, (a + 0.5) / G)
        for bb in range(G):
            for c in range(G):
                drafts[k, 0] = x
                ua[k, 0] = (bb + 0.5) / G
                ur[k, 0] = (c + 0.5) / G
                ur[k, 1] = 0.5
                k += 1
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, 2, dtype=torch.int32, device="cuda")
    M.medusa_speculative_sample(dev(P), dev(Q), dev(drafts), dev(ua), dev(ur), n_acc, out)
    torch.cuda.synchronize()
    first = out.cpu().numpy()[:, 0]
    freq = np.bincount(first, minlength=4) / B
    assert np.allclose(freq, p, atol=0.04), freq
    # and the same counts as the oracle's on the same uniforms
    ref = [oracle.speculative_sample_chain(np.stack([p, p]), q[None], drafts[i], ua[i].astype(np.float64),
                                           ur[i].astype(np.float64))[1][0] for i in range(B)]
    assert np.array_equal(first, np.asarray(ref))


def test_speculative_sample_argument_errors():
    import speculative_decoding_medusa_amd as M
    p = torch.zeros(1, 2, 10, device="cuda")
    u = torch.zeros(1, 2, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.zeros(1, 2, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MedusaError) as e:   # gamma = 1 without q / drafts / u_accept
        M.medusa_speculative_sample(p, None, None, None, u, n, o)
    assert e.value.status == M.EINVAL
