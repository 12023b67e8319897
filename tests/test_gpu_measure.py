"""The measurement kernels do the work they are timed on: the read-ceiling
and read-mix kernels load every word they are given (the XOR each workgroup
writes equals the XOR of its loads computed on the host), and the matrix-rate
kernel's products come out exact on constant operands."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,n_wg", [(1 << 20, 64), ((1 << 20) + 48, 37), (4096, 300)])
def test_stream_read_covers_every_byte(nbytes, n_wg):
    import speculative_decoding_medusa_amd as M
    r = np.random.default_rng(nbytes)
    host = r.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((n_wg,), -1, dtype=torch.int32, device="cuda")
    M.medusa_stream_read(buf, sink, n_wg=n_wg)
    torch.cuda.synchronize()
    words = host.reshape(-1, 4)          # 16-byte units
    per = -(-len(words) // n_wg)
    want = np.zeros(n_wg, dtype=np.uint32)
    for g in range(n_wg):
        sl = words[g * per:min(len(words), (g + 1) * per)]
        want[g] = np.bitwise_xor.reduce(sl.ravel()) if sl.size else 0
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("wp,sp,rounds,n_wg,w16", [
    (8, 0, 5, 5, 3 * 2048),     # window only (3 rounds' worth): reads wrap at its end
    (0, 8, 2, 7, 0),            # private slices only
    (4, 2, 5, 3, 3 * 1024),     # 2 : 1 mix
    (8, 4, 3, 4, 2 * 2048),
], ids=["window", "stream", "mix42", "mix84"])
def test_read_mix_covers_every_load(wp, sp, rounds, n_wg, w16):
    import speculative_decoding_medusa_amd as M
    r = np.random.default_rng(1000 * wp + sp)
    win = r.integers(0, 1 << 32, (max(w16, 1), 4), dtype=np.uint32)
    ssz = rounds * sp * 256 * n_wg
    src = r.integers(0, 1 << 32, (max(ssz, 1), 4), dtype=np.uint32)
    wdev = torch.from_numpy(win.view(np.int32)).cuda() if wp else None
    sdev = torch.from_numpy(src.view(np.int32)).cuda() if sp else None
    sink = torch.full((n_wg,), -1, dtype=torch.int32, device="cuda")
    M.medusa_read_mix(wdev, sdev, wp, sp, rounds, sink, n_wg=n_wg)
    torch.cuda.synchronize()
    want = np.zeros(n_wg, dtype=np.uint32)
    for g in range(n_wg):
        acc = np.uint32(0)
        for rr in range(rounds):
            if wp:
                idx = ((rr * wp * 256) % w16 + np.arange(wp * 256)) % w16
                acc ^= np.bitwise_xor.reduce(win[idx].ravel())
        if sp:
            per = rounds * sp * 256
            acc ^= np.bitwise_xor.reduce(src[g * per:(g + 1) * per].ravel())
        want[g] = acc
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)


def test_mfma_rate_products_are_exact_on_constant_operands():
    import speculative_decoding_medusa_amd as M
    n_wg, iters = 3, 10
    out = torch.full((n_wg * 256,), -1.0, device="cuda")
    M.medusa_mfma_rate(False, iters, out, n_wg=n_wg)
    torch.cuda.synchronize()
    assert torch.all(out == float(iters * 64 * 128))   # 128 accumulator elements of iters x 4 x 16 ones
    M.medusa_mfma_rate(True, iters, out, n_wg=n_wg)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o)) and len(np.unique(o)) > n_wg * 64
