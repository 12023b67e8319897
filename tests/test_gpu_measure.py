"""The read-ceiling measurement kernel reads every byte it is given: the XOR
each workgroup writes equals the XOR of its slice computed on the host."""
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
