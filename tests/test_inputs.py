"""The shared seeded input generator: known-answer vectors, C == NumPy, moments,
bf16 rounding against torch, and the static tree topologies."""
import collections

import numpy as np
import pytest
import torch

import medusa_inputs as mi

# Known-answer vectors of Philox4x32-10 as published with the Random123 library
# (Salmon et al., SC'11): (counter, key) -> output.
PHILOX_KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,out", PHILOX_KAT)
def test_philox_known_answers(ctr, key, out):
    assert mi.philox_block(ctr, key) == out
    got = mi.philox4x32_10_np(*[np.array([c], dtype=np.uint64) for c in ctr], key[0], key[1])
    assert [int(g[0]) for g in got] == out


def test_c_matches_numpy_definition():
    idx = np.concatenate([np.arange(5000), np.arange(2**32 - 100, 2**32 + 100), [2**40 + 17]])
    for seed, stream, sigma in [(1, 300, 0.02), (2**33 + 5, 0x100003, 1.0)]:
        ref = mi.normal_np(idx, seed, stream, sigma)
        got = np.concatenate([mi.normal((1,), seed, stream, sigma, "f32", offset=int(i)) for i in idx[5000:]])
        got = np.concatenate([mi.normal((5000,), seed, stream, sigma, "f32"), got])
        assert np.array_equal(got, ref)
        bf = mi.normal((5000,), seed, stream, sigma, "bf16")
        assert np.array_equal(bf, mi.f32_to_bf16_bits(ref[:5000]))


def test_normal_moments_and_bounds():
    x = mi.normal((2_000_000,), 11, 5, 1.0, "f32").astype(np.float64)
    n = x.size
    assert abs(x.mean()) < 5 / np.sqrt(n)
    # var of the sample variance of a near-normal: ~2/n (excess kurtosis -0.15)
    assert abs(x.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    assert np.abs(x).max() <= np.sqrt(24.0) + 1e-6
    w = mi.normal((1_000_000,), 11, 6, 0.02, "f32").astype(np.float64)
    assert abs(w.std() - 0.02) < 0.02 * 5 * np.sqrt(0.5 / w.size)


def test_bf16_rounding_matches_torch():
    x = np.concatenate([mi.normal((100000,), 3, 7, 3.0, "f32"),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mi.f32_to_bf16_bits(x), ref)


def test_uniform_int_range():
    v = mi.uniform_int((100000,), 4, 9, 1024, 8192)
    assert v.min() >= 1024 and v.max() <= 8192
    assert abs(v.mean() - (1024 + 8192) / 2) < 30


def _check_tree(t):
    parent, rank = t.arrays()
    assert parent[0] == -1
    for i in range(1, t.n):
        assert 0 <= parent[i] < i
        assert t.paths[i][:-1] == t.paths[parent[i]]
        assert t.paths[i][-1] == rank[i]
    sib = collections.Counter((int(parent[i]), int(rank[i])) for i in range(1, t.n))
    assert max(sib.values()) == 1


def test_tiny_tree_is_the_pages_2x3_example():
    # top-2 of head 1 x top-3 of head 2: six candidates sharing prefixes
    t = mi.tiny_tree()
    _check_tree(t)
    leaves = [p for p in t.paths if len(p) == 2]
    assert t.n == 9 and len(leaves) == 6
    assert sorted(leaves) == [(a, b) for a in range(2) for b in range(3)]


def test_sparse64_tree():
    t = mi.sparse_tree(64)
    _check_tree(t)
    assert t.n == 64
    assert collections.Counter(t.depth) == {0: 1, 1: 4, 2: 10, 3: 13, 4: 15, 5: 21}
    assert max(t.rank) == 3
    # best-first: every chosen node's prior product >= every unchosen child's
    chosen = set(t.paths)
    prod = lambda p: np.prod([mi.rank_prior(0.8, r) for r in p]) if p else 1.0
    worst = min(prod(p) for p in chosen)
    frontier = [p + (r,) for p in chosen if len(p) < 5 for r in range(8) if p + (r,) not in chosen]
    assert max(prod(p) for p in frontier) <= worst + 1e-15


def test_dense256_tree():
    t = mi.dense_tree(256)
    _check_tree(t)
    assert collections.Counter(t.depth) == {0: 1, 1: 3, 2: 9, 3: 27, 4: 81, 5: 135}


def test_configs_shapes():
    c1 = mi.config(1)
    assert (c1.H, c1.V, c1.K, c1.N, c1.nH * c1.D) == (256, 1000, 3, 9, 256)
    c2 = mi.config(2)
    assert (c2.H, c2.V, c2.K, c2.topk, c2.N, c2.nH, c2.D, c2.P) == (4096, 32000, 5, 4, 64, 32, 128, (2048,))
    c4 = mi.config(4)
    assert len(c4.P) == 8 and all(1024 <= p <= 8192 for p in c4.P)
