"""Pins of the oracle's GPU-shuffled ("prepacked") W4A16 layout: a pure
rearrangement of the canonical packed bytes and group tables, so it is pinned
by what a rearrangement must satisfy and by spot checks derived by hand from
its definition (16-byte chunk p of channel c holds canonical chunk
p ^ ((c/2) % 4); table entries interleave (scale, zero) of groups 2u, 2u+1):

* the inverse gives back every input byte and table entry (ragged N too);
* every channel's bytes are a permutation of its canonical bytes, padding
  channels are zero;
* literal positions: channel 2 (swizzle 1) stores chunk 1 in slot 0; channel 7
  (swizzle 3) stores chunk 2 in slot 1 of every 128-k step; channel 16 starts
  the second block.
"""
import numpy as np
import pytest


def random_tables(rng, N, K):
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    G = K // 128
    scales = (rng.random((N, G)) + 0.5).astype(np.float32)
    zeros = rng.integers(-20, 30, size=(N, G)).astype(np.float32)
    return packed, scales, zeros


@pytest.mark.parametrize("N,K", [(16, 512), (37, 512), (5, 1024), (48, 2048)])
def test_roundtrip(orc, N, K):
    rng = np.random.default_rng(N * K)
    p, s, z = random_tables(rng, N, K)
    wpp, szpp = orc.w4a16_prepack(p, s, z, K)
    assert wpp.shape == ((N + 15) // 16, K // 128, 16, 64) and szpp.shape == ((N + 15) // 16, K // 256, 16, 4)
    p2, s2, z2 = orc.w4a16_unprepack(wpp, szpp, K, N)
    assert np.array_equal(p2, p) and np.array_equal(s2, s) and np.array_equal(z2, z)


def test_permutation_and_padding(orc):
    rng = np.random.default_rng(3)
    N, K = 37, 1024
    p, s, z = random_tables(rng, N, K)
    wpp, szpp = orc.w4a16_prepack(p, s, z, K)
    per_ch = wpp.transpose(0, 2, 1, 3).reshape(-1, K // 2)       # [N16, K/2] in stored order
    for n in range(N):
        assert np.array_equal(np.sort(per_ch[n]), np.sort(p[n]))
    assert np.all(per_ch[N:] == 0)
    tab = szpp.transpose(0, 2, 1, 3).reshape(-1, K // 128, 2)     # [N16, G, (s, z)]
    assert np.array_equal(tab[:N, :, 0], s) and np.array_equal(tab[:N, :, 1], z)
    assert np.all(tab[N:] == 0)


def test_literal_positions(orc):
    N, K = 20, 512
    p = (np.arange(N * K // 2, dtype=np.int64) * 7 % 251).astype(np.uint8).reshape(N, K // 2)
    s = np.arange(N * 4, dtype=np.float32).reshape(N, 4) + 0.5
    z = -np.arange(N * 4, dtype=np.float32).reshape(N, 4)
    wpp, szpp = orc.w4a16_prepack(p, s, z, K)
    assert np.array_equal(wpp[0, 0, 2, 0:16], p[2, 16:32])            # channel 2, slot 0 <- chunk 1
    for t in range(4):
        assert np.array_equal(wpp[0, t, 7, 16:32], p[7, 64 * t + 32:64 * t + 48])  # ch 7, slot 1 <- chunk 2
    assert np.array_equal(wpp[0, 3, 0, :], p[0, 192:256])             # channel 0: no swizzle
    assert np.array_equal(wpp[1, 1, 0, 48:64], p[16, 64 + 48:64 + 64])  # block 1 = channel 16
    assert szpp[0, 1, 5].tolist() == [s[5, 2], z[5, 2], s[5, 3], z[5, 3]]
    assert szpp[1, 0, 3].tolist() == [s[19, 0], z[19, 0], s[19, 1], z[19, 1]]
    assert np.all(wpp[1, :, 4:] == 0)                                 # channels 20..31 pad


def test_rejects_unsupported_k(orc):
    p = np.zeros((16, 128), np.uint8)
    with pytest.raises(orc.OracleError):
        orc.w4a16_prepack(p, np.ones((16, 2), np.float32), np.zeros((16, 2), np.float32), 256)


@pytest.mark.parametrize("N,K", [(16, 128), (37, 384), (5, 1152), (300, 4096)])
def test_weights_only_roundtrip_and_agreement(orc, N, K):
    """The weight part alone: its own round trip for K % 128 == 0, and the same
    bytes as the full W4A16 conversion where both are defined."""
    rng = np.random.default_rng(N + K)
    p = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    wpp = orc.w4_prepack_weights(p, K)
    assert np.array_equal(orc.w4_unprepack_weights(wpp, K, N), p)
    per_ch = wpp.transpose(0, 2, 1, 3).reshape(-1, K // 2)
    for n in range(N):
        assert np.array_equal(np.sort(per_ch[n]), np.sort(p[n]))
    assert np.array_equal(wpp[0, K // 128 - 1, 3, 0:16], p[3, K // 2 - 64 + 16:K // 2 - 64 + 32])
    if K % 512 == 0:
        s = np.ones((N, K // 128), np.float32)
        w16, _ = orc.w4a16_prepack(p, s, s, K)
        assert np.array_equal(w16, wpp)
