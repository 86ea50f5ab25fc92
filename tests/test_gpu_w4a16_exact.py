"""W4A16: every dequantized weight the kernels feed to the matrix unit, exactly.

"4-bit Integer Quantization for LLMs", quantization principle: a weight is
dequantized at compute time as (W_int4 - zero_point) * scale; here
w' = bf16_rne(fl(fl(q - zero) * scale)).  The summation-order bounds of the
other W4A16 tests cannot see a single wrong w' (one slip moves y by far less
than gamma_K * sum |x w'|).  With one-hot activation rows, x = e_k, every
output is one product, y[m][n] = 1.0 * w'[k][n], which is exact in any
summation order: the kernels' outputs must equal the oracle's dequantized
weights value for value (+0 and -0 count as equal).

X is the K x K identity (every k, hence every lane, quarter-wave, stage slot,
ring stage and K half of the kernels, is one row), on random codes (every
nibble), scales that are not powers of two, and zero points inside the fast
range [-112, 128], outside it and fractional, so that both the fast and the
direct dequantization run (each wave votes per stage).
"""
import numpy as np
import pytest
import torch

import int4_weight_quantized_amd as W4
import oracle
import workloads

pytestmark = pytest.mark.gpu

BF16_ONE = 0x3F80


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def one_hot_rows(ks, K):
    X = np.zeros((len(ks), K), np.uint16)
    X[np.arange(len(ks)), ks] = BF16_ONE
    return X.view(np.int16)


def random_tables(rng, K, N, g, p_direct=0.03):
    """Random packed codes, scales and zero points [N][K/g].  Most zero points
    are integers in [-112, 128]; a few are outside that range or fractional."""
    G = K // g
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = np.exp(rng.uniform(np.log(1e-3), np.log(0.2), (N, G))).astype(np.float32)
    m, _ = np.frexp(scales)
    scales[m == 0.5] *= np.float32(1.25)  # no power of two
    zeros = rng.integers(-112, 129, (N, G)).astype(np.float32)
    odd = rng.random((N, G)) < p_direct
    kinds = rng.integers(0, 4, (N, G))
    zeros[odd & (kinds == 0)] = rng.integers(-400, -112, int((odd & (kinds == 0)).sum()))
    zeros[odd & (kinds == 1)] = rng.integers(129, 400, int((odd & (kinds == 1)).sum()))
    frac = odd & (kinds >= 2)
    zeros[frac] = rng.integers(-20, 30, int(frac.sum())) + np.float32(0.5) * rng.choice(
        [-1, 1], int(frac.sum())) * rng.choice([0.5, 1.0], int(frac.sum()))
    zeros[0, 0], zeros[N // 2, G // 2], zeros[N - 1, G - 1] = -200.0, 250.0, 3.5
    return packed, scales, zeros


def expected(packed, scales, zeros, K, g):
    """[K][N] fp32 values of the oracle's bf16 dequantized weights."""
    return oracle.bf16_bits_to_f32(oracle.w4a16_dequant(packed, scales, zeros, K, g))


def check_identity(K, N, g, seed, prepacked=False, want_path=None):
    rng = np.random.default_rng(seed)
    packed, scales, zeros = random_tables(rng, K, N, g)
    want = expected(packed, scales, zeros, K, g)
    X = dev(one_hot_rows(np.arange(K), K))
    if prepacked:
        wpp, szpp = W4.w4a16_prepack(dev(packed), dev(scales), dev(zeros), g)
        y = W4.w4a16_linear_prepacked(X, wpp, szpp, N)
    else:
        y = W4.w4a16_linear(X, dev(packed), dev(scales), dev(zeros), g)
    path = W4.w4_last_path()
    got = host(y)
    if want_path:
        assert path == want_path, path
    bad = got != want
    assert not bad.any(), (f"{path}: {int(bad.sum())} of {bad.size} dequantized weights differ, "
                           f"first at (k, n) = {tuple(np.argwhere(bad)[0])}")


# group 128, K % 512 == 0: the LDS-staged kernel; N picks 1, 2, 4 and 7 waves per
# K half (one round of channel blocks over the CUs); K gives 4, 3 and 2 stages
# per half (the 3-stage ring wraps at 4)
LDS_CASES = [(2048, 200), (2048, 4100), (1536, 8200), (1536, 16400), (1024, 4097)]


@pytest.mark.parametrize("K,N", LDS_CASES)
def test_lds_kernel_dequantizes_exactly(K, N):
    check_identity(K, N, 128, seed=K + N, want_path="w4a16_lds")


@pytest.mark.parametrize("K,N", LDS_CASES)
def test_prepacked_kernel_dequantizes_exactly(K, N):
    check_identity(K, N, 128, seed=K + N + 1, prepacked=True, want_path="w4a16_lds_prepacked")


# the register-ring kernel: group 128 with K % 512 != 0, and groups 32 and 64
@pytest.mark.parametrize("K,N,g", [(640, 300, 128), (1152, 70, 128), (1024, 200, 32),
                                   (1024, 129, 64), (384, 64, 32)])
def test_mfma_kernel_dequantizes_exactly(K, N, g):
    check_identity(K, N, g, seed=K * 7 + N + g, want_path="w4a16_mfma")


# anything else: K % 128 != 0, or a group that is not a multiple of 32
@pytest.mark.parametrize("K,N,g", [(96, 40, 32), (256, 33, 16), (200, 17, 2)])
def test_generic_kernel_dequantizes_exactly(K, N, g):
    check_identity(K, N, g, seed=K + N + g, want_path="w4a16_generic")


def test_full_layer_sampled_rows_exact():
    """The 70B-class layer (8192 x 28672, group 128) as quantized by the
    library: 16 one-hot rows whose k cover both K halves, every quarter-wave
    and both steps of a stage, against the oracle's dequantization of the
    same codes, scales and zero points (the 128-k group of each k)."""
    d = workloads.w4a16_inputs()
    W, g = d["W"], d["group"]
    K, N = W.shape
    packed, s, z = W4.w4_quantize_weight(dev(W), "asym", g)
    P, S, Z = host(packed), host(s), host(z)
    rng = np.random.default_rng(5)
    ks = np.array([0, 31, 32, 95, 127, 128, 255, 4095, 4096, 4097, 6000, 8191,
                   *rng.integers(0, K, 4)])
    X = dev(one_hot_rows(ks, K))
    wpp, szpp = W4.w4a16_prepack(packed, s, z, g)
    for prepacked in (False, True):
        y = (W4.w4a16_linear_prepacked(X, wpp, szpp, N) if prepacked
             else W4.w4a16_linear(X, packed, s, z, g))
        got = host(y)
        for m, k in enumerate(ks):
            gi = k // g
            want = expected(np.ascontiguousarray(P[:, gi * g // 2:(gi + 1) * g // 2]),
                            np.ascontiguousarray(S[:, gi:gi + 1]),
                            np.ascontiguousarray(Z[:, gi:gi + 1]), g, g)[k % g]
            assert np.array_equal(got[m], want), (prepacked, int(k))
