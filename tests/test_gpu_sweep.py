"""Seeded random sweep of layer shapes through the C ABI against the oracle:
M from 1 to 300 (dot4 GEMV, MFMA GEMV of every channel-block width, GEMM,
generic kernel), K with and without the fast paths' alignment, ragged N,
random bias and ReLU; W4A8 on both weight layouts and W8A8 bit-exact, and
W4A16 over random group sizes within the fp32 summation bound."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

W4 = None
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def w4():
    global W4
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_weight_quantized_amd as pkg
    pkg.lib()
    W4 = pkg
    return pkg


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b, np.float32).view(np.uint32))


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 40, 64, 65, 100, 257, 300]))
        kind = i % 3
        if kind == 0:
            K = 128 * int(rng.integers(1, 9))                 # MFMA and shuffled-tile paths
        elif kind == 1:
            K = 32 * int(rng.integers(1, 33))                 # dot4 alignment only
        else:
            K = int(rng.integers(1, 300))                     # generic kernel
        N = int(rng.integers(1, 700)) if i % 5 else int(rng.integers(6144, 13000))
        if M * K * N > 1.5e8:
            M = max(1, int(1.5e8 // (K * N)))
        out.append((M, K, N, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("M,K,N,bias,relu", _shapes(36, 2025) + _shapes(40, 1) + _shapes(40, 2))
def test_random_layer(M, K, N, bias, relu):
    d = workloads.random_case(M * 131 + K * 7 + N, M, K, N, outliers=min(4, K), bias=bias)
    b = d.get("bias")
    act = "relu" if relu else None
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, b)
    if relu:
        yref = oracle.relu(yref)
    X = dev(d["x"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    assert np.array_equal(host(packed), pref)
    bb = None if b is None else dev(b)
    y = host(W4.w4a8_linear_act(X, packed, sw, bias=bb, activation=act))
    assert same_bits(y, yref), f"w4a8 path={W4.w4_last_path()}"
    if K % 128 == 0:
        wpp = W4.w4_prepack_weights(packed)
        y2 = host(W4.w4a8_linear_prepacked(X, wpp, sw, bias=bb, activation=act))
        assert same_bits(y2, yref), f"prepacked path={W4.w4_last_path()}"
    qref, s8 = oracle.quantize_weight_w8(d["W"])
    y8ref = oracle.w8a8_linear(d["x"], qref, s8, b)
    if relu:
        y8ref = oracle.relu(y8ref)
    Wq, sw8 = W4.w8_quantize_weight(dev(d["W"]))
    y8 = host(W4.w8a8_linear_act(X, Wq, sw8, bias=bb, activation=act))
    assert same_bits(y8, y8ref), f"w8a8 path={W4.w4_last_path()}"


def _w4a16_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        g = int(rng.choice([4, 32, 64, 128, 128, 128]))
        K = g * int(rng.integers(1, 17))
        if i % 3 == 0:
            K = 512 * int(rng.integers(1, 5))            # LDS-staged kernel (group 128)
            g = 128
        M = int(rng.choice([1, 2, 5, 8, 16, 17, 33, 64]))
        N = int(rng.integers(1, 400)) if i % 4 else int(rng.integers(1000, 3000))
        if M * K * N > 1.5e8:
            M = max(1, int(1.5e8 // (K * N)))
        out.append((M, K, N, g))
    return out


@pytest.mark.parametrize("M,K,N,g", _w4a16_shapes(40, 7))
def test_random_w4a16(M, K, N, g):
    """W4A16 over random shapes and group sizes against the fp64 oracle sum:
    norm-wise 1e-5 and the elementwise gamma_K bound of the fp32 summation."""
    rng = np.random.default_rng(M * 977 + K * 13 + N + g)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    xb = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    pref, sref, zref = oracle.quantize_weight_asym(W, g)
    yref, absy = oracle.w4a16_linear(xb, pref, sref, zref, g)
    packed, s, z = W4.w4_quantize_weight(dev(W), "asym", g)
    assert np.array_equal(host(packed), pref)
    y = host(W4.w4a16_linear(dev(xb.view(np.int16)), packed, s, z, g))
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    diff = np.abs(y.astype(np.float64) - yref)
    assert np.linalg.norm(diff) <= 1e-5 * np.linalg.norm(yref), W4.w4_last_path()
    assert np.all(diff <= gamma * absy + 1e-30), W4.w4_last_path()
