"""Parity of the GPU-shuffled W4A16 layout: the conversion kernels against the
oracle's definition (bit-exact), the round trip, and the W4A16 forward on the
shuffled layout against the oracle (the fp32 summation bound) and against the
canonical-layout kernel (bit-identical: the same products in the same
order), on ragged channel counts and the full 70B-class layer."""
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


def quantized(rng, K, N):
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    return oracle.quantize_weight_asym(W, 128)


@pytest.mark.parametrize("K,N", [(512, 16), (512, 37), (1024, 130), (4096, 1000)])
def test_prepack_roundtrip(K, N):
    rng = np.random.default_rng(K + N)
    p, s, z = quantized(rng, K, N)
    wref, szref = oracle.w4a16_prepack(p, s, z, K)
    wpp, szpp = W4.w4a16_prepack(dev(p), dev(s), dev(z))
    assert np.array_equal(host(wpp), wref.ravel())
    assert np.array_equal(host(szpp).view(np.uint32), szref.ravel().view(np.uint32))
    p2, s2, z2 = W4.w4a16_unprepack(wpp, szpp, K, N)
    assert np.array_equal(host(p2), p)
    assert np.array_equal(host(s2), s) and np.array_equal(host(z2), z)


@pytest.mark.parametrize("M,K,N", [(16, 512, 16), (16, 1024, 130), (5, 2048, 600), (33, 512, 4200),
                                   (16, 8192, 1000)])
def test_linear_prepacked(M, K, N):
    rng = np.random.default_rng(M * K + N)
    p, s, z = quantized(rng, K, N)
    xb = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    yref, absy = oracle.w4a16_linear(xb, p, s, z, 128)
    wpp, szpp = W4.w4a16_prepack(dev(p), dev(s), dev(z))
    X = dev(xb.view(np.int16))
    y = host(W4.w4a16_linear_prepacked(X, wpp, szpp, N))
    assert W4.w4_last_path() == "w4a16_lds_prepacked"
    gamma = K * 2.0**-24 / (1 - K * 2.0**-24)
    assert np.all(np.abs(y.astype(np.float64) - yref) <= gamma * absy)
    assert np.linalg.norm(y - yref) <= 1e-5 * np.linalg.norm(yref)
    y0 = host(W4.w4a16_linear(X, dev(p), dev(s), dev(z), 128))
    assert W4.w4_last_path() == "w4a16_lds"
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))


def test_linear_prepacked_full_70b():
    """The 70B-class layer: whole on the GPU, both layouts bit-identical;
    sampled channels against the oracle."""
    d = workloads.w4a16_inputs()
    K, N = d["K"], d["N"]
    p, s, z = W4.w4_quantize_weight(dev(d["W"]), "asym", 128)
    X = dev(d["x_bf16"].view(np.int16))
    wpp, szpp = W4.w4a16_prepack(p, s, z)
    y = host(W4.w4a16_linear_prepacked(X, wpp, szpp, N))
    y0 = host(W4.w4a16_linear(X, p, s, z, 128))
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(5).choice(N, 62, replace=False)]))
    pr, sr, zr = oracle.quantize_weight_asym(np.ascontiguousarray(d["W"][:, cols]), 128)
    yref, absy = oracle.w4a16_linear(d["x_bf16"], pr, sr, zr, 128)
    gamma = K * 2.0**-24 / (1 - K * 2.0**-24)
    assert np.all(np.abs(y[:, cols].astype(np.float64) - yref) <= gamma * absy)


# ------------------------------------------- W4A8 on the shuffled int4 tiles
@pytest.mark.parametrize("K,N", [(128, 16), (1152, 37), (4096, 300)])
def test_w4_prepack_weights(K, N):
    rng = np.random.default_rng(K * 3 + N)
    p = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    wpp = W4.w4_prepack_weights(dev(p))
    assert np.array_equal(host(wpp), oracle.w4_prepack_weights(p, K).ravel())
    assert np.array_equal(host(W4.w4_unprepack_weights(wpp, K, N)), p)


W4A8_PP = [(1, 1152, 200, "gemv_dot4_prepacked"), (2, 4096, 70, "gemv_dot4_prepacked"),
           (3, 4096, 70, "gemv_mfma_fused_prepacked"),
           (4, 4096, 70, "gemv_mfma_fused_prepacked"),
           (3, 8192 + 128, 40, "gemv_mfma_prepacked"), (8, 1152, 130, "gemv_mfma_fused_prepacked"),
           (16, 4096, 96, "gemv_mfma_prepacked"), (64, 512, 33, "gemv_mfma_prepacked"),
           (100, 384, 260, "gemm_mfma_prepacked"), (300, 1152, 1000, "gemm_mfma_prepacked"),
           # the decode-batch kernel's 4, 3 and 2 channel-block widths
           (16, 256, 12304, "gemv_mfma_fused_prepacked"), (40, 128, 9232, "gemv_mfma_prepacked"),
           (64, 256, 6160, "gemv_mfma_prepacked")]


@pytest.mark.parametrize("M,K,N,path", W4A8_PP)
@pytest.mark.parametrize("relu", [False, True])
def test_w4a8_linear_prepacked(M, K, N, path, relu):
    d = workloads.random_case(M + K + 7 * N, M, K, N, outliers=6, bias=True)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, d["bias"])
    if relu:
        yref = oracle.relu(yref)
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    wpp = W4.w4_prepack_weights(packed)
    act = "relu" if relu else None
    y = host(W4.w4a8_linear_prepacked(dev(d["x"]), wpp, sw, bias=dev(d["bias"]), activation=act))
    assert W4.w4_last_path() == path
    assert np.array_equal(y.view(np.uint32), yref.view(np.uint32)), path
    y0 = host(W4.w4a8_linear_act(dev(d["x"]), packed, sw, bias=dev(d["bias"]), activation=act))
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))


def test_w4a8_prepacked_unaligned_x():
    """X not 16-byte aligned: the MFMA paths still apply (activation kernel)."""
    d = workloads.random_case(11, 2, 512, 48, outliers=2)
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    wpp = W4.w4_prepack_weights(packed)
    buf = torch.zeros(2 * 512 + 1, dtype=torch.float32, device=DEV)
    X = buf[1:].view(2, 512)
    X.copy_(dev(d["x"]))
    y = host(W4.w4a8_linear_prepacked(X, wpp, sw))
    assert W4.w4_last_path() == "gemv_mfma_prepacked"
    pref, sref = oracle.quantize_weight_sym(d["W"])
    assert np.array_equal(y.view(np.uint32), oracle.w4a8_linear(d["x"], pref, sref).view(np.uint32))


@pytest.mark.parametrize("name,M", [("gemma", 1), ("mlp7b", 16), ("prefill", None)])
def test_w4a8_prepacked_full_workloads(name, M):
    d = workloads.generate(name, M=M)
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    wpp = W4.w4_prepack_weights(packed)
    X = dev(d["x"])
    y = host(W4.w4a8_linear_prepacked(X, wpp, sw))
    y0 = host(W4.w4a8_linear(X, packed, sw))
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    rows = np.arange(min(8, y.shape[0]))
    cols = np.arange(0, d["N"], max(1, d["N"] // 64))
    pref, sref = oracle.quantize_weight_sym(np.ascontiguousarray(d["W"][:, cols]))
    yref = oracle.w4a8_linear(np.ascontiguousarray(d["x"][rows]), pref, sref)
    assert np.array_equal(y[np.ix_(rows, cols)].view(np.uint32), yref.view(np.uint32))
