"""Parity of the fused-activation entry points (w4a8_linear_act, w8a8_linear_act)
with the CPU oracle: Y = relu(dequant(acc) + bias), bit-exact, on every kernel
the dispatcher picks (the single-launch decode GEMV with the activation
quantization in its prologue, the MFMA GEMV, the MFMA GEMM, the generic
kernel), and a two-layer decode chain shaped like the Keras guide's toy model
(Dense + ReLU, then Dense) on the Gemma-sized layer.
"""
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


def bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint32),
                          np.ascontiguousarray(b, np.float32).view(np.uint32))


CASES = [(1, 1152, 200, "gemv_dot4"), (2, 4096, 70, "gemv_dot4"), (3, 4096, 70, "gemv_mfma_fused"),
         (3, 1152, 70, "gemv_mfma_fused"), (4, 4096, 70, "gemv_mfma_fused"),
         (4, 8192, 70, "gemv_dot4"), (16, 512, 64, "gemv_mfma_fused"),
         (24, 512, 64, "gemv_mfma"),
         (100, 384, 260, "gemm_mfma"), (300, 384, 520, "gemm_mfma"),  # interior + edge tiles
         (32, 10, 32, "w4a8_generic"), (3, 7, 5, "w4a8_generic")]


@pytest.mark.parametrize("M,K,N,path", CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_w4a8_relu(M, K, N, path, with_bias):
    d = workloads.random_case(M * 7 + K + N, M, K, N, outliers=min(6, K), bias=with_bias)
    b = d.get("bias")
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.relu(oracle.w4a8_linear(d["x"], pref, sref, b))
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    y = W4.w4a8_linear_act(dev(d["x"]), packed, sw, bias=None if b is None else dev(b),
                           activation="relu")
    got = host(y)
    assert W4.w4_last_path() == path
    assert bits_equal(got, yref), f"path={path}"
    assert 0 < (got > 0).mean() < 1
    # activation=None is the plain forward
    y0 = W4.w4a8_linear_act(dev(d["x"]), packed, sw, bias=None if b is None else dev(b),
                            activation=None)
    assert bits_equal(host(y0), oracle.w4a8_linear(d["x"], pref, sref, b))


W8_CASES = [(1, 1152, 200, "w8_gemv_dot4"), (2, 4096, 64, "w8_gemv_dot4"),
            (3, 4096, 64, "w8_gemv_mfma_fused"), (12, 1152, 64, "w8_gemv_mfma_fused"),
            (4, 4096, 64, "w8_gemv_mfma_fused"), (2, 8192, 64, "w8_gemv_mfma"),
            (16, 512, 64, "w8_gemv_mfma_fused"), (24, 512, 64, "w8_gemv_mfma"),
            (100, 384, 260, "w8_gemm_mfma"),
            (300, 256, 516, "w8_gemm_mfma"),
            (32, 10, 32, "w8a8_generic")]


@pytest.mark.parametrize("M,K,N,path", W8_CASES)
def test_w8a8_relu(M, K, N, path):
    d = workloads.random_case(M * 5 + K + N, M, K, N, outliers=min(6, K), bias=True)
    qref, sref = oracle.quantize_weight_w8(d["W"])
    yref = oracle.relu(oracle.w8a8_linear(d["x"], qref, sref, d["bias"]))
    Wq, sw = W4.w8_quantize_weight(dev(d["W"]))
    y = W4.w8a8_linear_act(dev(d["x"]), Wq, sw, bias=dev(d["bias"]), activation="relu")
    got = host(y)
    assert W4.w4_last_path() == path
    assert bits_equal(got, yref), f"path={path}"


def test_decode_chain_gemma():
    """Two W4A8 layers as one decode step: Dense 1152 -> 6912 with bias and ReLU
    (one launch: activation quantization, product, dequantization, bias, ReLU),
    then Dense 6912 -> 1152."""
    rng = np.random.default_rng(2024)
    d = workloads.generate("gemma", M=1, bias=True)
    W2 = (rng.standard_normal((6912, 1152)) * 0.02).astype(np.float32)
    p1, s1 = oracle.quantize_weight_sym(d["W"])
    p2, s2 = oracle.quantize_weight_sym(W2)
    h = oracle.relu(oracle.w4a8_linear(d["x"], p1, s1, d["bias"]))
    yref = oracle.w4a8_linear(h, p2, s2)
    gp1, gs1, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    gp2, gs2, _ = W4.w4_quantize_weight(dev(W2), "sym")
    gh = W4.w4a8_linear_act(dev(d["x"]), gp1, gs1, bias=dev(d["bias"]), activation="relu")
    assert W4.w4_last_path() == "gemv_dot4"
    y = W4.w4a8_linear(gh, gp2, gs2)
    assert W4.w4_last_path() == "gemv_dot4"
    assert bits_equal(host(gh), h)
    assert bits_equal(host(y), yref)
