"""Parity of the AWQ-style channel scaling ("INT4" concept entry, section 4.4)
with the CPU oracle, bit-exact: the channel scales from calibration rows, the
weight fold W diag(s), the int8 activation quantization of X / s, the bf16
activation division, and the W4A8 forward with the division fused into the
activation quantization (single-launch decode kernel for M <= 4, the
activation kernel otherwise); plus the end-to-end W4A16 path with AWQ."""
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


def beq(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.astype(np.float32).view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("M,K,alpha", [(64, 4096, (1, 2)), (7, 1152, (1, 4)), (3, 33, (1, 1)),
                                       (128, 11008, (3, 4))])
def test_channel_scales(M, K, alpha):
    rng = np.random.default_rng(M + K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, min(6, K), replace=False)
    X[:, cols] *= np.float32(50.0)
    X[:, 0] = 0.0                                    # all-zero channel
    if K > 2:
        X[:, 1] = np.float32(1e-40)                  # subnormal magnitude
    ref = oracle.awq_channel_scales(X, alpha)
    got = W4.awq_channel_scales(dev(X), alpha)
    assert beq(host(got), ref)


def test_channel_scales_zero_median():
    X = np.array([[0.0, 0.0, 2.0**-140], [0.0, 0.0, -(2.0**-141)]], np.float32)
    assert beq(host(W4.awq_channel_scales(dev(X), (1, 1))), oracle.awq_channel_scales(X, (1, 1)))


def test_fold_and_act():
    d = workloads.generate("mlp7b", M=16)
    X, W = d["x"], d["W"][:, :300].copy()
    s = oracle.awq_channel_scales(X)
    assert beq(host(W4.awq_fold_weight(dev(W), dev(s))), oracle.awq_fold_weight(W, s))
    Wg = dev(W)
    W4.awq_fold_weight(Wg, dev(s), W_out=Wg)         # in place
    assert beq(host(Wg), oracle.awq_fold_weight(W, s))
    xq, sx = W4.awq_quantize_act(dev(X), dev(s))
    rq, rs = oracle.awq_quantize_act(X, s)
    assert beq(host(xq), rq) and beq(host(sx), rs)
    # arbitrary (non power of two) divisors take the same correctly rounded path
    s2 = (1.0 + np.random.default_rng(1).random(X.shape[1])).astype(np.float32)
    xq2, sx2 = W4.awq_quantize_act(dev(X), dev(s2))
    rq2, rs2 = oracle.awq_quantize_act(X, s2)
    assert beq(host(xq2), rq2) and beq(host(sx2), rs2)


def test_scale_bf16():
    rng = np.random.default_rng(3)
    x = workloads.to_bf16_bits(rng.standard_normal((16, 8192)).astype(np.float32))
    for s in [oracle.awq_channel_scales(rng.standard_normal((4, 8192)).astype(np.float32) *
                                        (1 + 50 * (rng.random(8192) < 0.001)).astype(np.float32)),
              (1.0 + rng.random(8192)).astype(np.float32)]:
        got = W4.awq_scale_act_bf16(dev(x.view(np.int16)), dev(s))
        assert np.array_equal(host(got).view(np.uint16), oracle.awq_scale_bf16(x, s))


CASES = [(1, 1152, 200, "gemv_dot4"), (4, 4096, 96, "gemv_dot4"), (16, 512, 64, "gemv_mfma"),
         (100, 384, 260, "gemm_mfma"), (9, 40, 7, "w4a8_generic")]


@pytest.mark.parametrize("M,K,N,path", CASES)
def test_w4a8_linear_awq(M, K, N, path):
    d = workloads.random_case(M * 3 + K + N, M, K, N, outliers=min(6, K), bias=True)
    s = oracle.awq_channel_scales(d["x"], (1, 4))
    Wf = oracle.awq_fold_weight(d["W"], s)
    p, sw = oracle.quantize_weight_sym(Wf)
    yref = oracle.w4a8_linear_awq(d["x"], p, sw, s, d["bias"])
    gs = W4.awq_channel_scales(dev(d["x"]), (1, 4))
    gp, gsw, _ = W4.w4_quantize_weight(W4.awq_fold_weight(dev(d["W"]), gs), "sym")
    y = W4.w4a8_linear_awq(dev(d["x"]), gp, gsw, gs, bias=dev(d["bias"]))
    assert W4.w4_last_path() == path
    assert beq(host(y), yref), path
    yr = W4.w4a8_linear_awq(dev(d["x"]), gp, gsw, gs, bias=dev(d["bias"]), activation="relu")
    assert beq(host(yr), oracle.relu(yref))


def test_w4a16_awq_end_to_end():
    """70B-class layer slice (N = 1024, all of K): scales from 32 calibration
    rows, fold, asymmetric group-128 quantization, bf16 division, W4A16
    forward; against the oracle within the fp32 summation bound."""
    d = workloads.w4a16_inputs(N=1024)
    rng = np.random.default_rng(9)
    K = d["K"]
    cal = rng.standard_normal((32, K)).astype(np.float32)
    cols = rng.choice(K, 6, replace=False)
    cal[:, cols] *= 50.0
    xb = d["x_bf16"].copy()
    xf = oracle.bf16_bits_to_f32(xb).copy()
    xf[:, cols] *= 50.0
    xb = workloads.to_bf16_bits(xf)
    s = oracle.awq_channel_scales(cal)
    pa, sa, za = oracle.quantize_weight_asym(oracle.awq_fold_weight(d["W"], s), 128)
    yref, absy = oracle.w4a16_linear(oracle.awq_scale_bf16(xb, s), pa, sa, za, 128)
    gs = W4.awq_channel_scales(dev(cal))
    assert beq(host(gs), s)
    gp, gsa, gza = W4.w4_quantize_weight(W4.awq_fold_weight(dev(d["W"]), gs), "asym", 128)
    xs = W4.awq_scale_act_bf16(dev(xb.view(np.int16)), gs)
    y = host(W4.w4a16_linear(xs, gp, gsa, gza, 128)).astype(np.float64)
    gamma = K * 2.0**-24 / (1 - K * 2.0**-24)
    assert np.all(np.abs(y - yref) <= gamma * absy)
    assert np.linalg.norm(y - yref) <= 1e-5 * np.linalg.norm(yref)
