"""The decode GEMV's one-block-per-CU launch shape (int4 codes, fused
activation quantization, M <= 2; on shuffled tiles from 8 chunks per lane):
layers with more than 16 output
channels per CU run 32, 48 or 64 channels per block, each lane requesting
part of its weight chunks before the activation quantization and the rest
after it.  Bit-exact against the CPU oracle over every chunk count (K from 96
to 8192), every block width, ragged last blocks, bias, ReLU and the AWQ
division; the kernel that ran is checked for the expected block width."""
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


def expected_rows(N):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in (16, 32, 48):
        if N <= rows * cus:
            return rows
    return 64


# (M, K, N): K = 96, 1152, 2048, 4096, 8192 give 2, 3, 4, 8, 16 chunks per lane;
# N spans every block width on a 256-CU device, with ragged last blocks
CASES = [(1, 1152, 6912), (1, 4096, 11008), (2, 4096, 11008), (1, 96, 4100), (2, 1152, 8200),
         (1, 2048, 12300), (2, 2048, 5000), (1, 8192, 9000), (2, 8192, 4097), (1, 4096, 20000),
         (2, 96, 16500)]


@pytest.mark.parametrize("M,K,N", CASES)
def test_wide_dot4_bit_exact(M, K, N):
    d = workloads.random_case(M * 11 + K + N, M, K, N, outliers=min(6, K), bias=True)
    b = d["bias"]
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, b)
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    X, bb = dev(d["x"]), dev(b)
    y = W4.w4a8_linear(X, packed, sw, bias=bb)
    got = host(y)
    assert W4.w4_last_path() == "gemv_dot4"
    rows = expected_rows(N)
    assert f"ILi{M}ELi{rows}E" in W4.w4_last_kernel(), W4.w4_last_kernel()
    assert bits_equal(got, yref)
    yr = W4.w4a8_linear_act(X, packed, sw, bias=bb, activation="relu")
    assert bits_equal(host(yr), oracle.relu(yref))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 11008), (2, 1152, 8200)])
def test_wide_dot4_awq(M, K, N):
    d = workloads.random_case(M * 5 + K + N, M, K, N, outliers=min(6, K), bias=True)
    s = oracle.awq_channel_scales(d["x"], (1, 4))
    p, sw = oracle.quantize_weight_sym(oracle.awq_fold_weight(d["W"], s))
    yref = oracle.w4a8_linear_awq(d["x"], p, sw, s, d["bias"])
    gs = W4.awq_channel_scales(dev(d["x"]), (1, 4))
    gp, gsw, _ = W4.w4_quantize_weight(W4.awq_fold_weight(dev(d["W"]), gs), "sym")
    y = W4.w4a8_linear_awq(dev(d["x"]), gp, gsw, gs, bias=dev(d["bias"]))
    assert W4.w4_last_path() == "gemv_dot4"
    assert f"ILi{M}ELi{expected_rows(N)}E" in W4.w4_last_kernel()
    assert bits_equal(host(y), yref)


@pytest.mark.parametrize("M,K,N", [(1, 1152, 6912), (2, 4096, 11008), (1, 2048, 16500),
                                   (1, 8192, 4100), (2, 3072, 9000)])
def test_wide_dot4_prepacked(M, K, N):
    d = workloads.random_case(M * 13 + K + N, M, K, N, outliers=min(6, K), bias=True)
    pref, sref = oracle.quantize_weight_sym(d["W"])
    yref = oracle.w4a8_linear(d["x"], pref, sref, d["bias"])
    packed, sw, _ = W4.w4_quantize_weight(dev(d["W"]), "sym")
    wpp = W4.w4_prepack_weights(packed)
    y = W4.w4a8_linear_prepacked(dev(d["x"]), wpp, sw, bias=dev(d["bias"]))
    assert W4.w4_last_path() == "gemv_dot4_prepacked"
    chunks = (K // 32 + 15) // 16  # chunks per lane before rounding up to an instantiated count
    rows = expected_rows(N) if chunks > 4 else 16
    assert f"ILi{M}ELi{rows}E" in W4.w4_last_kernel()
    assert bits_equal(host(y), yref)


@pytest.mark.parametrize("M,K,N", [(1, 1152, 6912), (2, 4096, 11008), (2, 96, 4100)])
def test_dot4_w8_keeps_16_channels(M, K, N):
    d = workloads.random_case(M * 17 + K + N, M, K, N, outliers=min(6, K), bias=True)
    qref, sref = oracle.quantize_weight_w8(d["W"])
    yref = oracle.w8a8_linear(d["x"], qref, sref, d["bias"])
    Wq, sw = W4.w8_quantize_weight(dev(d["W"]))
    y = W4.w8a8_linear(dev(d["x"]), Wq, sw, bias=dev(d["bias"]))
    assert W4.w4_last_path() == "w8_gemv_dot4"
    assert f"ILi{M}ELi16E" in W4.w4_last_kernel()
    assert bits_equal(host(y), yref)
