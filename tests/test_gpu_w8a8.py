"""Parity of the W8A8 path (int8 per-channel weights: the INT8 path that the
Keras guide's "How it works" says the INT4 path follows, minus the unpacking)
with the CPU oracle, through the C ABI.

Bar: bit-exact on int8 codes, scales, int32 accumulators and fp32 outputs (the
output is a fixed sequence of fp32 roundings).  Cases cover every kernel the
dispatcher picks for 8-bit weights -- dot4 GEMV (M <= 4, K % 32 == 0,
K <= 4096), MFMA GEMV (M <= 64, K % 128 == 0), MFMA GEMM (M > 64) and the
generic kernel -- with ragged rows and channels; the full-size workloads run
whole on the GPU and are compared on sampled rows x channels.
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


CANARY = {torch.int8: -91, torch.float32: -12345.5, torch.int32: -0x5A5A5A5A}


def guarded(shape, dtype):
    """A contiguous output tensor with 256-byte canary regions on both sides."""
    n = int(np.prod(shape))
    pad = 256 // torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((pad + n + pad,), CANARY[dtype], dtype=dtype, device=DEV)
    return buf, buf[pad:pad + n].view(*shape), pad


def guards_intact(buf, pad):
    c = CANARY[buf.dtype]
    return bool((buf[:pad].cpu() == c).all()) and bool((buf[-pad:].cpu() == c).all())


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.astype(np.float32).view(np.uint32))
    return np.array_equal(a, b)


def report(name, got, want):
    bad = np.argwhere(~(got == want))
    return f"{name}: {len(bad)} mismatches, first {bad[:5].tolist()}"


# ---------------------------------------------------------- weight quantization
@pytest.mark.parametrize("K,N", [(1, 1), (10, 32), (32, 1), (7, 5), (33, 70), (128, 64),
                                 (300, 129), (1152, 6912)])
def test_quantize_weight_w8(K, N):
    d = workloads.random_case(K * 11 + N, 1, K, N, sigma=0.02)
    W = d["W"]
    if N > 3:
        W[:, 3] = 0.0                            # all-zero channel
    if K >= 8 and N > 1:                         # exact ties at scale 1
        W[:8, 1] = [127, 2.5, -2.5, 0.5, -0.5, 1.5, -3.5, 100.4]
        W[8:, 1] = 0
    qref, sref = oracle.quantize_weight_w8(W)
    bufq, Wq, pq = guarded((N, K), torch.int8)
    bufs, sw, ps = guarded((N,), torch.float32)
    W4.w8_quantize_weight(dev(W), Wq=Wq, sw=sw)
    assert bits_equal(host(sw), sref)
    assert np.array_equal(host(Wq), qref), report("Wq", host(Wq), qref)
    assert guards_intact(bufq, pq) and guards_intact(bufs, ps)


def test_quantize_weight_w8_full_7b():
    d = workloads.generate("mlp7b", M=1)
    qref, sref = oracle.quantize_weight_w8(d["W"])
    Wq, sw = W4.w8_quantize_weight(dev(d["W"]))
    assert bits_equal(host(sw), sref)
    assert np.array_equal(host(Wq), qref)


# ------------------------------------------------------- integer products
I32_CASES = [
    (1, 128, 16), (1, 1152, 100), (2, 4096, 33), (3, 96, 17), (4, 1152, 257),  # dot4
    (1, 8192, 40),                                                              # K > 4096: MFMA GEMV
    (5, 128, 16), (8, 1152, 130), (16, 4096, 96), (17, 256, 65), (33, 512, 31), (64, 1152, 200),
    (16, 256, 12304), (40, 128, 9232), (64, 256, 6160),  # MFMA GEMV, 4 / 3 / 2 channel blocks
    (65, 128, 130), (130, 256, 129), (256, 1152, 384), (300, 512, 1000),       # GEMM
    (1, 10, 32), (32, 10, 32), (32, 32, 1), (6, 96, 20), (3, 7, 5), (70, 200, 9),  # generic
]


@pytest.mark.parametrize("M,K,N", I32_CASES)
def test_w8a8_matmul_i32(M, K, N):
    xq = workloads.random_int8(M * 29 + K, (M, K))
    Wq = workloads.random_int8(K * 19 + N + 7, (N, K))      # every value incl. -128
    ref = oracle.matmul_w8_i32(xq, Wq)
    bufa, acc, pa = guarded((M, N), torch.int32)
    W4.w8a8_matmul_i32(dev(xq), dev(Wq), acc=acc)
    got = host(acc)
    assert np.array_equal(got, ref), report(f"acc path={W4.w4_last_path()}", got, ref)
    assert guards_intact(bufa, pa)


@pytest.mark.parametrize("M,K", [(1, 4096), (8, 4096), (128, 4096), (1, 131008)])
def test_w8a8_matmul_extremes(M, K):
    """-128 times -128 everywhere: the largest accumulator magnitude, 16384 K
    (K = 131008 is the largest multiple of 128 the boundary accepts)."""
    N = 48
    xq = np.full((M, K), -128, np.int8)
    Wq = np.full((N, K), -128, np.int8)
    acc = W4.w8a8_matmul_i32(dev(xq), dev(Wq))
    assert np.all(host(acc) == 16384 * K), W4.w4_last_path()


# ----------------------------------------------------------- W8A8 linear
LIN_CASES = [(1, 1152, 200), (1, 4096, 300), (4, 256, 70), (2, 8192, 64), (8, 1152, 130),
             (16, 512, 64), (64, 256, 33), (16, 256, 12304), (40, 128, 9232), (100, 384, 260),
             (32, 10, 32), (9, 40, 7)]


@pytest.mark.parametrize("M,K,N", LIN_CASES)
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_linear(M, K, N, with_bias):
    d = workloads.random_case(M + K + N + 3, M, K, N, outliers=min(6, K), bias=with_bias)
    qref, sref = oracle.quantize_weight_w8(d["W"])
    b = d.get("bias")
    yref = oracle.w8a8_linear(d["x"], qref, sref, b)
    Wq, sw = W4.w8_quantize_weight(dev(d["W"]))
    bufy, y, py = guarded((M, N), torch.float32)
    W4.w8a8_linear(dev(d["x"]), Wq, sw, bias=None if b is None else dev(b), Y=y)
    got = host(y)
    assert bits_equal(got, yref), report(f"y path={W4.w4_last_path()}", got, yref)
    assert np.all(np.abs(got - yref) <= 1e-5 * np.abs(yref))
    assert guards_intact(bufy, py)


def _sample(n, k, seed):
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, k) - 2, replace=False)]))


@pytest.mark.parametrize("name,M,path", [("gemma", 1, "w8_gemv_dot4"), ("gemma", 8, "w8_gemv_mfma_fused"),
                                         ("mlp7b", 1, "w8_gemv_dot4"),
                                         ("mlp7b", 16, "w8_gemv_mfma"),
                                         ("mlp7b", 64, "w8_gemv_mfma"),
                                         ("prefill", None, "w8_gemm_mfma")])
def test_w8a8_full_workloads(name, M, path):
    """Full-size layers with 8-bit weights; sampled rows x channels against the oracle."""
    d = workloads.generate(name, M=M)
    W, X = d["W"], d["x"]
    Wq, sw = W4.w8_quantize_weight(dev(W))
    y = W4.w8a8_linear(dev(X), Wq, sw)
    assert W4.w4_last_path() == path
    got = host(y)
    rows = _sample(X.shape[0], 64, 3)
    cols = _sample(W.shape[1], 256, 4)
    qref, sref = oracle.quantize_weight_w8(np.ascontiguousarray(W[:, cols]))
    assert np.array_equal(host(Wq)[cols], qref) and bits_equal(host(sw)[cols], sref)
    yref = oracle.w8a8_linear(np.ascontiguousarray(X[rows]), qref, sref)
    sub = got[np.ix_(rows, cols)]
    assert bits_equal(sub, yref), report(f"{name} M={M} path={path}", sub, yref)
    assert np.all(np.isfinite(got))
