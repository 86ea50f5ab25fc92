"""The library under HIP graph capture: each entry point captured once with
torch.cuda.CUDAGraph, then replayed several times with new data written
into the captured input and the same call run eagerly in between; every
replay must give the eager result bit for bit.  The benchmark times graph
replays, so this checks that what it times computes the right thing on
every path the dispatcher picks (the fused decode GEMV, the fused and the
two-launch MFMA GEMV, the GEMM, W8A8, W4A16 and the shuffled tiles).  The
library records no memset or allocation of its own into a graph: the
workspace and outputs come from the binding's torch tensors.
"""
import pytest
import torch

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


def _weights(K, N, seed):
    g = torch.Generator().manual_seed(seed)
    W = (torch.randn(K, N, generator=g) * 0.02).to(DEV)
    b = (torch.randn(N, generator=g) * 0.1).to(DEV)
    return W, b


def _op(kind, W, b, K):
    if kind == "w4a8":
        packed, sw, _ = W4.w4_quantize_weight(W, "sym")
        return (lambda X: W4.w4a8_linear(X, packed, sw, bias=b)), "gemv"
    if kind == "w4a8_relu_pp":
        packed, sw, _ = W4.w4_quantize_weight(W, "sym")
        wpp = W4.w4_prepack_weights(packed)
        return (lambda X: W4.w4a8_linear_prepacked(X, wpp, sw, bias=b, activation="relu")), "pp"
    if kind == "w8a8":
        Wq, sw = W4.w8_quantize_weight(W)
        return (lambda X: W4.w8a8_linear(X, Wq, sw, bias=b)), "w8"
    if kind == "w4a16":
        packed, s, z = W4.w4_quantize_weight(W, "asym", 128)
        return (lambda X: W4.w4a16_linear(X.to(torch.bfloat16), packed, s, z, 128)), "w4a16"
    raise ValueError(kind)


CASES = [
    ("w4a8", 1, 1152, 6912, "gemv_dot4"),
    ("w4a8", 8, 1152, 6912, "gemv_mfma_fused"),
    ("w4a8", 16, 4096, 1024, "gemv_mfma_fused"),     # 16 waves, one row each
    ("w4a8", 24, 4096, 1024, "gemv_mfma"),
    ("w4a8", 300, 512, 520, "gemm_mfma"),
    ("w4a8_relu_pp", 8, 1152, 1000, "gemv_mfma_fused_prepacked"),
    ("w8a8", 16, 4096, 1024, "w8_gemv_mfma"),
    ("w8a8", 1, 1152, 700, "w8_gemv_dot4"),
    ("w4a16", 16, 512, 70, "w4a16_lds"),
]


@pytest.mark.parametrize("kind,M,K,N,path", CASES)
def test_graph_replays_match_eager(kind, M, K, N, path):
    W, b = _weights(K, N, M + K + N)
    op, _ = _op(kind, W, b, K)
    gen = torch.Generator().manual_seed(7 * M + K)
    Xs = torch.randn(M, K, generator=gen).to(DEV)   # the captured input
    op(Xs)
    assert W4.w4_last_path() == path
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        op(Xs)                                       # warm-up off the default stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Yg = op(Xs)
    for r in range(3):
        Xs.copy_(torch.randn(M, K, generator=gen).to(DEV) * (1.0 + r))
        Ye = op(Xs)                                  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg, Ye), f"replay {r} differs from the eager result ({path})"
    del g
