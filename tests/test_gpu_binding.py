"""The Python binding checks every tensor against the sizes its call implies
and raises before anything is launched: the C entry points take raw device
pointers and trust the sizes, so a mis-sized output or table would otherwise
become an out-of-range access in a kernel.  Each case here fails in the
binding; the well-formed calls around them still run and agree with the
fresh-tensor results.
"""
import numpy as np
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


def _layer(M=4, K=256, N=48, seed=0):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(M, K, generator=g).to(DEV)
    W = (torch.randn(K, N, generator=g) * 0.02).to(DEV)
    return X, W


def test_w4a8_shapes_rejected():
    X, W = _layer()
    M, K = X.shape
    N = W.shape[1]
    packed, sw, _ = W4.w4_quantize_weight(W, "sym")
    ref = W4.w4a8_linear(X, packed, sw)
    with pytest.raises(ValueError, match="sw must have shape"):
        W4.w4a8_linear(X, packed, sw[:-1].contiguous())
    with pytest.raises(ValueError, match="bias must have shape"):
        W4.w4a8_linear(X, packed, sw, bias=torch.zeros(N + 1, device=DEV))
    with pytest.raises(ValueError, match="Y must have shape"):
        W4.w4a8_linear(X, packed, sw, Y=torch.empty(M, N - 1, device=DEV))
    with pytest.raises(ValueError, match="packed must have shape"):
        W4.w4a8_linear(X[:, :128].contiguous(), packed, sw)
    with pytest.raises(ValueError, match="2-D"):
        W4.w4a8_linear(X.reshape(-1), packed, sw)
    with pytest.raises(ValueError, match="acc must have shape"):
        Xq, _ = W4.a8_quantize_act(X)
        W4.w4a8_matmul_i32(Xq, packed, acc=torch.empty(M + 1, N, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="GPU tensor"):
        W4.w4a8_linear(X, packed, sw.cpu())
    # the rejected calls launched nothing: a well-formed call into a given Y
    # still gives the same bits
    Y = torch.full((M, N), float("nan"), device=DEV)
    W4.w4a8_linear(X, packed, sw, Y=Y)
    torch.cuda.synchronize()
    assert torch.equal(Y, ref)


def test_quantizer_outputs_checked():
    X, W = _layer()
    K, N = W.shape
    with pytest.raises(ValueError, match="packed must have shape"):
        W4.w4_quantize_weight(W, "sym",
                              packed=torch.empty(N, K // 2 - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="scales must have shape"):
        W4.w4_quantize_weight(W, "asym", 128, scales=torch.empty(N, 1, device=DEV))
    with pytest.raises(ValueError, match="sx must have shape"):
        W4.a8_quantize_act(X, sx=torch.empty(X.shape[0] - 1, device=DEV))
    with pytest.raises(ValueError, match="Wq must have shape"):
        W4.w8_quantize_weight(W, Wq=torch.empty(N, K + 1, dtype=torch.int8, device=DEV))


def test_w4a16_and_layouts_checked():
    X, W = _layer(M=16, K=512, N=64)
    M, K = X.shape
    N = W.shape[1]
    packed, s, z = W4.w4_quantize_weight(W, "asym", 128)
    xb = X.to(torch.bfloat16)
    ref = W4.w4a16_linear(xb, packed, s, z, 128)
    with pytest.raises(TypeError, match="bfloat16"):
        W4.w4a16_linear(X, packed, s, z, 128)            # fp32 is not bf16
    with pytest.raises(ValueError, match="zeros must have shape"):
        W4.w4a16_linear(xb, packed, s, z[:, :-1].contiguous(), 128)
    wpp, szpp = W4.w4a16_prepack(packed, s, z)
    with pytest.raises(ValueError, match="szpp must have shape"):
        W4.w4a16_linear_prepacked(xb, wpp, szpp[:-4].contiguous(), N)
    y2 = W4.w4a16_linear_prepacked(xb, wpp, szpp, N)
    torch.cuda.synchronize()
    assert torch.equal(y2, ref)
    p8, sw, _ = W4.w4_quantize_weight(W, "sym")
    w8pp = W4.w4_prepack_weights(p8)
    with pytest.raises(ValueError, match="wpp must have shape"):
        W4.w4a8_linear_prepacked(X, w8pp[:-16].contiguous(), sw)
    with pytest.raises(ValueError, match="wpp must have shape"):
        W4.w4_unprepack_weights(w8pp, K, N + 16)
    assert np.array_equal(W4.w4_unprepack_weights(w8pp, K, N).cpu().numpy(), p8.cpu().numpy())
