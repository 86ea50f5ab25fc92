"""Parity of weight dequantization and of the LoRA-style merge (Keras guide,
"Limitations": dequantize -> add delta -> requantize) with the CPU oracle,
bit-exact on the fp32 weights, codes, scales and zero points; and the
guide's save / reload check on the GPU path: a reloaded layer gives
bit-identical outputs."""
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


SYM = [(1, 1), (7, 5), (33, 70), (128, 64), (300, 129), (1152, 6912)]
ASYM = [(8, 3, 4), (256, 70, 128), (384, 5, 128), (1024, 130, 64)]


@pytest.mark.parametrize("K,N", SYM)
def test_dequant_sym(K, N):
    d = workloads.random_case(K + 3 * N, 1, K, N, sigma=0.02)
    p, s = oracle.quantize_weight_sym(d["W"])
    ref = oracle.dequant_weight(p, s, None, K)
    W = W4.w4_dequantize_weight(dev(p), dev(s), None, K, "sym")
    assert beq(host(W), ref)


@pytest.mark.parametrize("K,N,g", ASYM)
def test_dequant_asym(K, N, g):
    rng = np.random.default_rng(K * N + g)
    W = (rng.standard_normal((K, N)) * 0.015 + 0.003).astype(np.float32)
    p, s, z = oracle.quantize_weight_asym(W, g)
    ref = oracle.dequant_weight(p, s, z, K, g)
    got = W4.w4_dequantize_weight(dev(p), dev(s), dev(z), K, "asym", g)
    assert beq(host(got), ref)


def lora_delta(rng, K, N, r=8, scale=0.002):
    return ((rng.standard_normal((K, r)) @ rng.standard_normal((r, N))) * scale).astype(np.float32)


@pytest.mark.parametrize("K,N", [(7, 5), (300, 129), (1152, 6912)])
@pytest.mark.parametrize("in_place", [False, True])
def test_merge_sym(K, N, in_place):
    rng = np.random.default_rng(K + N)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    delta = lora_delta(rng, K, N)
    p, s = oracle.quantize_weight_sym(W)
    pr, sr, _ = oracle.merge_delta(p, s, None, K, delta)
    gp, gs = dev(p), dev(s)
    po, so, zo = W4.w4_merge_delta(gp, gs, None, dev(delta), "sym", in_place=in_place)
    assert zo is None
    assert beq(host(po), pr) and beq(host(so), sr)
    if in_place:
        assert po.data_ptr() == gp.data_ptr() and beq(host(gp), pr)
    assert not np.array_equal(pr, p)


@pytest.mark.parametrize("K,N,g", [(256, 70, 128), (1024, 130, 64)])
@pytest.mark.parametrize("in_place", [False, True])
def test_merge_asym(K, N, g, in_place):
    rng = np.random.default_rng(K + N + g)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    delta = lora_delta(rng, K, N)
    p, s, z = oracle.quantize_weight_asym(W, g)
    pr, sr, zr = oracle.merge_delta(p, s, z, K, delta, g)
    po, so, zo = W4.w4_merge_delta(dev(p), dev(s), dev(z), dev(delta), "asym", g,
                                   in_place=in_place)
    assert beq(host(po), pr) and beq(host(so), sr) and beq(host(zo), zr)


def test_save_reload_gpu(tmp_path):
    """Quantize on the GPU, save, reload onto the GPU: bit-identical layers and
    outputs for a W4A8 layer (with bias), a W8A8 layer and a W4A16 layer."""
    from int4_weight_quantized_amd import serialize as ser
    d = workloads.random_case(12, 8, 1152, 256, outliers=3, bias=True)
    X, W, b = dev(d["x"]), dev(d["W"]), dev(d["bias"])
    p, s, _ = W4.w4_quantize_weight(W, "sym")
    q8, s8 = W4.w8_quantize_weight(W)
    pa, sa, za = W4.w4_quantize_weight(W, "asym", 128)
    layers = {"w4": ser.QuantizedLayer("w4_sym", 1152, 256, p, s, bias=b),
              "w8": ser.QuantizedLayer("w8_sym", 1152, 256, q8, s8),
              "g128": ser.QuantizedLayer("w4_asym", 1152, 256, pa, sa, za, group_size=128)}
    path = str(tmp_path / "q.safetensors")
    ser.save(path, layers)
    R = ser.load(path, device=DEV)
    y0 = W4.w4a8_linear(X, p, s, bias=b)
    y1 = W4.w4a8_linear(X, R["w4"].packed, R["w4"].scales, bias=R["w4"].bias)
    assert beq(host(y0), host(y1))
    z0 = W4.w8a8_linear(X, q8, s8)
    z1 = W4.w8a8_linear(X, R["w8"].packed, R["w8"].scales)
    assert beq(host(z0), host(z1))
    xb = X.to(torch.bfloat16)
    u0 = W4.w4a16_linear(xb, pa, sa, za, 128)
    u1 = W4.w4a16_linear(xb, R["g128"].packed, R["g128"].scales, R["g128"].zeros, 128)
    assert beq(host(u0), host(u1))
