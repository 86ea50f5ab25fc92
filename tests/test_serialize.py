"""Save / reload of quantized layers (Keras guide, "Save and reload the
quantized model": scales and packed weights survive, outputs are identical).
Host-only: CPU tensors, the oracle as the forward pass."""
import json

import numpy as np
import pytest
import torch

import workloads
from int4_weight_quantized_amd import serialize as ser


def layer_from_oracle(orc, scheme, K, N, g=0, bias=False, seed=0):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32)) if bias else None
    if scheme == "w4_sym":
        p, s = orc.quantize_weight_sym(W)
        return ser.QuantizedLayer(scheme, K, N, torch.from_numpy(p), torch.from_numpy(s), bias=b)
    if scheme == "w8_sym":
        q, s = orc.quantize_weight_w8(W)
        return ser.QuantizedLayer(scheme, K, N, torch.from_numpy(q), torch.from_numpy(s), bias=b)
    p, s, z = orc.quantize_weight_asym(W, g)
    return ser.QuantizedLayer(scheme, K, N, torch.from_numpy(p), torch.from_numpy(s),
                              torch.from_numpy(z), bias=b, group_size=g)


def test_roundtrip_all_schemes(orc, tmp_path):
    layers = {"up": layer_from_oracle(orc, "w4_sym", 1152, 96, bias=True, seed=1),
              "odd": layer_from_oracle(orc, "w4_sym", 33, 7, seed=2),
              "down": layer_from_oracle(orc, "w4_asym", 512, 40, g=128, seed=3),
              "int8": layer_from_oracle(orc, "w8_sym", 300, 17, bias=True, seed=4)}
    path = str(tmp_path / "model.safetensors")
    ser.save(path, layers)
    back = ser.load(path, device="cpu")
    assert set(back) == set(layers)
    for name, L in layers.items():
        R = back[name]
        assert R.record() == L.record()
        for f in ("packed", "scales", "zeros", "bias"):
            a, b = getattr(L, f), getattr(R, f)
            assert (a is None) == (b is None), (name, f)
            if a is not None:
                assert a.dtype == b.dtype and torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                                                          b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


def test_reloaded_forward_identical(orc, tmp_path):
    """The guide's check: the reloaded quantized layer gives the same outputs."""
    d = workloads.random_case(9, 4, 1152, 64, outliers=3, bias=True)
    p, s = orc.quantize_weight_sym(d["W"])
    L = ser.QuantizedLayer("w4_sym", 1152, 64, torch.from_numpy(p), torch.from_numpy(s),
                           bias=torch.from_numpy(d["bias"]))
    path = str(tmp_path / "l.safetensors")
    ser.save(path, {"dense": L})
    R = ser.load(path, device="cpu")["dense"]
    y0 = orc.w4a8_linear(d["x"], p, s, d["bias"])
    y1 = orc.w4a8_linear(d["x"], R.packed.numpy(), R.scales.numpy(), R.bias.numpy())
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def test_rejects_bad_inputs(orc, tmp_path):
    L = layer_from_oracle(orc, "w4_sym", 16, 4)
    bad = ser.QuantizedLayer("w4_sym", 16, 4, L.packed[:, :3].contiguous(), L.scales)
    with pytest.raises(ValueError):
        ser.save(str(tmp_path / "a.safetensors"), {"x": bad})
    with pytest.raises(ValueError):
        ser.save(str(tmp_path / "a.safetensors"), {"a.b": L})
    with pytest.raises(ValueError):
        ser.save(str(tmp_path / "a.safetensors"),
                 {"x": ser.QuantizedLayer("w3", 16, 4, L.packed, L.scales)})
    # a file whose record disagrees with its tensors, and a foreign file
    from safetensors.torch import save_file
    save_file({"x.packed": L.packed, "x.scales": L.scales}, str(tmp_path / "b.safetensors"),
              metadata={"format": ser.FORMAT,
                        "layer.x": json.dumps({"scheme": "w4_sym", "K": 18, "N": 4})})
    with pytest.raises(ValueError):
        ser.load(str(tmp_path / "b.safetensors"), device="cpu")
    save_file({"x.packed": L.packed}, str(tmp_path / "c.safetensors"), metadata={"format": "other"})
    with pytest.raises(ValueError):
        ser.load(str(tmp_path / "c.safetensors"), device="cpu")


def test_rejects_group_sizes_the_library_refuses(orc, tmp_path):
    """The same group rule as the C ABI: even, >= 2, dividing K."""
    p, s, z = orc.quantize_weight_asym(np.ones((12, 2), np.float32), 3)
    odd = ser.QuantizedLayer("w4_asym", 12, 2, torch.from_numpy(p), torch.from_numpy(s),
                             torch.from_numpy(z), group_size=3)
    with pytest.raises(ValueError, match="even group size"):
        ser.save(str(tmp_path / "g.safetensors"), {"x": odd})
    p, s, z = orc.quantize_weight_asym(np.ones((12, 2), np.float32), 4)
    ok = ser.QuantizedLayer("w4_asym", 12, 2, torch.from_numpy(p), torch.from_numpy(s),
                            torch.from_numpy(z), group_size=4)
    ser.save(str(tmp_path / "g.safetensors"), {"x": ok})
