"""Save and reload quantized layers (Keras INT4 guide, "Save and reload the
quantized model": the quantization metadata -- scales and packed weights --
is kept, so the reloaded model gives the same outputs).

File format: one safetensors file.  For a layer named ``L`` the tensors are
``L.packed`` (uint8 [N, ceil(K/2)] int4 codes, or int8 [N, K] for ``w8_sym``),
``L.scales`` (fp32 [N] or [N, K/group]), ``L.zeros`` (asymmetric groups
only) and ``L.bias`` (optional, fp32 [N]).  The header metadata holds a
format tag and, per layer, a JSON record ``{"scheme", "K", "N",
"group_size"}`` under the key ``layer.L``.  Loading checks every shape and
dtype against that record.  Reading goes through safetensors, which parses a
JSON header and raw little-endian arrays and executes nothing from the file.

This is host-side I/O only: tensors are copied to host memory to be written
and placed on ``device`` when read; no arithmetic is done on them.
"""
from __future__ import annotations

import json
from dataclasses import dataclass

import torch

FORMAT = "int4-weight-quantized-linear/1"
SCHEMES = ("w4_sym", "w4_asym", "w8_sym")


@dataclass
class QuantizedLayer:
    """One quantized linear layer: codes, scales and (optionally) zero points
    and bias, with the metadata needed to run it."""
    scheme: str
    K: int
    N: int
    packed: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor | None = None
    bias: torch.Tensor | None = None
    group_size: int = 0

    def expected(self) -> dict:
        """Shape and dtype of every tensor the scheme requires."""
        K, N, g = self.K, self.N, self.group_size
        if self.scheme == "w4_sym":
            return {"packed": ((N, (K + 1) // 2), torch.uint8), "scales": ((N,), torch.float32)}
        if self.scheme == "w8_sym":
            return {"packed": ((N, K), torch.int8), "scales": ((N,), torch.float32)}
        if self.scheme == "w4_asym":
            if g < 2 or g % 2 or K % g:
                raise ValueError(f"w4_asym needs an even group size >= 2 dividing K "
                                 f"(K={K}, group={g})")
            return {"packed": ((N, (K + 1) // 2), torch.uint8),
                    "scales": ((N, K // g), torch.float32), "zeros": ((N, K // g), torch.float32)}
        raise ValueError(f"unknown scheme {self.scheme!r}; expected one of {SCHEMES}")

    def validate(self) -> None:
        if self.K < 1 or self.N < 1:
            raise ValueError(f"bad layer size K={self.K}, N={self.N}")
        want = self.expected()
        for name, (shape, dtype) in want.items():
            t = getattr(self, name)
            if t is None:
                raise ValueError(f"{self.scheme} layer is missing {name}")
            if tuple(t.shape) != shape or t.dtype != dtype:
                raise ValueError(f"{name}: expected {dtype} {shape}, got {t.dtype} {tuple(t.shape)}")
        if self.scheme != "w4_asym" and self.zeros is not None:
            raise ValueError(f"{self.scheme} layer has no zero points")
        if self.bias is not None and (tuple(self.bias.shape) != (self.N,)
                                      or self.bias.dtype != torch.float32):
            raise ValueError("bias must be fp32 [N]")

    def record(self) -> dict:
        return {"scheme": self.scheme, "K": self.K, "N": self.N, "group_size": self.group_size}


def save(path: str, layers: dict[str, QuantizedLayer]) -> None:
    """Write the layers (any device) to one safetensors file."""
    from safetensors.torch import save_file

    tensors, meta = {}, {"format": FORMAT}
    for name, L in layers.items():
        if "." in name or not name:
            raise ValueError(f"layer name {name!r} must be non-empty and contain no '.'")
        L.validate()
        for field in ("packed", "scales", "zeros", "bias"):
            t = getattr(L, field)
            if t is not None:
                tensors[f"{name}.{field}"] = t.detach().to("cpu").contiguous()
        meta[f"layer.{name}"] = json.dumps(L.record())
    save_file(tensors, path, metadata=meta)


def load(path: str, device: str | torch.device = "cuda") -> dict[str, QuantizedLayer]:
    """Read a file written by ``save``; tensors are placed on ``device``."""
    from safetensors import safe_open

    out = {}
    with safe_open(path, framework="pt", device="cpu") as f:
        meta = f.metadata() or {}
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not a {FORMAT} file (format={meta.get('format')!r})")
        keys = set(f.keys())
        for mk, mv in meta.items():
            if not mk.startswith("layer."):
                continue
            name = mk[len("layer."):]
            rec = json.loads(mv)
            get = (lambda fld: f.get_tensor(f"{name}.{fld}").to(device)
                   if f"{name}.{fld}" in keys else None)
            L = QuantizedLayer(scheme=rec["scheme"], K=int(rec["K"]), N=int(rec["N"]),
                               group_size=int(rec.get("group_size", 0)), packed=get("packed"),
                               scales=get("scales"), zeros=get("zeros"), bias=get("bias"))
            L.validate()
            out[name] = L
        stray = {k for k in keys if k.split(".", 1)[0] not in out}
        if stray:
            raise ValueError(f"{path}: tensors without a layer record: {sorted(stray)[:5]}")
    return out
