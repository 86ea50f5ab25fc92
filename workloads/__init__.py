"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random tensors; it holds none of the quantization
arithmetic, so the oracle and the HIP path can both be fed from it without
sharing any of the method's code.

Recipe (one stream per tensor): ``numpy.random.SeedSequence(20251014 + index)``
spawned into four generators used for X, W, the bias and the choice of
outlier columns.  All draws are fp32.

* ``toy``      -- the Keras guide's minimal model: Dense 10->32 (ReLU) then
                  Dense 32->1, x ~ U[0,1) of shape [32, 10], weights ~ N(0, 0.1),
                  zero biases (Keras Dense default).
* ``gemma``    -- Gemma3-1B-like MLP up-projection: x ~ N(0,1) [M, 1152],
                  W ~ N(0, 0.02) [1152, 6912], M in {1, 8}.
* ``mlp7b``    -- 7B-class MLP: x ~ N(0,1) [M, 4096] with 6 distinct outlier
                  columns scaled x50 (LLM activation outliers), W ~ N(0, 0.02)
                  [4096, 11008], M in {1, 16, 64}.
* ``prefill``  -- 7B-class prefill: x [4096, 4096] as above, W [4096, 4096].
* ``w4a16``    -- 70B-class MLP, weight-only: x ~ N(0,1) rounded to bf16
                  [16, 8192], W ~ N(0, 0.015) [8192, 28672], group 128.

The pages benchmark trained models (Gemma3, Falcon, Llama, OPT) that are not
available; these tensors stand in for their layer shapes and value ranges.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BASE_SEED = 20251014


@dataclass(frozen=True)
class Shape:
    name: str
    index: int          # seed offset
    M: int
    K: int
    N: int
    x_dist: str         # "uniform" or "normal"
    w_sigma: float
    outliers: int = 0
    group: int = 0      # >0: asymmetric group-wise W4A16


GEMMA_K, GEMMA_N = 1152, 6912
MLP7B_K, MLP7B_N = 4096, 11008
PREFILL = 4096
W4A16_M, W4A16_K, W4A16_N, W4A16_G = 16, 8192, 28672, 128

SHAPES = {
    "toy_l1": Shape("toy_l1", 0, 32, 10, 32, "uniform", 0.1),
    "gemma": Shape("gemma", 1, 1, GEMMA_K, GEMMA_N, "normal", 0.02),
    "mlp7b": Shape("mlp7b", 2, 1, MLP7B_K, MLP7B_N, "normal", 0.02, outliers=6),
    "prefill": Shape("prefill", 3, PREFILL, PREFILL, PREFILL, "normal", 0.02, outliers=6),
    "w4a16": Shape("w4a16", 4, W4A16_M, W4A16_K, W4A16_N, "normal", 0.015, group=W4A16_G),
}


def _rngs(index: int):
    ss = np.random.SeedSequence(BASE_SEED + index)
    return [np.random.default_rng(s) for s in ss.spawn(4)]


def make_x(rng, M, K, dist="normal", outliers=0, rng_o=None) -> np.ndarray:
    if dist == "uniform":
        x = rng.random((M, K), dtype=np.float32)
    else:
        x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        cols = rng_o.choice(K, outliers, replace=False)
        x[:, cols] *= np.float32(50.0)
    return x


def make_w(rng, K, N, sigma) -> np.ndarray:
    w = rng.standard_normal((K, N), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def generate(name: str, M: int | None = None, with_w: bool = True, bias: bool = False):
    """Inputs of one named workload: dict with x [M,K] fp32, W [K,N] fp32 and
    optionally a bias [N] ~ N(0, 1).  ``M`` overrides the shape's row count."""
    sh = SHAPES[name]
    rx, rw, rb, ro = _rngs(sh.index)
    m = sh.M if M is None else M
    out = {"shape": sh, "M": m, "K": sh.K, "N": sh.N}
    out["x"] = make_x(rx, m, sh.K, sh.x_dist, sh.outliers, ro)
    if with_w:
        out["W"] = make_w(rw, sh.K, sh.N, sh.w_sigma)
    if bias:
        out["bias"] = rb.standard_normal(sh.N, dtype=np.float32)
    return out


def toy_model():
    """The two-layer toy model: x [32,10], W1 [10,32], b1 = 0, W2 [32,1], b2 = 0."""
    rx, rw, _rb, _ro = _rngs(0)
    x = rx.random((32, 10), dtype=np.float32)
    W1 = make_w(rw, 10, 32, 0.1)
    W2 = make_w(rw, 32, 1, 0.1)
    return {"x": x, "W1": W1, "b1": np.zeros(32, np.float32),
            "W2": W2, "b2": np.zeros(1, np.float32)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 inputs to bf16 (torch's CPU conversion) and return the bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def w4a16_inputs(M: int | None = None, N: int | None = None, with_w: bool = True):
    """The weight-only workload: x as bf16 bits [M, K]; W fp32 [K, N].
    ``N`` < full width takes the first N columns (for sampled checks)."""
    sh = SHAPES["w4a16"]
    rx, rw, _rb, _ro = _rngs(sh.index)
    m = sh.M if M is None else M
    x = make_x(rx, m, sh.K, "normal")
    out = {"shape": sh, "M": m, "K": sh.K, "N": sh.N, "group": sh.group,
           "x_bf16": to_bf16_bits(x)}
    if with_w:
        W = make_w(rw, sh.K, sh.N, sh.w_sigma)
        if N is not None:
            W = np.ascontiguousarray(W[:, :N])
        out["W"] = W
    return out


def random_case(seed: int, M: int, K: int, N: int, sigma=0.02, outliers=0, bias=False):
    """A small random problem for parity sweeps."""
    rx, rw, rb, ro = _rngs(1000 + seed)
    d = {"x": make_x(rx, M, K, "normal", min(outliers, K), ro),
         "W": make_w(rw, K, N, sigma)}
    if bias:
        d["bias"] = rb.standard_normal(N, dtype=np.float32)
    return d


def random_bytes(seed: int, shape) -> np.ndarray:
    """Uniform random bytes (every nibble value, including code -8)."""
    rng = np.random.default_rng(BASE_SEED + 5000 + seed)
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def random_int8(seed: int, shape) -> np.ndarray:
    """Uniform random int8 values over the full range [-128, 127]."""
    rng = np.random.default_rng(BASE_SEED + 7000 + seed)
    return rng.integers(-128, 128, size=shape, dtype=np.int8)
