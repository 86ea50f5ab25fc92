"""CPU oracle of the INT4 weight-quantized linear layer (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never loads it and shares no code with it.

The arithmetic lives in ``w4_oracle.c`` (plain scalar C, one IEEE binary32
operation per step, round-half-to-even); this module only marshals numpy
arrays.  The formulas and their sources are documented there:

* symmetric per-output-channel int4 weights (scale = absmax / 7, codes in
  [-8, 7], two per byte) -- Keras INT4 guide, "How it works", steps 1-2;
* per-row dynamic int8 activations (scale = absmax / 127) -- same, step 3;
* the toy model's ReLU on a Dense output (after the bias);
* weight dequantization and the lossy LoRA merge (dequantize, add the delta,
  requantize) -- Keras guide, "Limitations";
* the GPU-shuffled ("prepacked") W4A16 layout and its inverse -- a pure
  rearrangement, defined here (the pages fix no such layout);
* AWQ-style activation-aware channel scaling (calibration magnitudes ->
  power-of-two channel scales, W diag(s), x / s) -- "INT4" concept entry,
  section 4.4;
* exact int8 x int4 products summed in int32 -- steps 4-5;
* dequantization by input_scale * per_channel_kernel_scale -- step 6;
* symmetric per-output-channel int8 weights (scale = absmax / 127, codes in
  [-128, 127], one per byte) and the W8A8 forward -- the INT8 path that the
  Keras guide's "How it works" says the INT4 path follows apart from the
  unpacking; "INT4" concept entry, section 4.1 with b = 8;
* asymmetric group-wise int4 (scale = range / 15, zero point, codes 0..15)
  and the weight-only W4A16 product -- "4-bit Integer Quantization for LLMs",
  quantization principle; "INT4" concept entry, sections 4.1, 4.2 and 4.5.

Parity status: every function here is pinned by the CPU pin tests
(brute force, closed forms, invariants, hand-derived golden fixtures).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# W4_ORACLE_LIB may name another build of the same source (the host
# sanitizer build of build.py --sanitize).
_LIB_PATH = os.environ.get("W4_ORACLE_LIB") or os.path.join(_HERE, "libw4oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


class OracleError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        sigs = {
            "orc_quantize_weight_sym": [_P, _I, _I, _P, _P],
            "orc_unpack_signed": [_P, _I, _I, _I],
            "orc_quantize_act": [_P, _I, _I, _P, _P],
            "orc_matmul_i32": [_P, _P, _I, _I, _I, _P],
            "orc_dequant": [_P, _P, _P, _P, _I, _I, _P],
            "orc_w4a8_linear": [_P, _I, _I, _I, _P, _P, _P, _P],
            "orc_quantize_weight_asym": [_P, _I, _I, _I, _P, _P, _P],
            "orc_quantize_weight_w8": [_P, _I, _I, _P, _P],
            "orc_matmul_w8_i32": [_P, _P, _I, _I, _I, _P],
            "orc_w8a8_linear": [_P, _I, _I, _I, _P, _P, _P, _P],
            "orc_relu": [_P, _I],
            "orc_w4a16_prepack": [_P, _P, _P, _I, _I, _P, _P],
            "orc_w4_prepack_weights": [_P, _I, _I, _P],
            "orc_w4_unprepack_weights": [_P, _I, _I, _P],
            "orc_w4a16_unprepack": [_P, _P, _I, _I, _P, _P, _P],
            "orc_awq_channel_scales": [_P, _I, _I, ctypes.c_int, ctypes.c_int, _P],
            "orc_awq_scale_bf16": [_P, _I, _I, _P, _P],
            "orc_awq_fold_weight": [_P, _I, _I, _P, _P],
            "orc_awq_quantize_act": [_P, _I, _I, _P, _P, _P],
            "orc_w4a8_linear_awq": [_P, _I, _I, _I, _P, _P, _P, _P, _P],
            "orc_dequant_weight": [_P, _P, _P, _I, _I, _I, _P],
            "orc_merge_delta": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P],
            "orc_w4a16_dequant": [_P, _P, _P, _I, _I, _I, _P],
            "orc_w4a16_linear": [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.orc_bf16_rne.argtypes = [ctypes.c_float]
        lib.orc_bf16_rne.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        names = {-1: "non-finite input", -2: "integer range exceeded",
                 -3: "rounding mode is not round-to-nearest", -4: "bad shape"}
        raise OracleError(f"{what}: {names.get(rc, rc)}")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def packed_bytes(K: int) -> int:
    """Bytes of one packed output channel: two codes per byte along K."""
    return (K + 1) // 2


def quantize_weight_sym(W: np.ndarray):
    """W [K, N] fp32 -> (packed uint8 [N, ceil(K/2)], sw fp32 [N])."""
    W = _f32(W)
    K, N = W.shape
    packed = np.zeros((N, packed_bytes(K)), np.uint8)
    sw = np.zeros(N, np.float32)
    _check(_load().orc_quantize_weight_sym(_ptr(W), K, N, _ptr(packed), _ptr(sw)),
           "quantize_weight_sym")
    return packed, sw


def unpack_signed(packed: np.ndarray, K: int) -> np.ndarray:
    """Packed [N, ceil(K/2)] -> int8 codes [N, K] (scalar calls; tiny inputs only)."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    lib = _load()
    out = np.zeros((N, K), np.int8)
    for n in range(N):
        for k in range(K):
            out[n, k] = lib.orc_unpack_signed(_ptr(packed), K, n, k)
    return out


def quantize_act(X: np.ndarray):
    """X [M, K] fp32 -> (Xq int8 [M, K], sx fp32 [M])."""
    X = _f32(X)
    M, K = X.shape
    Xq = np.zeros((M, K), np.int8)
    sx = np.zeros(M, np.float32)
    _check(_load().orc_quantize_act(_ptr(X), M, K, _ptr(Xq), _ptr(sx)), "quantize_act")
    return Xq, sx


def matmul_i32(Xq: np.ndarray, packed: np.ndarray, K: int) -> np.ndarray:
    """acc [M, N] int32 = Xq [M, K] times the unpacked codes (exact)."""
    Xq = np.ascontiguousarray(Xq, np.int8)
    packed = np.ascontiguousarray(packed, np.uint8)
    M = Xq.shape[0]
    N = packed.shape[0]
    assert Xq.shape[1] == K and packed.shape[1] == packed_bytes(K)
    acc = np.zeros((M, N), np.int32)
    _check(_load().orc_matmul_i32(_ptr(Xq), _ptr(packed), M, K, N, _ptr(acc)), "matmul_i32")
    return acc


def dequant(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias=None) -> np.ndarray:
    acc = np.ascontiguousarray(acc, np.int32)
    M, N = acc.shape
    sx, sw = _f32(sx), _f32(sw)
    b = None if bias is None else _f32(bias)
    Y = np.zeros((M, N), np.float32)
    _check(_load().orc_dequant(_ptr(acc), _ptr(sx), _ptr(sw), _ptr(b), M, N, _ptr(Y)),
           "dequant")
    return Y


def w4a8_linear(X: np.ndarray, packed: np.ndarray, sw: np.ndarray, bias=None) -> np.ndarray:
    """Y [M, N] fp32 of the whole W4A8 forward."""
    X = _f32(X)
    M, K = X.shape
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] == packed_bytes(K)
    sw = _f32(sw)
    b = None if bias is None else _f32(bias)
    Y = np.zeros((M, N), np.float32)
    _check(_load().orc_w4a8_linear(_ptr(X), M, K, N, _ptr(packed), _ptr(sw), _ptr(b), _ptr(Y)),
           "w4a8_linear")
    return Y


def relu(Y: np.ndarray) -> np.ndarray:
    """The Dense layer's ReLU on an fp32 output (a copy): y > 0 ? y : +0."""
    out = np.array(Y, dtype=np.float32, copy=True, order="C")
    _check(_load().orc_relu(_ptr(out), out.size), "relu")
    return out


def awq_channel_scales(Xcal: np.ndarray, alpha=(1, 2)) -> np.ndarray:
    """Calibration activations [M, K] -> power-of-two channel scales s [K]."""
    Xcal = _f32(Xcal)
    M, K = Xcal.shape
    s = np.zeros(K, np.float32)
    _check(_load().orc_awq_channel_scales(_ptr(Xcal), M, K, int(alpha[0]), int(alpha[1]),
                                          _ptr(s)), "awq_channel_scales")
    return s


def awq_scale_bf16(Xbf16: np.ndarray, s: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(Xbf16, np.uint16)
    M, K = X.shape
    out = np.zeros_like(X)
    _check(_load().orc_awq_scale_bf16(_ptr(X), M, K, _ptr(_f32(s)), _ptr(out)), "awq_scale_bf16")
    return out


def awq_fold_weight(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    W = _f32(W)
    K, N = W.shape
    out = np.zeros_like(W)
    _check(_load().orc_awq_fold_weight(_ptr(W), K, N, _ptr(_f32(s)), _ptr(out)), "awq_fold")
    return out


def awq_quantize_act(X: np.ndarray, s: np.ndarray):
    X = _f32(X)
    M, K = X.shape
    Xq = np.zeros((M, K), np.int8)
    sx = np.zeros(M, np.float32)
    _check(_load().orc_awq_quantize_act(_ptr(X), M, K, _ptr(_f32(s)), _ptr(Xq), _ptr(sx)),
           "awq_quantize_act")
    return Xq, sx


def w4a8_linear_awq(X: np.ndarray, packed: np.ndarray, sw: np.ndarray, s: np.ndarray,
                    bias=None) -> np.ndarray:
    X = _f32(X)
    M, K = X.shape
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    b = None if bias is None else _f32(bias)
    Y = np.zeros((M, N), np.float32)
    _check(_load().orc_w4a8_linear_awq(_ptr(X), M, K, N, _ptr(packed), _ptr(_f32(sw)),
                                       _ptr(_f32(s)), _ptr(b), _ptr(Y)), "w4a8_linear_awq")
    return Y


def quantize_weight_w8(W: np.ndarray):
    """W [K, N] fp32 -> (Wq int8 [N, K], sw fp32 [N])."""
    W = _f32(W)
    K, N = W.shape
    Wq = np.zeros((N, K), np.int8)
    sw = np.zeros(N, np.float32)
    _check(_load().orc_quantize_weight_w8(_ptr(W), K, N, _ptr(Wq), _ptr(sw)),
           "quantize_weight_w8")
    return Wq, sw


def matmul_w8_i32(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """acc [M, N] int32 = Xq [M, K] times Wq [N, K] transposed (exact)."""
    Xq = np.ascontiguousarray(Xq, np.int8)
    Wq = np.ascontiguousarray(Wq, np.int8)
    M, K = Xq.shape
    N = Wq.shape[0]
    assert Wq.shape[1] == K
    acc = np.zeros((M, N), np.int32)
    _check(_load().orc_matmul_w8_i32(_ptr(Xq), _ptr(Wq), M, K, N, _ptr(acc)), "matmul_w8_i32")
    return acc


def w8a8_linear(X: np.ndarray, Wq: np.ndarray, sw: np.ndarray, bias=None) -> np.ndarray:
    """Y [M, N] fp32 of the whole W8A8 forward."""
    X = _f32(X)
    M, K = X.shape
    Wq = np.ascontiguousarray(Wq, np.int8)
    N = Wq.shape[0]
    assert Wq.shape[1] == K
    sw = _f32(sw)
    b = None if bias is None else _f32(bias)
    Y = np.zeros((M, N), np.float32)
    _check(_load().orc_w8a8_linear(_ptr(X), M, K, N, _ptr(Wq), _ptr(sw), _ptr(b), _ptr(Y)),
           "w8a8_linear")
    return Y


def quantize_weight_asym(W: np.ndarray, group: int):
    """W [K, N] fp32 -> (packed [N, ceil(K/2)], scales [N, K/g], zeros [N, K/g])."""
    W = _f32(W)
    K, N = W.shape
    G = K // group if group > 0 else 0
    packed = np.zeros((N, packed_bytes(K)), np.uint8)
    scales = np.zeros((N, max(G, 1)), np.float32)
    zeros = np.zeros((N, max(G, 1)), np.float32)
    _check(_load().orc_quantize_weight_asym(_ptr(W), K, N, group, _ptr(packed),
                                            _ptr(scales), _ptr(zeros)), "quantize_weight_asym")
    return packed, scales, zeros


def dequant_weight(packed, scales, zeros, K: int, group: int = 0) -> np.ndarray:
    """W [K, N] fp32 from packed codes: symmetric when zeros is None."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    W = np.zeros((K, N), np.float32)
    z = None if zeros is None else _f32(zeros)
    _check(_load().orc_dequant_weight(_ptr(packed), _ptr(_f32(scales)), _ptr(z), K, N, group,
                                      _ptr(W)), "dequant_weight")
    return W


def merge_delta(packed, scales, zeros, K: int, delta: np.ndarray, group: int = 0):
    """Requantize dequant(packed) + delta [K, N]; returns (packed, scales, zeros)."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    delta = _f32(delta)
    assert delta.shape == (K, N)
    po = np.zeros_like(packed)
    so = np.zeros_like(_f32(scales))
    zo = None if zeros is None else np.zeros_like(_f32(zeros))
    _check(_load().orc_merge_delta(_ptr(packed), _ptr(_f32(scales)),
                                   _ptr(None if zeros is None else _f32(zeros)), K, N, group,
                                   _ptr(delta), _ptr(po), _ptr(so), _ptr(zo)), "merge_delta")
    return po, so, zo


def w4_prepack_weights(packed, K: int) -> np.ndarray:
    """Packed int4 codes [N, K/2] -> the shuffled tiles uint8 [N16/16, K/128, 16, 64]."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    wpp = np.zeros(((N + 15) // 16, K // 128, 16, 64), np.uint8)
    _check(_load().orc_w4_prepack_weights(_ptr(packed), K, N, _ptr(wpp)), "w4_prepack_weights")
    return wpp


def w4_unprepack_weights(wpp, K: int, N: int) -> np.ndarray:
    packed = np.zeros((N, K // 2), np.uint8)
    _check(_load().orc_w4_unprepack_weights(_ptr(np.ascontiguousarray(wpp, np.uint8)), K, N,
                                            _ptr(packed)), "w4_unprepack_weights")
    return packed


def w4a16_prepack(packed, scales, zeros, K: int):
    """Canonical W4A16 tensors -> (wpp uint8 [N16/16, K/128, 16, 64], szpp fp32 [N16/16, K/256, 16, 4])."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    nb = (N + 15) // 16
    wpp = np.zeros((nb, K // 128, 16, 64), np.uint8)
    szpp = np.zeros((nb, K // 256, 16, 4), np.float32)
    _check(_load().orc_w4a16_prepack(_ptr(packed), _ptr(_f32(scales)), _ptr(_f32(zeros)), K, N,
                                     _ptr(wpp), _ptr(szpp)), "w4a16_prepack")
    return wpp, szpp


def w4a16_unprepack(wpp, szpp, K: int, N: int):
    """Inverse of w4a16_prepack on the first N channels."""
    packed = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 128), np.float32)
    zeros = np.zeros((N, K // 128), np.float32)
    _check(_load().orc_w4a16_unprepack(_ptr(np.ascontiguousarray(wpp, np.uint8)),
                                       _ptr(_f32(szpp)), K, N, _ptr(packed), _ptr(scales),
                                       _ptr(zeros)), "w4a16_unprepack")
    return packed, scales, zeros


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round half to even (scalar calls)."""
    lib = _load()
    flat = _f32(x).ravel()
    out = np.array([lib.orc_bf16_rne(ctypes.c_float(float(v))) for v in flat], np.uint16)
    return out.reshape(np.shape(x))


def w4a16_dequant(packed, scales, zeros, K: int, group: int) -> np.ndarray:
    """bf16 bit patterns [K, N] of the dequantized weights."""
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    scales, zeros = _f32(scales), _f32(zeros)
    Wd = np.zeros((K, N), np.uint16)
    _check(_load().orc_w4a16_dequant(_ptr(packed), _ptr(scales), _ptr(zeros), K, N, group,
                                     _ptr(Wd)), "w4a16_dequant")
    return Wd


def w4a16_linear(Xbf16: np.ndarray, packed, scales, zeros, group: int):
    """Xbf16: bf16 bit patterns uint16 [M, K].  Returns (y fp64 [M, N], sum|x*w'| fp64)."""
    X = np.ascontiguousarray(Xbf16, np.uint16)
    M, K = X.shape
    packed = np.ascontiguousarray(packed, np.uint8)
    N = packed.shape[0]
    scales, zeros = _f32(scales), _f32(zeros)
    Y = np.zeros((M, N), np.float64)
    A = np.zeros((M, N), np.float64)
    _check(_load().orc_w4a16_linear(_ptr(X), M, K, N, _ptr(packed), _ptr(scales), _ptr(zeros),
                                    group, _ptr(Y), _ptr(A)), "w4a16_linear")
    return Y, A


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)
