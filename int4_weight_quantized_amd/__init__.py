"""Python binding of libw4.so, the MI355X (gfx950) INT4 weight-quantized linear layer.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/w4.h``.  PyTorch provides the
device memory (tensors) and the stream (the current HIP stream).  The
functions carry the C names:

* ``w4_quantize_weight``  -- symmetric per-channel int4 (``scheme="sym"``) or
  asymmetric group-wise int4 (``scheme="asym"``) weights, packed two per byte;
* ``w4_dequantize_weight`` -- packed codes back to fp32 weights;
* ``w4_merge_delta``      -- the lossy LoRA merge (dequantize, add, requantize);
* ``a8_quantize_act``     -- per-row dynamic int8 activations;
* ``w4a8_linear``         -- the W4A8 forward from fp32 activations;
* ``w4a8_linear_act``     -- the same with a fused activation (ReLU);
* ``w4a8_linear_noalloc`` -- ``w4a8_linear`` with the library's fixed device
  scratch instead of a workspace (for callers that cannot allocate);
* ``w4a8_linear_q``       -- the W4A8 forward from int8 activations;
* ``w4a8_matmul_i32``     -- the exact int32 accumulators alone;
* ``w8_quantize_weight``  -- symmetric per-channel int8 weights (W8A8);
* ``w8a8_linear``         -- the W8A8 forward from fp32 activations;
* ``w8a8_linear_act``     -- the same with a fused activation (ReLU);
* ``w8a8_matmul_i32``     -- its exact int32 accumulators alone;
* ``w4a16_linear``        -- the weight-only forward with bf16 activations;
* ``w4a16_prepack``, ``w4a16_unprepack``, ``w4a16_linear_prepacked`` -- the
  GPU-shuffled W4A16 layout, its inverse and the forward on it;
* ``w4_prepack_weights``, ``w4_unprepack_weights``, ``w4a8_linear_prepacked``
  -- the same tile layout for the W4A8 int4 codes and the forward on it;
* ``awq_channel_scales``, ``awq_fold_weight``, ``awq_quantize_act``,
  ``awq_scale_act_bf16``, ``w4a8_linear_awq`` -- AWQ-style activation-aware
  channel scaling (power-of-two scales from calibration activations).

There is no CPU fallback: without the built library (``build.py``) or
without a GPU every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# W4_LIB may name another build of the same sources (the host-sanitizer build
# of build_hostsan.py).
LIB_PATH = os.environ.get("W4_LIB") or os.path.join(_HERE, "libw4.so")

W4_OK = 0
W4_SYM_PER_CHANNEL = 0
W4_ASYM_GROUP = 1
W4_MAX_K = 131071
W4_ACT_NONE = 0
W4_ACT_RELU = 1
W4_NOALLOC_SCRATCH_BYTES = 16777216 + 65536
_ACTS = {None: W4_ACT_NONE, "none": W4_ACT_NONE, "relu": W4_ACT_RELU}

_P = ctypes.c_void_p
_I = ctypes.c_int64
_Z = ctypes.c_size_t
_lib = None


class W4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {w4_status_string(status)} (status {status})")


def lib():
    """The loaded libw4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python int4_weight_quantized_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "w4_quantize_weight": ([_P, _I, _I, ctypes.c_int, _I, _P, _P, _P, _P], ctypes.c_int),
            "a8_quantize_act": ([_P, _I, _I, _P, _P, _P], ctypes.c_int),
            "w4a8_workspace_bytes": ([_I, _I, _I], _Z),
            "w4a8_linear": ([_P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
            "w4a8_linear_noalloc": ([_P, _I, _I, _I, _P, _P, _P, _P, _P], ctypes.c_int),
            "w4a8_linear_act": ([_P, _I, _I, _I, _P, _P, _P, ctypes.c_int, _P, _P, _Z, _P],
                                ctypes.c_int),
            "w8a8_linear_act": ([_P, _I, _I, _I, _P, _P, _P, ctypes.c_int, _P, _P, _Z, _P],
                                ctypes.c_int),
            "w4a8_linear_q": ([_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _Z, _P], ctypes.c_int),
            "w4a8_matmul_i32": ([_P, _P, _I, _I, _I, _P, _P, _Z, _P], ctypes.c_int),
            "w4a16_linear": ([_P, _I, _I, _I, _P, _P, _P, _I, _P, _P], ctypes.c_int),
            "w8_quantize_weight": ([_P, _I, _I, _P, _P, _P], ctypes.c_int),
            "w4a16_prepacked_weight_bytes": ([_I, _I], ctypes.c_int64),
            "w4_prepacked_weight_bytes": ([_I, _I], ctypes.c_int64),
            "w4_prepack_weights": ([_P, _I, _I, _P, _P], ctypes.c_int),
            "w4_unprepack_weights": ([_P, _I, _I, _P, _P], ctypes.c_int),
            "w4a8_linear_prepacked": ([_P, _I, _I, _I, _P, _P, _P, ctypes.c_int, _P, _P, _Z, _P],
                                      ctypes.c_int),
            "w4a16_prepacked_table_floats": ([_I, _I], ctypes.c_int64),
            "w4a16_prepack": ([_P, _P, _P, _I, _I, _I, _P, _P, _P], ctypes.c_int),
            "w4a16_unprepack": ([_P, _P, _I, _I, _I, _P, _P, _P, _P], ctypes.c_int),
            "w4a16_linear_prepacked": ([_P, _I, _I, _I, _P, _P, _P, _P], ctypes.c_int),
            "awq_channel_scales": ([_P, _I, _I, ctypes.c_int, ctypes.c_int, _P, _P], ctypes.c_int),
            "awq_fold_weight": ([_P, _I, _I, _P, _P, _P], ctypes.c_int),
            "awq_quantize_act": ([_P, _I, _I, _P, _P, _P, _P], ctypes.c_int),
            "awq_scale_act_bf16": ([_P, _I, _I, _P, _P, _P], ctypes.c_int),
            "w4a8_linear_awq": ([_P, _I, _I, _I, _P, _P, _P, _P, ctypes.c_int, _P, _P, _Z, _P],
                                ctypes.c_int),
            "w4_dequantize_weight": ([_P, _P, _P, _I, _I, ctypes.c_int, _I, _P, _P], ctypes.c_int),
            "w4_merge_delta": ([_P, _P, _P, _I, _I, ctypes.c_int, _I, _P, _P, _P, _P, _P, _P],
                               ctypes.c_int),
            "w8a8_workspace_bytes": ([_I, _I, _I], _Z),
            "w8a8_linear": ([_P, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P], ctypes.c_int),
            "w8a8_matmul_i32": ([_P, _P, _I, _I, _I, _P, _P, _Z, _P], ctypes.c_int),
            "w4_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "w4_last_path": ([], ctypes.c_char_p),
            "w4_last_kernel": ([], ctypes.c_char_p),
            "w4_probe_empty": ([_I, _P], ctypes.c_int),
            "w4_probe_read": ([_P, _I, _P, _P], ctypes.c_int),
            "w4_probe_write": ([_P, _I, ctypes.c_uint32, _P], ctypes.c_int),
            "w4_probe_mfma": ([_I, ctypes.c_int, _P, _P, _P, _P], ctypes.c_int),
            "w4_time_next_kernel": ([_P, _P], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def w4_status_string(status: int) -> str:
    return lib().w4_status_string(int(status)).decode()


def w4_last_path() -> str:
    """Kernel variant of the last call's main product (e.g. "gemv_dot4")."""
    return lib().w4_last_path().decode()


def w4_last_kernel() -> str:
    """Device symbol (mangled) of the last successful call's main kernel."""
    return lib().w4_last_kernel().decode()


def w4_probe_empty(blocks: int, stream=None) -> None:
    """Launch an empty kernel of `blocks` workgroups (a measurement helper)."""
    _check("w4_probe_empty", lib().w4_probe_empty(int(blocks), _stream(stream)))


def w4_probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of `src` once (a measurement helper); sink: 64 int32."""
    dev = src.device
    _check("w4_probe_read", lib().w4_probe_read(_dev(src, "src", src.dtype), src.numel() *
                                                src.element_size(),
                                                _dev(sink, "sink", torch.int32, (64,), dev),
                                                _stream(stream)))


def w4_probe_write(dst: torch.Tensor, value: int = 0, stream=None) -> None:
    """Write every byte of `dst` once, each 32-bit word = `value` (a measurement helper)."""
    _check("w4_probe_write", lib().w4_probe_write(_dev(dst, "dst", dst.dtype),
                                                  dst.numel() * dst.element_size(),
                                                  int(value) & 0xFFFFFFFF, _stream(stream)))


def w4_probe_mfma(blocks: int, iters: int, times: torch.Tensor, sink: torch.Tensor,
                  ops: torch.Tensor = None, stream=None) -> None:
    """Int8 MFMA clock / rate probe (a measurement helper); times: int64
    [blocks, 4]; ops: int32 [blocks * 512 * 32] operands, or None for constant ones."""
    dev = times.device
    _check("w4_probe_mfma", lib().w4_probe_mfma(int(blocks), int(iters),
                                                _opt(ops, "ops", torch.int32,
                                                     (int(blocks) * 512 * 32,), dev),
                                                _dev(times, "times", torch.int64, (blocks, 4)),
                                                _dev(sink, "sink", torch.int32, (64,), dev),
                                                _stream(stream)))


def w4_time_next_kernel(start_event: int | None, stop_event: int | None) -> None:
    """Attach raw hipEvent_t handles to the next product kernel launched
    from this thread (recorded when it starts and when it completes)."""
    _check("w4_time_next_kernel", lib().w4_time_next_kernel(start_event, stop_event))


def w4a8_workspace_bytes(M: int, K: int, N: int) -> int:
    return int(lib().w4a8_workspace_bytes(M, K, N))


# ------------------------------------------------------------------ helpers
def _dev(t: torch.Tensor, name: str, dtype, shape=None, device=None) -> int:
    """Device pointer of t after checking what the C side cannot: the kernels
    take raw pointers and trust the sizes, so every tensor is checked against
    the exact shape the call implies (and against the device of the call's
    first operand)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's operands on {device}")
    return t.data_ptr()


def _opt(t, name, dtype, shape=None, device=None):
    return None if t is None else _dev(t, name, dtype, shape, device)


_HALF_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _half(t: torch.Tensor, name: str, shape=None, device=None) -> int:
    """bf16 activations, or their 16-bit patterns as int16 / uint16."""
    if not isinstance(t, torch.Tensor) or t.dtype not in _HALF_DTYPES:
        raise TypeError(f"{name} must be a bfloat16 (or int16 / uint16 bit-pattern) tensor")
    return _dev(t, name, t.dtype, shape, device)


def _matrix(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return t.shape


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, rc: int):
    if rc != W4_OK:
        raise W4Error(fn, rc)


def _workspace(M, K, N, device, workspace):
    need = w4a8_workspace_bytes(M, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


# ------------------------------------------------------------------ calls
def w4_quantize_weight(W: torch.Tensor, scheme: str = "sym", group_size: int = 0,
                       packed=None, scales=None, zeros=None, stream=None):
    """W [K, N] fp32 -> (packed uint8 [N, ceil(K/2)], scales, zeros).

    ``scheme="sym"``: scales [N], zeros None.  ``scheme="asym"``: scales and
    zeros [N, K/group_size]."""
    K, N = _matrix(W, "W")
    sch = {"sym": W4_SYM_PER_CHANNEL, "asym": W4_ASYM_GROUP}.get(scheme, -1)
    dev = W.device
    if packed is None:
        packed = torch.empty((N, (K + 1) // 2), dtype=torch.uint8, device=dev)
    tshape = None
    if sch == W4_ASYM_GROUP and group_size > 0:
        tshape = (N, K // group_size)
        if scales is None:
            scales = torch.empty(tshape, dtype=torch.float32, device=dev)
        if zeros is None:
            zeros = torch.empty(tshape, dtype=torch.float32, device=dev)
    else:
        tshape = (N,)
        if scales is None:
            scales = torch.empty(tshape, dtype=torch.float32, device=dev)
    rc = lib().w4_quantize_weight(_dev(W, "W", torch.float32), K, N, sch, group_size,
                                  _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                                  _dev(scales, "scales", torch.float32, tshape, dev),
                                  _opt(zeros, "zeros", torch.float32, tshape, dev), _stream(stream))
    _check("w4_quantize_weight", rc)
    return packed, scales, zeros


def _scheme(scheme: str) -> int:
    return {"sym": W4_SYM_PER_CHANNEL, "asym": W4_ASYM_GROUP}.get(scheme, -1)


def _table_shape(scheme: str, N: int, K: int, group_size: int):
    """Shape of the scale / zero-point tables, or None where the C side
    rejects the arguments anyway (before launching anything)."""
    if scheme == "sym":
        return (N,)
    if group_size > 0 and K % group_size == 0:
        return (N, K // group_size)
    return None


def w4_dequantize_weight(packed: torch.Tensor, scales: torch.Tensor, zeros, K: int,
                         scheme: str = "sym", group_size: int = 0, W=None, stream=None):
    """packed [N, ceil(K/2)] (+ scales, zeros) -> W [K, N] fp32."""
    N = _matrix(packed, "packed")[0]
    dev = packed.device
    ts = _table_shape(scheme, N, K, group_size)
    if W is None:
        W = torch.empty((K, N), dtype=torch.float32, device=dev)
    rc = lib().w4_dequantize_weight(_dev(packed, "packed", torch.uint8, (N, (K + 1) // 2)),
                                    _dev(scales, "scales", torch.float32, ts, dev),
                                    _opt(zeros, "zeros", torch.float32, ts, dev), K, N,
                                    _scheme(scheme), group_size,
                                    _dev(W, "W", torch.float32, (K, N), dev), _stream(stream))
    _check("w4_dequantize_weight", rc)
    return W


def w4_merge_delta(packed: torch.Tensor, scales: torch.Tensor, zeros, delta: torch.Tensor,
                   scheme: str = "sym", group_size: int = 0, in_place: bool = False,
                   work=None, stream=None):
    """Requantize dequant(packed) + delta [K, N]; returns (packed, scales, zeros),
    new tensors unless in_place (then the inputs are overwritten)."""
    K, N = _matrix(delta, "delta")
    dev = delta.device
    ts = _table_shape(scheme, N, K, group_size)
    if in_place:
        po, so, zo = packed, scales, zeros
    else:
        po, so = torch.empty_like(packed), torch.empty_like(scales)
        zo = None if zeros is None else torch.empty_like(zeros)
    if work is None:
        work = torch.empty((K, N), dtype=torch.float32, device=dev)
    pshape = (N, (K + 1) // 2)
    rc = lib().w4_merge_delta(_dev(packed, "packed", torch.uint8, pshape, dev),
                              _dev(scales, "scales", torch.float32, ts, dev),
                              _opt(zeros, "zeros", torch.float32, ts, dev), K, N, _scheme(scheme),
                              group_size, _dev(delta, "delta", torch.float32),
                              _dev(po, "packed_out", torch.uint8, pshape, dev),
                              _dev(so, "scales_out", torch.float32, ts, dev),
                              _opt(zo, "zeros_out", torch.float32, ts, dev),
                              _dev(work, "work", torch.float32, (K, N), dev), _stream(stream))
    _check("w4_merge_delta", rc)
    return po, so, zo


def a8_quantize_act(X: torch.Tensor, Xq=None, sx=None, stream=None):
    """X [M, K] fp32 -> (Xq int8 [M, K], sx fp32 [M])."""
    M, K = _matrix(X, "X")
    dev = X.device
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=dev)
    rc = lib().a8_quantize_act(_dev(X, "X", torch.float32), M, K,
                               _dev(Xq, "Xq", torch.int8, (M, K), dev),
                               _dev(sx, "sx", torch.float32, (M,), dev), _stream(stream))
    _check("a8_quantize_act", rc)
    return Xq, sx


def w4a8_linear(X: torch.Tensor, packed: torch.Tensor, sw: torch.Tensor, bias=None, Y=None,
                workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] fp32 = dequant(quant(X) . unpack(packed)) (+ bias)."""
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    workspace, need = _workspace(M, K, N, X.device, workspace)
    rc = lib().w4a8_linear(_dev(X, "X", torch.float32), M, K, N,
                           _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                           _dev(sw, "sw", torch.float32, (N,), dev),
                           _opt(bias, "bias", torch.float32, (N,), dev),
                           _dev(Y, "Y", torch.float32, (M, N), dev),
                           _dev(workspace, "workspace", torch.uint8, None, dev), workspace.numel(),
                           _stream(stream))
    _check("w4a8_linear", rc)
    return Y


def w4a8_linear_noalloc(X: torch.Tensor, packed: torch.Tensor, sw: torch.Tensor,
                        Y: torch.Tensor, bias=None, stream=None) -> torch.Tensor:
    """w4a8_linear without a workspace: the library's fixed device scratch
    (W4_NOALLOC_SCRATCH_BYTES per GPU) serves instead, and nothing is allocated,
    so the output Y [M, N] fp32 must be passed in.  Calls overlapping on one GPU race."""
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    dev = X.device
    rc = lib().w4a8_linear_noalloc(_dev(X, "X", torch.float32), M, K, N,
                                   _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                                   _dev(sw, "sw", torch.float32, (N,), dev),
                                   _opt(bias, "bias", torch.float32, (N,), dev),
                                   _dev(Y, "Y", torch.float32, (M, N), dev), _stream(stream))
    _check("w4a8_linear_noalloc", rc)
    return Y


def _act(activation) -> int:
    if activation not in _ACTS:
        raise ValueError(f"unknown activation {activation!r} (None or 'relu')")
    return _ACTS[activation]


def w4a8_linear_act(X: torch.Tensor, packed: torch.Tensor, sw: torch.Tensor, bias=None,
                    activation="relu", Y=None, workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] fp32 = act(dequant(quant(X) . unpack(packed)) (+ bias)), one fused epilogue."""
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    workspace, need = _workspace(M, K, N, X.device, workspace)
    rc = lib().w4a8_linear_act(_dev(X, "X", torch.float32), M, K, N,
                               _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                               _dev(sw, "sw", torch.float32, (N,), dev),
                               _opt(bias, "bias", torch.float32, (N,), dev), _act(activation),
                               _dev(Y, "Y", torch.float32, (M, N), dev),
                               _dev(workspace, "workspace", torch.uint8, None, dev),
                               workspace.numel(), _stream(stream))
    _check("w4a8_linear_act", rc)
    return Y


def w4a8_linear_q(Xq: torch.Tensor, sx: torch.Tensor, packed: torch.Tensor, sw: torch.Tensor,
                  bias=None, Y=None, workspace=None, stream=None) -> torch.Tensor:
    M, K = _matrix(Xq, "Xq")
    N = _matrix(packed, "packed")[0]
    dev = Xq.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    workspace, need = _workspace(M, K, N, Xq.device, workspace)
    rc = lib().w4a8_linear_q(_dev(Xq, "Xq", torch.int8), _dev(sx, "sx", torch.float32, (M,), dev),
                             _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                             _dev(sw, "sw", torch.float32, (N,), dev),
                             _opt(bias, "bias", torch.float32, (N,), dev), M, K, N,
                             _dev(Y, "Y", torch.float32, (M, N), dev),
                             _dev(workspace, "workspace", torch.uint8, None, dev),
                             workspace.numel(), _stream(stream))
    _check("w4a8_linear_q", rc)
    return Y


def w4a8_matmul_i32(Xq: torch.Tensor, packed: torch.Tensor, acc=None, workspace=None,
                    stream=None) -> torch.Tensor:
    M, K = _matrix(Xq, "Xq")
    N = _matrix(packed, "packed")[0]
    dev = Xq.device
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    workspace, need = _workspace(M, K, N, Xq.device, workspace)
    rc = lib().w4a8_matmul_i32(_dev(Xq, "Xq", torch.int8),
                               _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev), M, K, N,
                               _dev(acc, "acc", torch.int32, (M, N), dev),
                               _dev(workspace, "workspace", torch.uint8, None, dev),
                               workspace.numel(), _stream(stream))
    _check("w4a8_matmul_i32", rc)
    return acc


def w8_quantize_weight(W: torch.Tensor, Wq=None, sw=None, stream=None):
    """W [K, N] fp32 -> (Wq int8 [N, K], sw fp32 [N])."""
    K, N = _matrix(W, "W")
    dev = W.device
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if sw is None:
        sw = torch.empty((N,), dtype=torch.float32, device=W.device)
    rc = lib().w8_quantize_weight(_dev(W, "W", torch.float32), K, N,
                                  _dev(Wq, "Wq", torch.int8, (N, K), dev),
                                  _dev(sw, "sw", torch.float32, (N,), dev), _stream(stream))
    _check("w8_quantize_weight", rc)
    return Wq, sw


def w8a8_linear(X: torch.Tensor, Wq: torch.Tensor, sw: torch.Tensor, bias=None, Y=None,
                workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] fp32 = dequant(quant(X) . Wq^T) (+ bias)."""
    M, K = _matrix(X, "X")
    N = _matrix(Wq, "Wq")[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    workspace, need = _workspace(M, K, N, X.device, workspace)
    rc = lib().w8a8_linear(_dev(X, "X", torch.float32), M, K, N,
                           _dev(Wq, "Wq", torch.int8, (N, K), dev),
                           _dev(sw, "sw", torch.float32, (N,), dev),
                           _opt(bias, "bias", torch.float32, (N,), dev),
                           _dev(Y, "Y", torch.float32, (M, N), dev),
                           _dev(workspace, "workspace", torch.uint8, None, dev), workspace.numel(),
                           _stream(stream))
    _check("w8a8_linear", rc)
    return Y


def w8a8_linear_act(X: torch.Tensor, Wq: torch.Tensor, sw: torch.Tensor, bias=None,
                    activation="relu", Y=None, workspace=None, stream=None) -> torch.Tensor:
    """Y [M, N] fp32 = act(dequant(quant(X) . Wq^T) (+ bias)), one fused epilogue."""
    M, K = _matrix(X, "X")
    N = _matrix(Wq, "Wq")[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    workspace, need = _workspace(M, K, N, X.device, workspace)
    rc = lib().w8a8_linear_act(_dev(X, "X", torch.float32), M, K, N,
                               _dev(Wq, "Wq", torch.int8, (N, K), dev),
                               _dev(sw, "sw", torch.float32, (N,), dev),
                               _opt(bias, "bias", torch.float32, (N,), dev), _act(activation),
                               _dev(Y, "Y", torch.float32, (M, N), dev),
                               _dev(workspace, "workspace", torch.uint8, None, dev),
                               workspace.numel(), _stream(stream))
    _check("w8a8_linear_act", rc)
    return Y


def w8a8_matmul_i32(Xq: torch.Tensor, Wq: torch.Tensor, acc=None, workspace=None,
                    stream=None) -> torch.Tensor:
    M, K = _matrix(Xq, "Xq")
    N = _matrix(Wq, "Wq")[0]
    dev = Xq.device
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=Xq.device)
    workspace, need = _workspace(M, K, N, Xq.device, workspace)
    rc = lib().w8a8_matmul_i32(_dev(Xq, "Xq", torch.int8), _dev(Wq, "Wq", torch.int8, (N, K), dev),
                               M, K, N, _dev(acc, "acc", torch.int32, (M, N), dev),
                               _dev(workspace, "workspace", torch.uint8, None, dev),
                               workspace.numel(), _stream(stream))
    _check("w8a8_matmul_i32", rc)
    return acc


def awq_channel_scales(Xcal: torch.Tensor, alpha=(1, 2), s=None, stream=None) -> torch.Tensor:
    """Calibration activations [M, K] fp32 -> power-of-two channel scales s [K]."""
    M, K = _matrix(Xcal, "Xcal")
    if s is None:
        s = torch.empty((K,), dtype=torch.float32, device=Xcal.device)
    rc = lib().awq_channel_scales(_dev(Xcal, "Xcal", torch.float32), M, K, int(alpha[0]),
                                  int(alpha[1]), _dev(s, "s", torch.float32, (K,), Xcal.device),
                                  _stream(stream))
    _check("awq_channel_scales", rc)
    return s


def awq_fold_weight(W: torch.Tensor, s: torch.Tensor, W_out=None, stream=None) -> torch.Tensor:
    """W [K, N] -> W diag(s) (W_out may be W)."""
    K, N = _matrix(W, "W")
    dev = W.device
    if W_out is None:
        W_out = torch.empty_like(W)
    rc = lib().awq_fold_weight(_dev(W, "W", torch.float32), K, N,
                               _dev(s, "s", torch.float32, (K,), dev),
                               _dev(W_out, "W_out", torch.float32, (K, N), dev), _stream(stream))
    _check("awq_fold_weight", rc)
    return W_out


def awq_quantize_act(X: torch.Tensor, s: torch.Tensor, Xq=None, sx=None, stream=None):
    """(Xq, sx) of X / s (per column)."""
    M, K = _matrix(X, "X")
    dev = X.device
    if Xq is None:
        Xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    if sx is None:
        sx = torch.empty((M,), dtype=torch.float32, device=dev)
    rc = lib().awq_quantize_act(_dev(X, "X", torch.float32), M, K,
                                _dev(s, "s", torch.float32, (K,), dev),
                                _dev(Xq, "Xq", torch.int8, (M, K), dev),
                                _dev(sx, "sx", torch.float32, (M,), dev), _stream(stream))
    _check("awq_quantize_act", rc)
    return Xq, sx


def awq_scale_act_bf16(X_bf16: torch.Tensor, s: torch.Tensor, X_out=None, stream=None):
    """bf16 (or int16 bit-pattern) activations divided by s per column."""
    M, K = _matrix(X_bf16, "X_bf16")
    dev = X_bf16.device
    if X_out is None:
        X_out = torch.empty_like(X_bf16)
    rc = lib().awq_scale_act_bf16(_half(X_bf16, "X_bf16"), M, K,
                                  _dev(s, "s", torch.float32, (K,), dev),
                                  _half(X_out, "X_out", (M, K), dev), _stream(stream))
    _check("awq_scale_act_bf16", rc)
    return X_out


def w4a8_linear_awq(X: torch.Tensor, packed: torch.Tensor, sw: torch.Tensor, s: torch.Tensor,
                    bias=None, activation=None, Y=None, workspace=None,
                    stream=None) -> torch.Tensor:
    """Y = act(dequant(quant(X / s) . unpack(packed)) (+ bias)); packed, sw from W diag(s)."""
    M, K = _matrix(X, "X")
    N = _matrix(packed, "packed")[0]
    dev = X.device
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    workspace, need = _workspace(M, K, N, X.device, workspace)
    rc = lib().w4a8_linear_awq(_dev(X, "X", torch.float32), M, K, N,
                               _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                               _dev(sw, "sw", torch.float32, (N,), dev),
                               _dev(s, "s", torch.float32, (K,), dev),
                               _opt(bias, "bias", torch.float32, (N,), dev), _act(activation),
                               _dev(Y, "Y", torch.float32, (M, N), dev),
                               _dev(workspace, "workspace", torch.uint8, None, dev),
                               workspace.numel(), _stream(stream))
    _check("w4a8_linear_awq", rc)
    return Y


def w4_prepack_weights(packed: torch.Tensor, stream=None) -> torch.Tensor:
    """Packed int4 codes [N, K/2] -> the shuffled tiles (uint8, flat)."""
    N, KB = _matrix(packed, "packed")
    K = 2 * KB
    nb = int(lib().w4_prepacked_weight_bytes(K, N))
    if nb == 0:
        raise ValueError("the shuffled layout needs K % 128 == 0")
    wpp = torch.empty((nb,), dtype=torch.uint8, device=packed.device)
    rc = lib().w4_prepack_weights(_dev(packed, "packed", torch.uint8), K, N,
                                  _dev(wpp, "wpp", torch.uint8), _stream(stream))
    _check("w4_prepack_weights", rc)
    return wpp


def w4_unprepack_weights(wpp: torch.Tensor, K: int, N: int, stream=None) -> torch.Tensor:
    nb = int(lib().w4_prepacked_weight_bytes(K, N))
    if nb == 0:
        raise ValueError("the shuffled layout needs K % 128 == 0")
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=wpp.device)
    rc = lib().w4_unprepack_weights(_dev(wpp, "wpp", torch.uint8, (nb,)), K, N,
                                    _dev(packed, "packed", torch.uint8), _stream(stream))
    _check("w4_unprepack_weights", rc)
    return packed


def w4a8_linear_prepacked(X: torch.Tensor, wpp: torch.Tensor, sw: torch.Tensor, bias=None,
                          activation=None, Y=None, workspace=None, stream=None) -> torch.Tensor:
    """The W4A8 forward on the shuffled int4 tiles; N = sw.numel()."""
    M, K = _matrix(X, "X")
    N = sw.shape[0]
    dev = X.device
    nb = int(lib().w4_prepacked_weight_bytes(K, N))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    workspace, need = _workspace(M, K, N, dev, workspace)
    rc = lib().w4a8_linear_prepacked(_dev(X, "X", torch.float32), M, K, N,
                                     _dev(wpp, "wpp", torch.uint8, (nb,) if nb else None, dev),
                                     _dev(sw, "sw", torch.float32, (N,), dev),
                                     _opt(bias, "bias", torch.float32, (N,), dev), _act(activation),
                                     _dev(Y, "Y", torch.float32, (M, N), dev),
                                     _dev(workspace, "workspace", torch.uint8, None, dev),
                                     workspace.numel(), _stream(stream))
    _check("w4a8_linear_prepacked", rc)
    return Y


def w4a16_prepack(packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                  group_size: int = 128, stream=None):
    """Canonical W4A16 tensors -> (wpp uint8, szpp fp32), the GPU-shuffled layout."""
    N, KB = _matrix(packed, "packed")
    K = 2 * KB
    dev = packed.device
    nw = int(lib().w4a16_prepacked_weight_bytes(K, N))
    nt = int(lib().w4a16_prepacked_table_floats(K, N))
    if nw == 0 or group_size != 128:
        raise ValueError("the shuffled layout needs group_size 128 and K % 512 == 0")
    wpp = torch.empty((nw,), dtype=torch.uint8, device=dev)
    szpp = torch.empty((nt,), dtype=torch.float32, device=dev)
    rc = lib().w4a16_prepack(_dev(packed, "packed", torch.uint8),
                             _dev(scales, "scales", torch.float32, (N, K // 128), dev),
                             _dev(zeros, "zeros", torch.float32, (N, K // 128), dev), K, N,
                             group_size, _dev(wpp, "wpp", torch.uint8),
                             _dev(szpp, "szpp", torch.float32), _stream(stream))
    _check("w4a16_prepack", rc)
    return wpp, szpp


def w4a16_unprepack(wpp: torch.Tensor, szpp: torch.Tensor, K: int, N: int,
                    group_size: int = 128, stream=None):
    """(wpp, szpp) -> canonical (packed [N, K/2], scales, zeros [N, K/128])."""
    dev = wpp.device
    nw = int(lib().w4a16_prepacked_weight_bytes(K, N))
    nt = int(lib().w4a16_prepacked_table_floats(K, N))
    if nw == 0 or group_size != 128:
        raise ValueError("the shuffled layout needs group_size 128 and K % 512 == 0")
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 128), dtype=torch.float32, device=dev)
    zeros = torch.empty((N, K // 128), dtype=torch.float32, device=dev)
    rc = lib().w4a16_unprepack(_dev(wpp, "wpp", torch.uint8, (nw,)),
                               _dev(szpp, "szpp", torch.float32, (nt,), dev), K, N, group_size,
                               _dev(packed, "packed", torch.uint8),
                               _dev(scales, "scales", torch.float32),
                               _dev(zeros, "zeros", torch.float32), _stream(stream))
    _check("w4a16_unprepack", rc)
    return packed, scales, zeros


def w4a16_linear_prepacked(X_bf16: torch.Tensor, wpp: torch.Tensor, szpp: torch.Tensor, N: int,
                           Y=None, stream=None) -> torch.Tensor:
    """The W4A16 forward on the shuffled layout; X_bf16 [M, K] bf16 / 16-bit patterns."""
    M, K = _matrix(X_bf16, "X_bf16")
    dev = X_bf16.device
    nw = int(lib().w4a16_prepacked_weight_bytes(K, N))
    nt = int(lib().w4a16_prepacked_table_floats(K, N))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    rc = lib().w4a16_linear_prepacked(_half(X_bf16, "X_bf16"), M, K, N,
                                      _dev(wpp, "wpp", torch.uint8, (nw,) if nw else None, dev),
                                      _dev(szpp, "szpp", torch.float32, (nt,) if nt else None, dev),
                                      _dev(Y, "Y", torch.float32, (M, N), dev), _stream(stream))
    _check("w4a16_linear_prepacked", rc)
    return Y


def w4a16_linear(X_bf16: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor, group_size: int, Y=None, stream=None) -> torch.Tensor:
    """X_bf16 [M, K] (torch.bfloat16, or int16/uint16 bit patterns) -> Y [M, N] fp32."""
    M, K = _matrix(X_bf16, "X_bf16")
    N = _matrix(packed, "packed")[0]
    dev = X_bf16.device
    xptr = _half(X_bf16, "X_bf16")
    ts = _table_shape("asym", N, K, group_size)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    rc = lib().w4a16_linear(xptr, M, K, N,
                            _dev(packed, "packed", torch.uint8, (N, (K + 1) // 2), dev),
                            _dev(scales, "scales", torch.float32, ts, dev),
                            _dev(zeros, "zeros", torch.float32, ts, dev), group_size,
                            _dev(Y, "Y", torch.float32, (M, N), dev), _stream(stream))
    _check("w4a16_linear", rc)
    return Y
