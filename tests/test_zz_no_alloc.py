"""w4a8_linear_noalloc: the no-allocation variant of w4a8_linear.

Its scratch (the activation codes and row scales of the MFMA paths) is the
library's fixed device array instead of a caller's workspace.  Its outputs
must be bit-identical to w4a8_linear's on the same inputs, on two calls in a
row whose second is smaller (the array keeps the first call's contents), at
the largest shape the array holds, and on a one-row decode step (which needs
no scratch at all).  Shapes past the array's size are refused before any
launch.
"""
import numpy as np
import pytest
import torch

import int4_weight_quantized_amd as W4
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def layer(seed, M, K, N, bias=True):
    d = workloads.random_case(seed, M, K, N, outliers=3, bias=bias)
    packed, sw, _ = W4.w4_quantize_weight(torch.from_numpy(d["W"]).to(DEV), "sym")
    x = torch.from_numpy(d["x"]).to(DEV)
    b = torch.from_numpy(d["bias"]).to(DEV) if bias else None
    return x, packed, sw, b


def both(x, packed, sw, b):
    M, N = x.shape[0], packed.shape[0]
    y_ref = W4.w4a8_linear(x, packed, sw, bias=b)
    path_ref = W4.w4_last_path()
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    W4.w4a8_linear_noalloc(x, packed, sw, y, bias=b)
    path = W4.w4_last_path()
    torch.cuda.synchronize()
    return y_ref, y, path_ref, path


def test_two_calls_in_a_row_second_smaller():
    cases = [(11, 300, 1024, 520, "gemm_mfma"),      # GEMM: row-major codes in the scratch
             (12, 20, 512, 200, "gemv_mfma")]        # decode batch: chunk-major codes
    for seed, M, K, N, want in cases:
        print(f"noalloc: {M}x{K}x{N}", flush=True)
        y_ref, y, p_ref, p = both(*layer(seed, M, K, N))
        assert p == p_ref == want, (p, p_ref)
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (M, K, N)


def test_largest_shape_the_scratch_holds():
    M = K = N = 4096
    assert W4.w4a8_workspace_bytes(M, K, N) <= W4.W4_NOALLOC_SCRATCH_BYTES
    print("noalloc: 4096x4096x4096", flush=True)
    y_ref, y, p_ref, p = both(*layer(13, M, K, N, bias=False))
    assert p == p_ref == "gemm_mfma"
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))


def test_decode_step_without_scratch_use():
    print("noalloc: 1x1152x6912", flush=True)
    y_ref, y, p_ref, p = both(*layer(14, 1, 1152, 6912))
    assert p == p_ref == "gemv_dot4"
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))


def test_refuses_shapes_past_the_scratch():
    M, K, N = 4200, 4096, 16
    assert W4.w4a8_workspace_bytes(M, K, N) > W4.W4_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    packed = torch.zeros((N, K // 2), dtype=torch.uint8, device=DEV)
    sw = torch.ones(N, dtype=torch.float32, device=DEV)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(W4.W4Error, match="scratch") as e:
        W4.w4a8_linear_noalloc(x, packed, sw, y)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "nothing is launched on refusal"
