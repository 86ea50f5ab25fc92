"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* libw4.so loads and exports every function include/w4.h declares;
* every argument check returns its documented status before any launch
  (NULL pointers, bad sizes, unknown scheme, misaligned pointers, missing or
  short workspace);
* the workspace size formula.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")

W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_SCHEME, W4_ERR_WORKSPACE, W4_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
W4_ERR_ARG = -7
W4_ERR_SCRATCH = -8
FAKE = 1 << 20  # a non-NULL, 256-aligned address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def w4():
    import int4_weight_quantized_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        pkg_build = __import__("int4_weight_quantized_amd.build", fromlist=["build"])
        pkg_build.build()
    return pkg


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["w4_quantize_weight", "a8_quantize_act", "w4a8_linear", "w4a16_linear",
                 "w4a8_linear_q", "w4a8_matmul_i32", "w4a8_workspace_bytes",
                 "w8_quantize_weight", "w8a8_workspace_bytes", "w8a8_linear",
                 "w8a8_matmul_i32", "w4a8_linear_act", "w8a8_linear_act",
                 "w4_dequantize_weight", "w4_merge_delta", "awq_channel_scales",
                 "awq_fold_weight", "awq_quantize_act", "awq_scale_act_bf16", "w4a8_linear_awq",
                 "w4a16_prepack", "w4a16_unprepack", "w4a16_linear_prepacked",
                 "w4a16_prepacked_weight_bytes", "w4a16_prepacked_table_floats",
                 "w4_prepacked_weight_bytes", "w4_prepack_weights", "w4_unprepack_weights",
                 "w4a8_linear_prepacked", "w4a8_linear_noalloc",
                 "w4_status_string", "w4_last_path"]:
        assert want in names, names


def test_library_exports_every_declared_symbol(w4):
    lib = w4.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libw4.so does not export {name}"


def test_status_strings(w4):
    for st in range(-8, 1):
        assert w4.w4_status_string(st) and w4.w4_status_string(st) != "unknown status"
    assert w4.w4_status_string(-99) == "unknown status"


def test_workspace_formula(w4):
    assert w4.w4a8_workspace_bytes(1, 1152, 6912) == 1280 + 256
    assert w4.w4a8_workspace_bytes(4096, 4096, 4096) == 4096 * 4096 + 16384
    assert w4.w4a8_workspace_bytes(0, 4096, 4096) == 0
    assert w4.w4a8_workspace_bytes(1, w4.W4_MAX_K + 1, 1) == 0


def test_quantize_weight_checks(w4):
    f = w4.lib().w4_quantize_weight
    assert f(None, 4, 4, 0, 0, FAKE, FAKE, None, None) == W4_ERR_NULL
    assert f(FAKE, 4, 4, 0, 0, None, FAKE, None, None) == W4_ERR_NULL
    assert f(FAKE, 0, 4, 0, 0, FAKE, FAKE, None, None) == W4_ERR_SHAPE
    assert f(FAKE, 4, -1, 0, 0, FAKE, FAKE, None, None) == W4_ERR_SHAPE
    assert f(FAKE, w4.W4_MAX_K + 1, 4, 0, 0, FAKE, FAKE, None, None) == W4_ERR_SHAPE
    assert f(FAKE + 2, 4, 4, 0, 0, FAKE, FAKE, None, None) == W4_ERR_ALIGN
    assert f(FAKE, 4, 4, 7, 0, FAKE, FAKE, None, None) == W4_ERR_SCHEME
    assert f(FAKE, 4, 4, 0, 128, FAKE, FAKE, None, None) == W4_ERR_SHAPE    # sym takes no group
    assert f(FAKE, 4, 4, 0, 0, FAKE, FAKE, FAKE, None) == W4_ERR_SHAPE      # sym takes no zeros
    assert f(FAKE, 256, 4, 1, 128, FAKE, FAKE, None, None) == W4_ERR_NULL   # asym needs zeros
    assert f(FAKE, 200, 4, 1, 128, FAKE, FAKE, FAKE, None) == W4_ERR_SHAPE  # K % group
    assert f(FAKE, 9, 4, 1, 3, FAKE, FAKE, FAKE, None) == W4_ERR_SHAPE      # odd group
    assert f(FAKE, 256, 4, 1, 128, FAKE, FAKE, FAKE + 1, None) == W4_ERR_ALIGN


def test_act_checks(w4):
    f = w4.lib().a8_quantize_act
    assert f(None, 1, 4, FAKE, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 0, 4, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert f(FAKE, 2, 0, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert f(FAKE + 1, 2, 4, FAKE, FAKE, None) == W4_ERR_ALIGN


def test_linear_checks(w4):
    f = w4.lib().w4a8_linear
    ws = w4.w4a8_workspace_bytes(2, 64, 8)
    assert f(None, 2, 64, 8, FAKE, FAKE, None, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 64, 8, FAKE, None, None, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 0, 8, FAKE, FAKE, None, FAKE, FAKE, ws, None) == W4_ERR_SHAPE
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE + 2, FAKE, ws, None) == W4_ERR_ALIGN
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, FAKE + 1, FAKE, FAKE, ws, None) == W4_ERR_ALIGN
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE, None, 0, None) == W4_ERR_WORKSPACE
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE, FAKE, ws - 1, None) == W4_ERR_WORKSPACE
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE, FAKE + 16, ws, None) == W4_ERR_ALIGN
    g = w4.lib().w4a8_linear_q
    assert g(FAKE, None, FAKE, FAKE, None, 2, 64, 8, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert g(FAKE, FAKE, FAKE, FAKE, None, 2, 64, -8, FAKE, FAKE, ws, None) == W4_ERR_SHAPE
    h = w4.lib().w4a8_matmul_i32
    assert h(FAKE, FAKE, 2, 64, 8, None, FAKE, ws, None) == W4_ERR_NULL
    assert h(FAKE, FAKE, 2, 64, 8, FAKE + 2, FAKE, ws, None) == W4_ERR_ALIGN
    assert h(FAKE, FAKE, 2, 64, 8, FAKE, FAKE, 3, None) == W4_ERR_WORKSPACE


def test_w8a8_checks(w4):
    q = w4.lib().w8_quantize_weight
    assert q(None, 4, 4, FAKE, FAKE, None) == W4_ERR_NULL
    assert q(FAKE, 4, 4, None, FAKE, None) == W4_ERR_NULL
    assert q(FAKE, 0, 4, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert q(FAKE, w4.W4_MAX_K + 1, 4, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert q(FAKE, 4, 4, FAKE, FAKE + 2, None) == W4_ERR_ALIGN
    ws = w4.lib().w8a8_workspace_bytes(2, 64, 8)
    assert ws == w4.w4a8_workspace_bytes(2, 64, 8)
    assert w4.lib().w8a8_workspace_bytes(1, 0, 8) == 0
    f = w4.lib().w8a8_linear
    assert f(None, 2, 64, 8, FAKE, FAKE, None, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 64, 8, None, FAKE, None, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 64, 0, FAKE, FAKE, None, FAKE, FAKE, ws, None) == W4_ERR_SHAPE
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE + 2, FAKE, ws, None) == W4_ERR_ALIGN
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE, None, 0, None) == W4_ERR_WORKSPACE
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, FAKE, FAKE + 16, ws, None) == W4_ERR_ALIGN
    h = w4.lib().w8a8_matmul_i32
    assert h(FAKE, None, 2, 64, 8, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert h(FAKE, FAKE, 2, 64, 8, FAKE + 2, FAKE, ws, None) == W4_ERR_ALIGN
    assert h(FAKE, FAKE, 2, 64, 8, FAKE, FAKE, 3, None) == W4_ERR_WORKSPACE


def test_linear_act_checks(w4):
    ws = w4.w4a8_workspace_bytes(2, 64, 8)
    for f in (w4.lib().w4a8_linear_act, w4.lib().w8a8_linear_act):
        assert f(None, 2, 64, 8, FAKE, FAKE, None, 1, FAKE, FAKE, ws, None) == W4_ERR_NULL
        assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, 2, FAKE, FAKE, ws, None) == W4_ERR_ARG
        assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, -1, FAKE, FAKE, ws, None) == W4_ERR_ARG
        assert f(FAKE, 0, 64, 8, FAKE, FAKE, None, 1, FAKE, FAKE, ws, None) == W4_ERR_SHAPE
        assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, 1, FAKE + 2, FAKE, ws, None) == W4_ERR_ALIGN
        assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, 1, FAKE, FAKE, ws - 1, None) == W4_ERR_WORKSPACE
    with pytest.raises(ValueError):
        w4._act("gelu")


def test_dequant_merge_checks(w4):
    d = w4.lib().w4_dequantize_weight
    assert d(None, FAKE, None, 4, 4, 0, 0, FAKE, None) == W4_ERR_NULL
    assert d(FAKE, FAKE, None, 4, 4, 0, 0, None, None) == W4_ERR_NULL
    assert d(FAKE, FAKE, None, 0, 4, 0, 0, FAKE, None) == W4_ERR_SHAPE
    assert d(FAKE, FAKE, None, 4, 4, 5, 0, FAKE, None) == W4_ERR_SCHEME
    assert d(FAKE, FAKE, FAKE, 4, 4, 0, 0, FAKE, None) == W4_ERR_SHAPE     # sym takes no zeros
    assert d(FAKE, FAKE, None, 256, 4, 1, 128, FAKE, None) == W4_ERR_NULL  # asym needs zeros
    assert d(FAKE, FAKE, FAKE, 200, 4, 1, 128, FAKE, None) == W4_ERR_SHAPE
    assert d(FAKE, FAKE, None, 4, 4, 0, 0, FAKE + 2, None) == W4_ERR_ALIGN
    m = w4.lib().w4_merge_delta
    assert m(FAKE, FAKE, None, 4, 4, 0, 0, None, FAKE, FAKE, None, FAKE, None) == W4_ERR_NULL
    assert m(FAKE, FAKE, None, 4, 4, 0, 0, FAKE, FAKE, FAKE, None, None, None) == W4_ERR_NULL
    assert m(FAKE, FAKE, None, 4, 4, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert m(FAKE, FAKE, FAKE, 256, 4, 1, 128, FAKE, FAKE, FAKE, None, FAKE, None) == W4_ERR_NULL
    assert m(FAKE, FAKE, None, 4, 4, 0, 0, FAKE, FAKE, FAKE, None, FAKE + 1, None) == W4_ERR_ALIGN
    assert m(FAKE, FAKE, None, 4, 4, 9, 0, FAKE, FAKE, FAKE, None, FAKE, None) == W4_ERR_SCHEME


def test_awq_checks(w4):
    L = w4.lib()
    assert L.awq_channel_scales(None, 4, 8, 1, 2, FAKE, None) == W4_ERR_NULL
    assert L.awq_channel_scales(FAKE, 0, 8, 1, 2, FAKE, None) == W4_ERR_SHAPE
    assert L.awq_channel_scales(FAKE, 4, 8, 1, 0, FAKE, None) == W4_ERR_ARG
    assert L.awq_channel_scales(FAKE, 4, 8, -1, 2, FAKE, None) == W4_ERR_ARG
    assert L.awq_channel_scales(FAKE, 4, 8, 1, 2, FAKE + 2, None) == W4_ERR_ALIGN
    assert L.awq_fold_weight(FAKE, 4, 8, None, FAKE, None) == W4_ERR_NULL
    assert L.awq_fold_weight(FAKE, 4, 0, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert L.awq_quantize_act(FAKE, 2, 8, None, FAKE, FAKE, None) == W4_ERR_NULL
    assert L.awq_scale_act_bf16(FAKE + 1, 2, 8, FAKE, FAKE, None) == W4_ERR_ALIGN
    ws = w4.w4a8_workspace_bytes(2, 64, 8)
    f = L.w4a8_linear_awq
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, None, None, 0, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, FAKE + 4, None, 0, FAKE, FAKE, ws, None) == W4_ERR_ALIGN
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, FAKE, None, 5, FAKE, FAKE, ws, None) == W4_ERR_ARG
    assert f(FAKE, 2, 64, 8, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 0, None) == W4_ERR_WORKSPACE


def test_prepacked_checks(w4):
    L = w4.lib()
    assert L.w4a16_prepacked_weight_bytes(8192, 28672) == 28672 * 4096
    assert L.w4a16_prepacked_weight_bytes(512, 37) == 48 * 256
    assert L.w4a16_prepacked_table_floats(512, 37) == 48 * 4 * 2
    assert L.w4a16_prepacked_weight_bytes(256, 16) == 0            # K % 512 != 0
    p = L.w4a16_prepack
    assert p(None, FAKE, FAKE, 512, 16, 128, FAKE, FAKE, None) == W4_ERR_NULL
    assert p(FAKE, FAKE, FAKE, 512, 16, 64, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert p(FAKE, FAKE, FAKE, 768, 16, 128, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert p(FAKE + 4, FAKE, FAKE, 512, 16, 128, FAKE, FAKE, None) == W4_ERR_ALIGN
    u = L.w4a16_unprepack
    assert u(FAKE, None, 512, 16, 128, FAKE, FAKE, FAKE, None) == W4_ERR_NULL
    assert u(FAKE, FAKE, 512, 16, 128, FAKE, FAKE, FAKE + 2, None) == W4_ERR_ALIGN
    f = L.w4a16_linear_prepacked
    assert f(FAKE, 1, 512, 16, None, FAKE, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 1, 384, 16, FAKE, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert f(FAKE + 2, 1, 512, 16, FAKE, FAKE, FAKE, None) == W4_ERR_ALIGN


def test_w4a8_prepacked_checks(w4):
    L = w4.lib()
    assert L.w4_prepacked_weight_bytes(1152, 6912) == 6912 * 576
    assert L.w4_prepacked_weight_bytes(1152, 37) == 48 * 576
    assert L.w4_prepacked_weight_bytes(1000, 16) == 0
    assert L.w4_prepack_weights(None, 128, 16, FAKE, None) == W4_ERR_NULL
    assert L.w4_prepack_weights(FAKE, 96, 16, FAKE, None) == W4_ERR_SHAPE
    assert L.w4_prepack_weights(FAKE, 128, 16, FAKE + 8, None) == W4_ERR_ALIGN
    assert L.w4_unprepack_weights(FAKE, 128, 0, FAKE, None) == W4_ERR_SHAPE
    ws = w4.w4a8_workspace_bytes(2, 128, 8)
    f = L.w4a8_linear_prepacked
    assert f(FAKE, 2, 128, 8, None, FAKE, None, 0, FAKE, FAKE, ws, None) == W4_ERR_NULL
    assert f(FAKE, 2, 96, 8, FAKE, FAKE, None, 0, FAKE, FAKE, ws, None) == W4_ERR_SHAPE
    assert f(FAKE, 2, 128, 8, FAKE + 4, FAKE, None, 0, FAKE, FAKE, ws, None) == W4_ERR_ALIGN
    assert f(FAKE, 2, 128, 8, FAKE, FAKE, None, 3, FAKE, FAKE, ws, None) == W4_ERR_ARG
    assert f(FAKE, 2, 128, 8, FAKE, FAKE, None, 0, FAKE, FAKE, 0, None) == W4_ERR_WORKSPACE


def test_w4a16_checks(w4):
    f = w4.lib().w4a16_linear
    assert f(None, 1, 256, 8, FAKE, FAKE, FAKE, 128, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 1, 256, 8, FAKE, FAKE, None, 128, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 1, 200, 8, FAKE, FAKE, FAKE, 128, FAKE, None) == W4_ERR_SHAPE
    assert f(FAKE, 1, 256, 8, FAKE, FAKE, FAKE, 0, FAKE, None) == W4_ERR_SHAPE
    assert f(FAKE + 1, 1, 256, 8, FAKE, FAKE, FAKE, 128, FAKE, None) == W4_ERR_ALIGN


def test_probe_checks(w4):
    lib = w4.lib()
    assert lib.w4_probe_read(None, 64, FAKE, None) == W4_ERR_NULL
    assert lib.w4_probe_read(FAKE, 24, FAKE, None) == W4_ERR_SHAPE
    assert lib.w4_probe_read(FAKE + 8, 64, FAKE, None) == W4_ERR_ALIGN
    assert lib.w4_probe_write(None, 64, 0, None) == W4_ERR_NULL
    assert lib.w4_probe_write(FAKE, 8, 0, None) == W4_ERR_SHAPE
    assert lib.w4_probe_write(FAKE, 24, 0, None) == W4_ERR_SHAPE
    assert lib.w4_probe_write(FAKE, 0x7F000010, 0, None) == W4_ERR_SHAPE
    assert lib.w4_probe_write(FAKE + 8, 64, 0, None) == W4_ERR_ALIGN
    assert lib.w4_probe_mfma(8, 100, None, None, FAKE, None) == W4_ERR_NULL
    assert lib.w4_probe_mfma(0, 100, None, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert lib.w4_probe_mfma(8, 102, None, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert lib.w4_probe_mfma(8, 0, None, FAKE, FAKE, None) == W4_ERR_SHAPE
    assert lib.w4_probe_mfma(8, 100, FAKE + 8, FAKE, FAKE, None) == W4_ERR_ALIGN


def test_binding_refuses_cpu_tensors(w4):
    import torch
    with pytest.raises(ValueError):
        w4.a8_quantize_act(torch.zeros(2, 8))


def test_product_path_has_no_cpu_fallback(tmp_path):
    """The package never imports the oracle, and without its HIP library
    every call fails loudly instead of computing anything on the CPU."""
    import subprocess
    import sys
    code = (
        "import sys\n"
        "import int4_weight_quantized_amd as w4\n"
        "w4.lib()\n"
        "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'\n"
        f"w4.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "w4._lib = None\n"
        "try:\n"
        "    w4.lib()\n"
        "except RuntimeError as e:\n"
        "    assert 'missing' in str(e)\n"
        "else:\n"
        "    raise AssertionError('no error without the library')\n"
        "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]


def test_noalloc_checks_before_any_hip_call(w4):
    """The no-allocation call refuses NULL pointers, bad sizes and shapes whose
    scratch would exceed its fixed buffer on the host, before touching HIP."""
    f = w4.lib().w4a8_linear_noalloc
    assert f(None, 1, 64, 8, FAKE, FAKE, None, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 1, 64, 8, FAKE, None, None, FAKE, None) == W4_ERR_NULL
    assert f(FAKE, 0, 64, 8, FAKE, FAKE, None, FAKE, None) == W4_ERR_SHAPE
    cap = w4.W4_NOALLOC_SCRATCH_BYTES
    assert w4.w4a8_workspace_bytes(4096, 4096, 4096) <= cap
    assert w4.w4a8_workspace_bytes(4200, 4096, 8) > cap
    assert f(FAKE, 4200, 4096, 8, FAKE, FAKE, None, FAKE, None) == W4_ERR_SCRATCH
    assert f(FAKE, 1 << 20, 64, 8, FAKE, FAKE, None, FAKE, None) == W4_ERR_SCRATCH
