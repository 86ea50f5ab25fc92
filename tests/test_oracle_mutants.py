"""The oracle's pins catch plausible slips in its arithmetic.

Each case below copies `oracle/w4_oracle.c`, plants one mistake inside one
function (a quotient formed with the rounded reciprocal instead of the
correctly rounded division, the dequantization product associated the other
way, the bias fused into the last multiply), builds the copy with the
oracle's own compiler flags into a temporary directory, points the oracle's
Python front end at it, and checks that at least one of the pin checks of
`test_oracle_quotient_pins.py` fails.  The unmodified source, built the same
way, passes all of them.  CPU only; nothing is written outside the temporary
directory.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import test_oracle_quotient_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "w4_oracle.c")

# (name, function whose body is edited, text there, replacement)
MUTANTS = [
    ("dequant_acc_sx_first", "orc_dequant", "float y = a * s;",
     "float y = (a * sx[m]) * sw[n]; (void)s;"),
    ("dequant_acc_sw_first", "orc_dequant", "float y = a * s;",
     "float y = (a * sw[n]) * sx[m]; (void)s;"),
    ("dequant_bias_fma", "orc_dequant", "if (bias) y = y + bias[n];",
     "if (bias) y = fmaf(a, s, bias[n]);"),
    ("act_reciprocal", "orc_quantize_act", "float t = X[m * K + k] / s;",
     "float t = X[m * K + k] * (1.0f / s);"),
    ("sym_reciprocal", "orc_quantize_weight_sym", "float t = W[k * N + n] / s;",
     "float t = W[k * N + n] * (1.0f / s);"),
    ("w8_reciprocal", "orc_quantize_weight_w8", "float t = W[k * N + n] / s;",
     "float t = W[k * N + n] * (1.0f / s);"),
    ("asym_code_reciprocal", "orc_quantize_weight_asym", "float t = W[k * N + n] / s;",
     "float t = W[k * N + n] * (1.0f / s);"),
    ("asym_zero_point_reciprocal", "orc_quantize_weight_asym",
     "float zp = 0.0f - rne(lo / s);", "float zp = 0.0f - rne(lo * (1.0f / s));"),
]


def _mutate(src, func, old, new):
    """Replace `old` by `new` once, inside the definition of `func`."""
    start = src.index(f"\nint {func}(")
    end = src.find("\nint orc_", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) == 1, (func, old)
    return src[:start] + body.replace(old, new) + src[end:]


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    # the oracle's flags (oracle/build.py) without -Werror
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-frounding-math", "-I", os.path.dirname(SRC), "-o", path, c, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _run_checks(lib_path):
    """Which pin checks fail with the oracle library at lib_path."""
    saved = (oracle._LIB_PATH, oracle._lib)
    oracle._LIB_PATH, oracle._lib = lib_path, None
    failed = []
    try:
        for name, check in pins.CHECKS.items():
            try:
                check(oracle)
            except AssertionError:
                failed.append(name)
    finally:
        oracle._LIB_PATH, oracle._lib = saved
    return failed


@pytest.fixture(scope="module")
def src():
    if shutil.which("gcc") is None:
        pytest.skip("gcc is needed to build oracle variants")
    with open(SRC) as f:
        return f.read()


def test_unmodified_oracle_passes(src, tmp_path):
    lib = str(tmp_path / "control.so")
    _build(src, lib)
    assert _run_checks(lib) == []


@pytest.mark.parametrize("name,func,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(src, tmp_path, name, func, old, new):
    lib = str(tmp_path / f"{name}.so")
    _build(_mutate(src, func, old, new), lib)
    failed = _run_checks(lib)
    assert failed, f"planted slip {name} passes every pin"
