"""Pins of the CPU oracle against facts the pages and mathematics fix.

Nothing here re-types the oracle's formulas.  Each test checks the oracle
against something else:

* hand-derived worked examples under tests/golden/ (each cites its page);
* brute force: every code is the nearest point of the allowed code set to
  the fp32 quotient (ties to even), found by exhaustive search;
* the fp32 quotient and scale computed by a different route (fp64 divide,
  then one rounding to fp32, which equals the correctly rounded fp32 quotient
  because 53 >= 2*24 + 2);
* a textbook decode of two's-complement nibbles (arithmetic shift);
* closed forms: integer-grid inputs quantize losslessly, so the layer output
  equals the exact integer matrix product; y matches sum_k (qx*sx)(qw*sw)
  within two fp32 roundings;
* invariants: code ranges, max |code| = 7 / 127 per channel / row, reconstruction
  error <= scale/2, clamp-then-round equals round-then-clamp;
* library special cases: torch's bf16 conversion and numpy fp64 products.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers
def textbook_decode_signed(packed: np.ndarray, K: int) -> np.ndarray:
    """Two's complement nibbles via arithmetic shifts of int8."""
    p = packed.astype(np.uint8)
    lo = ((p << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int64)
    hi = (p.view(np.int8) >> 4).astype(np.int64)
    N = p.shape[0]
    out = np.zeros((N, K), np.int64)
    out[:, 0::2] = lo[:, : (K + 1) // 2]
    out[:, 1::2] = hi[:, : K // 2]
    return out


def textbook_decode_unsigned(packed: np.ndarray, K: int) -> np.ndarray:
    p = packed.astype(np.int64)
    N = p.shape[0]
    out = np.zeros((N, K), np.int64)
    out[:, 0::2] = (p % 16)[:, : (K + 1) // 2]
    out[:, 1::2] = (p // 16)[:, : K // 2]
    return out


def f32_quotient(a, b):
    """Correctly rounded fp32 a/b via an fp64 divide and one rounding."""
    return (np.asarray(a, np.float64) / np.asarray(b, np.float64)).astype(np.float32)


def nearest_code(t: np.ndarray, lo: int, hi: int, offset=None) -> np.ndarray:
    """Exhaustive search: the code c in [lo, hi] closest to t + offset, where
    ties go to the c whose c - offset is even (round half to even applied to
    t before the integer offset is added)."""
    t = np.asarray(t, np.float64)
    off = np.zeros_like(t) if offset is None else np.asarray(offset, np.float64)
    best = np.full(t.shape, np.nan)
    bestd = np.full(t.shape, np.inf)
    for c in range(lo, hi + 1):
        d = np.abs(t - (c - off))
        even = ((c - off) % 2) == 0
        take = (d < bestd) | ((d == bestd) & even)
        best = np.where(take, c, best)
        bestd = np.where(take, d, bestd)
    return best.astype(np.int64)


def int_grid_weights(rng, K, N):
    """Integer weights in [-7, 7] with a +-7 in every column (scale exactly 1)."""
    W = rng.integers(-7, 8, size=(K, N)).astype(np.float32)
    rows = rng.integers(0, K, size=N)
    W[rows, np.arange(N)] = rng.choice([-7.0, 7.0], size=N)
    return W


def int_grid_acts(rng, M, K):
    X = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    cols = rng.integers(0, K, size=M)
    X[np.arange(M), cols] = rng.choice([-127.0, 127.0], size=M)
    return X


SMALL_SHAPES = [(1, 1), (2, 1), (3, 4), (7, 5), (16, 3), (33, 2), (64, 7), (129, 3)]


# ------------------------------------------------------- symmetric weights
def test_sym_weight_golden(orc):
    g = _gold("w4a8_sym_weights.json")
    for case in g["cases"]:
        K = case["K"]
        W = np.array(case["W_column"], np.float32).reshape(K, 1)
        packed, sw = orc.quantize_weight_sym(W)
        assert sw[0] == np.float32(case["scale"])
        assert [int(v) for v in textbook_decode_signed(packed, K)[0]] == case["codes"]
        assert [f"{b:02x}" for b in packed[0]] == case["packed_hex"]


@pytest.mark.parametrize("K,N", SMALL_SHAPES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sym_weight_bruteforce(orc, K, N, seed):
    rng = np.random.default_rng(seed * 1000 + K * 7 + N)
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    if seed == 2:  # exact ties: half-integer multiples of the scale
        W = (rng.integers(-14, 15, size=(K, N)) * 0.5 * 0.25).astype(np.float32)
        W[0, :] = 7 * 0.25
    packed, sw = orc.quantize_weight_sym(W)
    absmax = np.abs(W).max(axis=0)
    expect_s = np.where(absmax == 0, np.float32(0), f32_quotient(absmax, 7.0))
    assert np.array_equal(sw.view(np.uint32), expect_s.astype(np.float32).view(np.uint32))
    codes = textbook_decode_signed(packed, K).T  # [K, N]
    t = np.where(sw > 0, f32_quotient(W, np.where(sw > 0, sw, 1)), 0)
    assert np.array_equal(codes, nearest_code(t, -8, 7))
    if K % 2:  # the unused high nibble of the last byte is zero
        assert np.all(packed[:, -1] >> 4 == 0)


def test_sym_weight_invariants(orc):
    d = workloads.random_case(3, 4, 300, 64, sigma=0.02)
    W = d["W"]
    W[:, 5] = 0.0  # an all-zero channel
    packed, sw = orc.quantize_weight_sym(W)
    codes = textbook_decode_signed(packed, 300).T
    assert codes.min() >= -7 and codes.max() <= 7       # finite inputs never emit -8
    nz = sw > 0
    assert np.all(np.abs(codes[:, nz]).max(axis=0) == 7)  # absmax element maps to +-7
    assert sw[5] == 0 and np.all(codes[:, 5] == 0)
    err = np.abs(W.astype(np.float64) - codes * sw.astype(np.float64))
    assert np.all(err <= sw.astype(np.float64) * (0.5 + 2.0**-20))
    # the blog's clamp-then-round form gives the same codes
    t = np.where(nz, f32_quotient(W, np.where(nz, sw, 1)), 0)
    assert np.array_equal(np.rint(np.clip(t, -8, 7)).astype(np.int64), codes)
    # power-of-two rescaling is exact: same codes, scale times 2^5
    p2, s2 = orc.quantize_weight_sym(W * np.float32(32))
    assert np.array_equal(p2, packed) and np.array_equal(s2, sw * np.float32(32))


def test_sym_weight_int_grid_lossless(orc):
    rng = np.random.default_rng(11)
    W = int_grid_weights(rng, 37, 9)
    packed, sw = orc.quantize_weight_sym(W)
    assert np.all(sw == 1.0)
    assert np.array_equal(textbook_decode_signed(packed, 37).T, W.astype(np.int64))


def test_unpack_all_bytes(orc):
    """Every byte value decodes to the two's complement pair (incl. code -8)."""
    packed = np.arange(256, dtype=np.uint8).reshape(256, 1)
    dec = orc.unpack_signed(packed, 2)
    want = textbook_decode_signed(packed, 2)
    assert np.array_equal(dec.astype(np.int64), want)
    assert dec.min() == -8 and dec.max() == 7


def test_pack_roundtrip_all_pairs(orc):
    """Codes a, b for every pair in [-7, 7]^2 survive quantize -> pack -> decode."""
    a, b = np.meshgrid(np.arange(-7, 8), np.arange(-7, 8), indexing="ij")
    N = a.size
    W = np.zeros((3, N), np.float32)
    W[0] = a.ravel()
    W[1] = b.ravel()
    W[2] = 7.0  # fixes every scale at 1
    packed, sw = orc.quantize_weight_sym(W)
    assert packed.shape == (N, 2)
    dec = textbook_decode_signed(packed, 3)
    assert np.array_equal(dec[:, 0], a.ravel()) and np.array_equal(dec[:, 1], b.ravel())
    assert np.array_equal(packed[:, 0], ((a.ravel() & 15) | ((b.ravel() & 15) << 4)).astype(np.uint8))


# ------------------------------------------------------------ activations
def test_act_golden(orc):
    g = _gold("a8_act_rows.json")
    for row in g["rows"]:
        x = np.array(row["x"], np.float32).reshape(1, -1)
        xq, sx = orc.quantize_act(x)
        assert sx[0] == np.float32(row["scale"])
        assert xq[0].tolist() == row["codes"]


@pytest.mark.parametrize("M,K", [(1, 1), (1, 10), (3, 33), (8, 1152), (5, 4096)])
def test_act_bruteforce(orc, M, K):
    d = workloads.random_case(M * 31 + K, M, K, 1, outliers=min(6, K))
    X = d["x"]
    xq, sx = orc.quantize_act(X)
    absmax = np.abs(X).max(axis=1)
    assert np.array_equal(sx, f32_quotient(absmax, 127.0))
    t = f32_quotient(X, sx[:, None])
    assert np.array_equal(xq.astype(np.int64), nearest_code(t, -128, 127))
    assert np.all(np.abs(xq.astype(np.int64)).max(axis=1) == 127)
    assert xq.min() >= -127
    err = np.abs(X.astype(np.float64) - xq * sx[:, None].astype(np.float64))
    assert np.all(err <= sx[:, None] * (0.5 + 2.0**-20))


def test_act_zero_row_and_ties(orc):
    X = np.zeros((3, 6), np.float32)
    X[1] = [127, 0.5, 1.5, 2.5, -0.5, -1.5]
    X[2] = [-254, 1, 3, 5, -1, 0]  # scale 2: 1/2, 3/2, 5/2 are ties
    xq, sx = orc.quantize_act(X)
    assert sx[0] == 0 and np.all(xq[0] == 0)
    assert xq[1].tolist() == [127, 0, 2, 2, 0, -2]
    assert sx[2] == 2.0 and xq[2].tolist() == [-127, 0, 2, 2, 0, 0]


def test_nonfinite_rejected(orc):
    X = np.ones((2, 4), np.float32)
    X[1, 2] = np.inf
    with pytest.raises(orc.OracleError):
        orc.quantize_act(X)
    W = np.ones((4, 2), np.float32)
    W[0, 0] = np.nan
    with pytest.raises(orc.OracleError):
        orc.quantize_weight_sym(W)


# ---------------------------------------------------------- integer GEMM
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (1, 7, 3), (4, 64, 5), (3, 33, 17), (16, 130, 9)])
def test_matmul_bruteforce(orc, M, K, N):
    packed = workloads.random_bytes(K * 3 + N, (N, (K + 1) // 2))
    if K % 2:
        packed[:, -1] &= 0x0F
    xq = workloads.random_int8(M * 5 + K, (M, K))
    acc = orc.matmul_i32(xq, packed, K)
    Wc = textbook_decode_signed(packed, K)
    want = np.zeros((M, N), np.int64)
    for m in range(M):          # plain triple loop on tiny shapes
        for n in range(N):
            want[m, n] = sum(int(xq[m, k]) * int(Wc[n, k]) for k in range(K))
    assert np.array_equal(acc.astype(np.int64), want)
    assert np.array_equal(acc.astype(np.int64), xq.astype(np.int64) @ Wc.T)


def test_matmul_extremes(orc):
    """Code -8 times -128 everywhere: acc = 1024 K, the largest magnitude."""
    K = 4096
    packed = np.full((2, K // 2), 0x88, np.uint8)
    xq = np.full((1, K), -128, np.int8)
    acc = orc.matmul_i32(xq, packed, K)
    assert np.all(acc == 1024 * K)


# ---------------------------------------------------------------- dequant
def test_linear_golden(orc):
    g = _gold("w4a8_linear_small.json")
    x = np.array(g["x"], np.float32)
    W = np.array(g["W"], np.float32)
    packed, sw = orc.quantize_weight_sym(W)
    assert sw.tolist() == g["sw"]
    xq, sx = orc.quantize_act(x)
    assert xq.tolist() == g["xq"] and sx.tolist() == g["sx"]
    acc = orc.matmul_i32(xq, packed, W.shape[0])
    assert acc.tolist() == g["acc"]
    assert orc.w4a8_linear(x, packed, sw).tolist() == g["y_nobias"]
    assert orc.w4a8_linear(x, packed, sw, np.array(g["bias"], np.float32)).tolist() == g["y_bias"]


@pytest.mark.parametrize("M,K,N", [(1, 10, 32), (4, 1152, 40), (9, 301, 13)])
def test_dequant_closed_form(orc, M, K, N):
    d = workloads.random_case(M + K + N, M, K, N, outliers=3, bias=True)
    packed, sw = orc.quantize_weight_sym(d["W"])
    xq, sx = orc.quantize_act(d["x"])
    y = orc.w4a8_linear(d["x"], packed, sw).astype(np.float64)
    qw = textbook_decode_signed(packed, K).astype(np.float64)      # [N, K]
    exact = (xq.astype(np.float64) * sx[:, None]) @ (qw * sw[:, None]).T
    tol = 2.0**-23 * np.abs(exact) + 1e-300
    assert np.all(np.abs(y - exact) <= tol)
    yb = orc.w4a8_linear(d["x"], packed, sw, d["bias"])
    assert np.array_equal(yb, (y.astype(np.float32) + d["bias"]).astype(np.float32))


def test_linear_int_grid_exact(orc):
    rng = np.random.default_rng(5)
    M, K, N = 6, 50, 11
    W = int_grid_weights(rng, K, N)
    X = int_grid_acts(rng, M, K)
    packed, sw = orc.quantize_weight_sym(W)
    y = orc.w4a8_linear(X, packed, sw)
    assert np.array_equal(y.astype(np.int64), X.astype(np.int64) @ W.astype(np.int64))


def test_toy_model_mse(orc):
    """The guide's toy model: two quantized Dense layers with ReLU between.
    The printed MSE (about 3e-4) used unseeded, unstated initializers, so only
    its order of magnitude is comparable."""
    t = workloads.toy_model()
    h = np.maximum(t["x"] @ t["W1"] + t["b1"], 0)
    y32 = h @ t["W2"] + t["b2"]
    p1, s1 = orc.quantize_weight_sym(t["W1"])
    p2, s2 = orc.quantize_weight_sym(t["W2"])
    hq = np.maximum(orc.w4a8_linear(t["x"], p1, s1, t["b1"]), 0)
    yq = orc.w4a8_linear(hq, p2, s2, t["b2"])
    mse = float(np.mean((y32 - yq) ** 2))
    print(f"toy model fp32 vs W4A8 MSE = {mse:.3e}")
    assert 0 < mse < 1e-2


# -------------------------------------------------- asymmetric groups, W4A16
def test_asym_golden(orc):
    g = _gold("w4a16_group.json")
    K, grp = g["K"], g["group"]
    W = np.array(g["W_column"], np.float32).reshape(K, 1)
    packed, s, z = orc.quantize_weight_asym(W, grp)
    assert s[0].tolist() == g["scales"] and z[0].tolist() == g["zeros"]
    assert textbook_decode_unsigned(packed, K)[0].tolist() == g["codes"]
    assert [f"{b:02x}" for b in packed[0]] == g["packed_hex"]
    wd = orc.bf16_bits_to_f32(orc.w4a16_dequant(packed, s, z, K, grp))
    assert wd[:, 0].tolist() == g["dequant"]
    x = orc.bf16_rne(np.array(g["x"], np.float32)).reshape(1, K)
    y, _ = orc.w4a16_linear(x, packed, s, z, grp)
    assert y[0, 0] == g["y"]


@pytest.mark.parametrize("K,N,grp", [(4, 3, 4), (8, 5, 4), (256, 6, 128), (384, 4, 128), (64, 9, 32)])
def test_asym_bruteforce(orc, K, N, grp):
    rng = np.random.default_rng(K + N + grp)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    W[:, 0] += np.float32(0.05)          # an all-positive channel: zero point < 0
    packed, s, z = orc.quantize_weight_asym(W, grp)
    G = K // grp
    Wg = W.T.reshape(N, G, grp)
    lo, hi = Wg.min(axis=2), Wg.max(axis=2)
    rng32 = (hi.astype(np.float64) - lo.astype(np.float64)).astype(np.float32)
    assert np.array_equal(s, f32_quotient(rng32, 15.0))
    zp = -np.rint(f32_quotient(lo, s).astype(np.float64))
    assert np.array_equal(z.astype(np.float64), zp)
    codes = textbook_decode_unsigned(packed, K).reshape(N, G, grp)
    t = f32_quotient(Wg, s[:, :, None])
    want = nearest_code(t, 0, 15, offset=np.broadcast_to(zp[:, :, None], t.shape))
    assert np.array_equal(codes, want)
    # invariants: every group spans code 0 and code 14 or 15; error <= scale/2
    assert np.all(codes.min(axis=2) == 0)
    assert np.all(np.isin(codes.max(axis=2), [14, 15]))
    err = np.abs(Wg - (codes - zp[:, :, None]) * s[:, :, None].astype(np.float64))
    assert np.all(err <= s[:, :, None] * (0.5 + 2.0**-18))


def test_asym_degenerate_groups(orc):
    W = np.zeros((8, 3), np.float32)
    W[:4, 0] = -0.75           # constant negative group
    W[4:, 0] = 0.0             # constant zero group
    W[:, 1] = 3.0              # constant positive channel
    W[:4, 2] = [0, 0, 0, 1e-3]
    W[4:, 2] = 5.0
    packed, s, z = orc.quantize_weight_asym(W, 4)
    wd = orc.bf16_bits_to_f32(orc.w4a16_dequant(packed, s, z, 8, 4))
    bf = orc.bf16_bits_to_f32(orc.bf16_rne(W))
    for n, g in [(0, 0), (0, 1), (1, 0), (1, 1), (2, 1)]:
        assert np.array_equal(wd[4 * g:4 * g + 4, n], bf[4 * g:4 * g + 4, n])  # exact reconstruction
    assert not np.any((z == 0) & np.signbit(z))  # a zero point of 0 is +0.0, never -0.0


def test_asym_int_grid_exact(orc):
    """Groups of integers 0..15 holding both 0 and 15: scale 1, zero point 0,
    so the W4A16 product is the exact product with the original weights."""
    rng = np.random.default_rng(9)
    K, N, M, grp = 256, 7, 3, 128
    W = rng.integers(0, 16, size=(K, N)).astype(np.float32)
    for g in range(K // grp):
        W[g * grp, :] = 0
        W[g * grp + 1, :] = 15
    packed, s, z = orc.quantize_weight_asym(W, grp)
    assert np.all(s == 1) and np.all(z == 0)
    xb = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    y, a = orc.w4a16_linear(xb, packed, s, z, grp)
    x = orc.bf16_bits_to_f32(xb).astype(np.float64)
    assert np.array_equal(y, x @ W.astype(np.float64))
    assert np.allclose(a, np.abs(x) @ np.abs(W.astype(np.float64)), rtol=1e-15, atol=0)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 2000),
        # exact ties between neighbouring bf16 values, both parities
        (np.arange(0x3F800000, 0x3F800000 + 64 * 0x10000, 0x10000, dtype=np.uint32) + 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-40], np.float32),
    ]).astype(np.float32)
    mine = orc.bf16_rne(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_w4a16_dequant_and_product_vs_library(orc):
    d = workloads.w4a16_inputs(M=3, N=24, with_w=False)
    rng = np.random.default_rng(4)
    K, N, grp = 512, 24, 128
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    packed, s, z = orc.quantize_weight_asym(W, grp)
    codes = textbook_decode_unsigned(packed, K).T            # [K, N]
    sk = np.repeat(s.T, grp, axis=0)                            # [K, N]
    zk = np.repeat(z.T, grp, axis=0)
    w32 = ((codes.astype(np.float32) - zk).astype(np.float32) * sk).astype(np.float32)
    wbf = torch.from_numpy(w32).to(torch.bfloat16).float().numpy()
    wd = orc.bf16_bits_to_f32(orc.w4a16_dequant(packed, s, z, K, grp))
    assert np.array_equal(wd, wbf)
    x = d["x_bf16"][:, :K].copy()
    y, a = orc.w4a16_linear(x, packed, s, z, grp)
    xf = orc.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ wbf.astype(np.float64)
    bound = 1e-13 * (np.abs(xf) @ np.abs(wbf.astype(np.float64)))
    assert np.all(np.abs(y - ref) <= bound)
    assert np.allclose(a, np.abs(xf) @ np.abs(wbf.astype(np.float64)), rtol=1e-13, atol=0)


# ---------------------------------------------------------- storage sizes
def test_storage_formulas():
    """W4A8: N*ceil(K/2) + 4N bytes, about 8x smaller than fp32 (Keras guide,
    'What is INT4 quantization').  W4A16 with group 128, 32-bit scale and zero
    point: 4 + 64/128 = 4.5 bits per weight (INT4 concept entry, 4.2)."""
    K, N = 1152, 6912
    w4a8 = N * ((K + 1) // 2) + 4 * N
    assert w4a8 == 3_981_312 + 27_648
    assert 7.9 < (4 * K * N) / w4a8 < 8.0
    M, K, N, g = 16, 8192, 28672, 128
    per_weight_bits = (N * K // 2 + 2 * 4 * N * K // g) * 8 / (N * K)
    assert per_weight_bits == 4.5
    assert N * K // 2 + 2 * 4 * N * K // g + 2 * M * K + 4 * M * N == 2**27


# ------------------------------------------------------------------- ReLU
def test_relu_special_values(orc):
    """IEEE facts: positive values pass unchanged (bit for bit), negative values,
    -0.0 and +0.0 give +0.0; non-finite outputs are rejected."""
    y = np.array([[1.5, -2.0, -0.0, 0.0, 3.4e38, -1e-45, 1e-45]], np.float32)
    r = orc.relu(y)
    assert r.view(np.uint32).tolist() == np.array(
        [[1.5, 0.0, 0.0, 0.0, 3.4e38, 0.0, 1e-45]], np.float32).view(np.uint32).tolist()
    assert y[0, 1] == -2.0  # the input is not modified
    with pytest.raises(orc.OracleError):
        orc.relu(np.array([np.nan], np.float32))


def test_relu_on_layer_outputs(orc):
    """Invariants on a real layer output: r >= +0 everywhere (no -0), r == y
    where y > 0, and the positive part plus the negative part gives y back."""
    d = workloads.random_case(77, 9, 301, 40, outliers=3, bias=True)
    packed, sw = orc.quantize_weight_sym(d["W"])
    y = orc.w4a8_linear(d["x"], packed, sw, d["bias"])
    r = orc.relu(y)
    assert np.all(r.view(np.uint32) >> 31 == 0)
    assert np.array_equal(r[y > 0], y[y > 0]) and np.all(r[y <= 0] == 0)
    assert np.array_equal(r + np.minimum(y, 0), y)
    assert 0 < (y > 0).mean() < 1
