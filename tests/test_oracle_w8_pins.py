"""Pins of the oracle's W8A8 functions (int8 per-channel weights, the INT8 path
that the Keras guide's "How it works" says the INT4 path follows apart from the
unpacking) against facts fixed by the pages and by mathematics:

* a hand-derived worked example (tests/golden/w8a8_small.json, with its source);
* brute force: each code is the nearest integer in [-128, 127] to the fp32
  quotient (ties to even), found by exhaustive search, with the quotient and
  the scale computed by another route (fp64 divide, one rounding to fp32);
* invariants: codes within [-127, 127] for finite inputs, max |code| = 127 in
  every non-zero channel, reconstruction error <= scale / 2, exact power-of-two
  rescaling;
* closed forms: integer-grid weights in [-127, 127] quantize losslessly, so the
  layer equals the exact integer product; y matches sum_k (qx sx)(qw sw) within
  two fp32 roundings; the int32 product equals a plain loop and numpy's int64
  matrix product.
"""
import json
import os

import numpy as np
import pytest

import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def f32_quotient(a, b):
    """Correctly rounded fp32 a/b via an fp64 divide and one rounding."""
    return (np.asarray(a, np.float64) / np.asarray(b, np.float64)).astype(np.float32)


def nearest_int(t: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Exhaustive search over [lo, hi]: the nearest integer, ties to even."""
    t = np.asarray(t, np.float64)
    best = np.zeros(t.shape, np.int64)
    bestd = np.full(t.shape, np.inf)
    for c in range(lo, hi + 1):
        d = np.abs(t - c)
        take = (d < bestd) | ((d == bestd) & (c % 2 == 0))
        best = np.where(take, c, best)
        bestd = np.where(take, d, bestd)
    return best


def test_w8_golden(orc):
    with open(os.path.join(GOLD, "w8a8_small.json")) as f:
        g = json.load(f)
    W = np.array(g["W"], np.float32)
    Wq, sw = orc.quantize_weight_w8(W)
    assert sw.tolist() == g["sw"]
    assert Wq.astype(int).tolist() == g["codes"]
    x = np.array(g["x"], np.float32)
    xq, sx = orc.quantize_act(x)
    assert xq.astype(int).tolist() == g["xq"] and sx.tolist() == g["sx"]
    assert orc.matmul_w8_i32(xq, Wq).tolist() == g["acc"]
    assert orc.w8a8_linear(x, Wq, sw).tolist() == g["y_nobias"]
    assert orc.w8a8_linear(x, Wq, sw, np.array(g["bias"], np.float32)).tolist() == g["y_bias"]


@pytest.mark.parametrize("K,N", [(1, 1), (2, 3), (7, 5), (33, 2), (64, 7), (129, 3)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_w8_weight_bruteforce(orc, K, N, seed):
    rng = np.random.default_rng(seed * 1000 + K * 7 + N)
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    if seed == 2:  # exact ties: half-integer multiples of the scale 2^-3
        W = (rng.integers(-254, 255, size=(K, N)) * 0.5 * 0.125).astype(np.float32)
        W[0, :] = 127 * 0.125
    Wq, sw = orc.quantize_weight_w8(W)
    absmax = np.abs(W).max(axis=0)
    expect_s = np.where(absmax == 0, np.float32(0), f32_quotient(absmax, 127.0))
    assert np.array_equal(sw.view(np.uint32), expect_s.astype(np.float32).view(np.uint32))
    t = np.where(sw > 0, f32_quotient(W, np.where(sw > 0, sw, 1)), 0)
    assert np.array_equal(Wq.T.astype(np.int64), nearest_int(t, -128, 127))


def test_w8_weight_invariants(orc):
    d = workloads.random_case(3, 4, 300, 64, sigma=0.02)
    W = d["W"]
    W[:, 5] = 0.0  # an all-zero channel
    Wq, sw = orc.quantize_weight_w8(W)
    codes = Wq.T.astype(np.int64)                       # [K, N]
    assert codes.min() >= -127 and codes.max() <= 127   # finite inputs never emit -128
    nz = sw > 0
    assert np.all(np.abs(codes[:, nz]).max(axis=0) == 127)
    assert sw[5] == 0 and np.all(codes[:, 5] == 0)
    err = np.abs(W.astype(np.float64) - codes * sw.astype(np.float64))
    assert np.all(err <= sw.astype(np.float64) * (0.5 + 2.0**-20))
    # power-of-two rescaling is exact: same codes, scale times 2^-4
    q2, s2 = orc.quantize_weight_w8(W * np.float32(1 / 16))
    assert np.array_equal(q2, Wq) and np.array_equal(s2, sw * np.float32(1 / 16))


def test_w8_int_grid_lossless(orc):
    rng = np.random.default_rng(12)
    K, N, M = 45, 9, 5
    W = rng.integers(-127, 128, size=(K, N)).astype(np.float32)
    W[rng.integers(0, K, size=N), np.arange(N)] = rng.choice([-127.0, 127.0], size=N)
    Wq, sw = orc.quantize_weight_w8(W)
    assert np.all(sw == 1.0)
    assert np.array_equal(Wq.T.astype(np.int64), W.astype(np.int64))
    X = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    X[np.arange(M), rng.integers(0, K, size=M)] = 127.0
    y = orc.w8a8_linear(X, Wq, sw)
    assert np.array_equal(y.astype(np.int64), X.astype(np.int64) @ W.astype(np.int64))


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (1, 7, 3), (4, 64, 5), (3, 33, 17)])
def test_w8_matmul_bruteforce(orc, M, K, N):
    Wq = workloads.random_int8(K * 3 + N, (N, K))
    xq = workloads.random_int8(M * 5 + K, (M, K))
    acc = orc.matmul_w8_i32(xq, Wq)
    want = np.zeros((M, N), np.int64)
    for m in range(M):          # plain triple loop on tiny shapes
        for n in range(N):
            want[m, n] = sum(int(xq[m, k]) * int(Wq[n, k]) for k in range(K))
    assert np.array_equal(acc.astype(np.int64), want)
    assert np.array_equal(acc.astype(np.int64), xq.astype(np.int64) @ Wq.astype(np.int64).T)


def test_w8_matmul_extremes(orc):
    """-128 times -128 everywhere: acc = 16384 K."""
    K = 4096
    Wq = np.full((2, K), -128, np.int8)
    xq = np.full((1, K), -128, np.int8)
    assert np.all(orc.matmul_w8_i32(xq, Wq) == 16384 * K)


@pytest.mark.parametrize("M,K,N", [(1, 10, 32), (4, 1152, 40), (9, 301, 13)])
def test_w8_dequant_closed_form(orc, M, K, N):
    d = workloads.random_case(M + K + N + 1, M, K, N, outliers=3, bias=True)
    Wq, sw = orc.quantize_weight_w8(d["W"])
    xq, sx = orc.quantize_act(d["x"])
    y = orc.w8a8_linear(d["x"], Wq, sw).astype(np.float64)
    exact = (xq.astype(np.float64) * sx[:, None]) @ (Wq.astype(np.float64) * sw[:, None]).T
    tol = 2.0**-23 * np.abs(exact) + 1e-300
    assert np.all(np.abs(y - exact) <= tol)
    yb = orc.w8a8_linear(d["x"], Wq, sw, d["bias"])
    assert np.array_equal(yb, (y.astype(np.float32) + d["bias"]).astype(np.float32))
    # W8A8 is closer to the fp32 layer than W4A8 on the same data
    ref = d["x"].astype(np.float64) @ d["W"].astype(np.float64)
    p4, s4 = orc.quantize_weight_sym(d["W"])
    y4 = orc.w4a8_linear(d["x"], p4, s4).astype(np.float64)
    assert np.linalg.norm(y - ref) < np.linalg.norm(y4 - ref)


def test_w8_nonfinite_rejected(orc):
    W = np.ones((4, 2), np.float32)
    W[1, 1] = np.inf
    with pytest.raises(orc.OracleError):
        orc.quantize_weight_w8(W)
