"""Pins of the oracle's AWQ-style channel scaling ("INT4" concept entry,
section 4.4: measure each input channel's activation magnitude on
calibration data, scale the important channels' weights up, W' = W diag(s),
and divide the activations by s at inference), against facts that do not
re-type the oracle:

* closed forms: calibration columns with power-of-two magnitudes 2^j above a
  median level 2^0 get s = 2^floor(alpha j); all-zero, sub-median and
  subnormal channels get s = 1; the lower median for even K;
* invariances: row order, signs and a global power-of-two rescaling of the
  calibration data leave s unchanged;
* exactness: with power-of-two s, W*s/s == W, (x/s)(W s) == x W term by term
  (equal fp64 products), and bf16 x/2^e only lowers the exponent field;
* special case: s = 1 reduces to the plain activation quantization and
  forward;
* the accuracy effect on the 7B-class input with six x50 outlier channels
  (fixed seeds): the error against the fp32 layer drops for the group-wise
  W4A16 layer at alpha = 1/2 and for the per-channel W4A8 layer at
  alpha = 1/4.
"""
import numpy as np
import pytest

import workloads


def calib(K, M=8, big=None, seed=0):
    """Calibration rows whose channel absmax is exactly 1.0, except the
    channels in `big` (index -> absmax)."""
    rng = np.random.default_rng(seed)
    X = (rng.random((M, K)) * 0.9).astype(np.float32)
    X[rng.integers(0, M), :] = 1.0
    for k, a in (big or {}).items():
        X[:, k] *= np.float32(a) / np.float32(1.0)
        X[:, k] = np.minimum(np.abs(X[:, k]), np.float32(a)) * np.sign(X[:, k] + 0.5)
        X[0, k] = np.float32(a)
    return X


def test_scales_closed_form(orc):
    K = 32
    big = {3: 2.0, 5: 4.0, 7: 8.0, 11: 64.0, 13: 96.0, 17: 2.0**20}
    X = calib(K, big=big)
    X[:, 20] = 0.0                 # all-zero channel
    X[:, 21] *= np.float32(0.25)   # below the median
    X[:, 22] = np.float32(1e-40)   # subnormal magnitude
    for num, den in [(1, 2), (1, 4), (3, 4), (1, 1)]:
        s = orc.awq_channel_scales(X, (num, den))
        want = np.ones(K, np.float32)
        for k, a in big.items():
            j = int(np.floor(np.log2(a)))
            want[k] = 2.0 ** min(24, (j * num) // den)
        assert np.array_equal(s, want), (num, den, s)


def test_zero_channels_as_median(orc):
    """All-zero channels sit below every finite magnitude (E = -150): with two
    of three channels zero the median is -150, so a channel of magnitude
    2^-140 (E = -140) is 10 octaves above it: s = 2^10 at alpha = 1."""
    X = np.array([[0.0, 0.0, 2.0**-140], [0.0, 0.0, -(2.0**-141)]], np.float32)
    assert orc.awq_channel_scales(X, (1, 1)).tolist() == [1.0, 1.0, 1024.0]
    assert orc.awq_channel_scales(X, (1, 2)).tolist() == [1.0, 1.0, 32.0]


def test_scales_huge_channel_capped(orc):
    X = calib(16, big={2: 2.0**100})
    s = orc.awq_channel_scales(X, (1, 1))
    assert s[2] == 2.0**24 and np.all(np.delete(s, 2) == 1)


def test_lower_median_even_K(orc):
    """K = 4 with exponents [0, 0, 4, 4]: the lower median is 0, so the two
    large channels get 2^floor(4/2) = 4 (the upper median would give 1)."""
    X = np.array([[1.0, 1.0, 16.0, 16.0]], np.float32)
    assert orc.awq_channel_scales(X, (1, 2)).tolist() == [1.0, 1.0, 4.0, 4.0]


def test_scales_invariances(orc):
    d = workloads.generate("mlp7b", M=32)
    X = d["x"]
    s = orc.awq_channel_scales(X)
    assert np.array_equal(orc.awq_channel_scales(X[::-1].copy()), s)
    assert np.array_equal(orc.awq_channel_scales(-X), s)
    assert np.array_equal(orc.awq_channel_scales(X * np.float32(2.0**-7)), s)
    assert (s > 1).sum() == 6      # exactly the six x50 outlier channels


def test_fold_exact_and_product_identity(orc):
    d = workloads.random_case(5, 6, 256, 24, outliers=4)
    s = orc.awq_channel_scales(d["x"])
    assert (s > 1).any()
    Wf = orc.awq_fold_weight(d["W"], s)
    assert np.array_equal(Wf / s[:, None], d["W"])
    xs = d["x"] / s[None, :]
    assert np.array_equal(xs * s[None, :], d["x"])        # exact (powers of two)
    lhs = xs.astype(np.float64) @ Wf.astype(np.float64)
    rhs = d["x"].astype(np.float64) @ d["W"].astype(np.float64)
    assert np.array_equal(lhs, rhs)


def test_bf16_scaling_lowers_exponent(orc):
    rng = np.random.default_rng(4)
    K = 64
    x = workloads.to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32) + 3.0)
    e = rng.integers(0, 6, size=K)
    s = (2.0 ** e).astype(np.float32)
    out = orc.awq_scale_bf16(x, s)
    want = x.astype(np.int64) - (e[None, :] << 7)      # exponent field is bits 7..14
    assert np.array_equal(out.astype(np.int64), want)


def test_unit_scales_reduce_to_plain(orc):
    d = workloads.random_case(6, 5, 300, 17, outliers=3, bias=True)
    ones = np.ones(300, np.float32)
    xq, sx = orc.quantize_act(d["x"])
    xq1, sx1 = orc.awq_quantize_act(d["x"], ones)
    assert np.array_equal(xq, xq1) and np.array_equal(sx, sx1)
    p, sw = orc.quantize_weight_sym(d["W"])
    assert np.array_equal(orc.w4a8_linear_awq(d["x"], p, sw, ones, d["bias"]),
                          orc.w4a8_linear(d["x"], p, sw, d["bias"]))


def test_accuracy_on_outlier_channels(orc):
    """Fixed-seed accuracy effect on the 7B-class input (6 channels x50)."""
    d = workloads.generate("mlp7b", M=80)
    X, W = d["x"], d["W"][:, :192].copy()
    cal, ev = X[:64], X[64:]
    ref = ev.astype(np.float64) @ W.astype(np.float64)

    def err(y, r=ref):
        return np.linalg.norm(y - r) / np.linalg.norm(r)

    p, sw = orc.quantize_weight_sym(W)
    plain8 = err(orc.w4a8_linear(ev, p, sw))
    s4 = orc.awq_channel_scales(cal, (1, 4))
    p4, sw4 = orc.quantize_weight_sym(orc.awq_fold_weight(W, s4))
    awq8 = err(orc.w4a8_linear_awq(ev, p4, sw4, s4))

    xb = workloads.to_bf16_bits(ev)
    ref16 = orc.bf16_bits_to_f32(xb).astype(np.float64) @ W.astype(np.float64)
    pa, sa, za = orc.quantize_weight_asym(W, 128)
    plain16 = err(orc.w4a16_linear(xb, pa, sa, za, 128)[0], ref16)
    s2 = orc.awq_channel_scales(cal, (1, 2))
    pb, sb, zb = orc.quantize_weight_asym(orc.awq_fold_weight(W, s2), 128)
    awq16 = err(orc.w4a16_linear(orc.awq_scale_bf16(xb, s2), pb, sb, zb, 128)[0], ref16)
    print(f"W4A8 {plain8:.4f} -> {awq8:.4f} (alpha 1/4); W4A16 {plain16:.4f} -> {awq16:.4f} (alpha 1/2)")
    assert awq8 < 0.8 * plain8
    assert awq16 < 0.7 * plain16
