"""Pins of the oracle's weight dequantization and LoRA-style merge (Keras guide,
"Limitations": the LoRA export path dequantizes, adds the delta and
requantizes), against facts that do not re-type the oracle:

* dequantized values by another route: codes decoded with a textbook nibble
  decode, the exact product q*s (or (q - zp)*s) formed in fp64 and rounded to
  fp32 once (both factors are exact in fp64, so this is fl(q*s));
* the reconstruction bound |dequant(quantize(W)) - W| <= scale/2;
* idempotence: a zero delta gives back the same codes (symmetric channels;
  asymmetric groups whose codes span 0..15), scales within 2 ulp;
* a closed form: integer-grid weights (scale 1) plus an integer delta that
  keeps every channel's absmax at 7 requantize to codes W + delta exactly;
* the merged codes stay in their range, and the merged weights are within
  half a new scale of the fp32 sum dequant(q) + delta.
"""
import numpy as np
import pytest

import workloads
from test_oracle_pins import textbook_decode_signed, textbook_decode_unsigned


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("K,N", [(1, 1), (7, 5), (64, 9), (300, 33)])
def test_dequant_sym_other_route(orc, K, N):
    d = workloads.random_case(K + 5 * N, 1, K, N, sigma=0.03)
    packed, sw = orc.quantize_weight_sym(d["W"])
    Wd = orc.dequant_weight(packed, sw, None, K)
    q = textbook_decode_signed(packed, K).astype(np.float64)          # [N, K]
    want = (q * sw.astype(np.float64)[:, None]).T.astype(np.float32)  # one rounding
    assert np.array_equal(Wd.view(np.uint32), want.view(np.uint32))
    err = np.abs(Wd.astype(np.float64) - d["W"].astype(np.float64))
    assert np.all(err <= sw.astype(np.float64)[None, :] * (0.5 + 2.0**-20))


@pytest.mark.parametrize("K,N,g", [(8, 3, 4), (256, 6, 128), (384, 5, 64)])
def test_dequant_asym_other_route(orc, K, N, g):
    rng = np.random.default_rng(K + N + g)
    W = (rng.standard_normal((K, N)) * 0.015 + 0.004).astype(np.float32)
    packed, s, z = orc.quantize_weight_asym(W, g)
    Wd = orc.dequant_weight(packed, s, z, K, g)
    q = textbook_decode_unsigned(packed, K).astype(np.float64)        # [N, K]
    sk = np.repeat(s.astype(np.float64), g, axis=1)                   # [N, K]
    zk = np.repeat(z.astype(np.float64), g, axis=1)
    want = ((q - zk) * sk).T.astype(np.float32)
    assert np.array_equal(Wd.view(np.uint32), want.view(np.uint32))
    assert np.all(np.abs(Wd.astype(np.float64) - W) <= sk.T * (0.5 + 2.0**-20) + 1e-12)


def test_merge_zero_delta_sym_idempotent(orc):
    d = workloads.random_case(41, 1, 1152, 96, sigma=0.02)
    K, N = 1152, 96
    packed, sw = orc.quantize_weight_sym(d["W"])
    p2, s2, _ = orc.merge_delta(packed, sw, None, K, np.zeros((K, N), np.float32))
    assert np.array_equal(p2, packed)
    assert np.all(ulp_diff(s2, sw) <= 2)


def test_merge_zero_delta_asym_idempotent(orc):
    K, N, g = 512, 24, 128
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((K, N)) * 0.015).astype(np.float32)
    packed, s, z = orc.quantize_weight_asym(W, g)
    p2, s2, z2 = orc.merge_delta(packed, s, z, K, np.zeros((K, N), np.float32), g)
    q, q2 = textbook_decode_unsigned(packed, K), textbook_decode_unsigned(p2, K)
    G = K // g
    full = np.zeros((N, G), bool)  # groups whose codes span 0..15
    for gi in range(G):
        blk = q[:, gi * g:(gi + 1) * g]
        full[:, gi] = (blk.min(axis=1) == 0) & (blk.max(axis=1) == 15)
    assert full.mean() > 0.3
    for n in range(N):
        for gi in range(G):
            if full[n, gi]:
                sl = slice(gi * g, (gi + 1) * g)
                assert np.array_equal(q2[n, sl], q[n, sl])
                assert z2[n, gi] == z[n, gi] and ulp_diff(s2[n, gi], s[n, gi]) <= 2


def test_merge_integer_grid_closed_form(orc):
    rng = np.random.default_rng(3)
    K, N = 40, 12
    W = rng.integers(-3, 4, size=(K, N)).astype(np.float32)
    W[0, :] = 7.0                                      # absmax 7 -> scale 1
    delta = rng.integers(-2, 3, size=(K, N)).astype(np.float32)
    delta[0, :] = 0.0                                  # keeps the absmax at 7
    packed, sw = orc.quantize_weight_sym(W)
    assert np.all(sw == 1.0)
    p2, s2, _ = orc.merge_delta(packed, sw, None, K, delta)
    assert np.all(s2 == 1.0)
    assert np.array_equal(textbook_decode_signed(p2, K).T, (W + delta).astype(np.int64))


@pytest.mark.parametrize("asym", [False, True])
def test_merge_lora_delta_bounds(orc, asym):
    """A rank-4 delta B @ A of about 10% of the weights' size."""
    rng = np.random.default_rng(17)
    K, N, g, r = 256, 40, 128, 4
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    delta = ((rng.standard_normal((K, r)) @ rng.standard_normal((r, N))) * 0.001).astype(np.float32)
    if asym:
        packed, s, z = orc.quantize_weight_asym(W, g)
        p2, s2, z2 = orc.merge_delta(packed, s, z, K, delta, g)
        codes = textbook_decode_unsigned(p2, K)
        assert codes.min() >= 0 and codes.max() <= 15
        target = orc.dequant_weight(packed, s, z, K, g) + delta
        back = orc.dequant_weight(p2, s2, z2, K, g)
        bound = np.repeat(s2, g, axis=1).T
    else:
        packed, s = orc.quantize_weight_sym(W)
        p2, s2, _ = orc.merge_delta(packed, s, None, K, delta)
        codes = textbook_decode_signed(p2, K)
        assert codes.min() >= -7 and codes.max() <= 7
        target = orc.dequant_weight(packed, s, None, K) + delta
        back = orc.dequant_weight(p2, s2, None, K)
        bound = np.broadcast_to(s2, (K, N))
    err = np.abs(back.astype(np.float64) - target.astype(np.float64))
    assert np.all(err <= bound * (0.5 + 2.0**-20) + 1e-12)
    assert not np.array_equal(p2, packed)              # the delta changed some codes
