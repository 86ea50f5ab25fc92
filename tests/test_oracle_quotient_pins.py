"""Pins of the oracle's correctly rounded quotients and of step 6's order.

Keras INT4 guide, "How it works": weights and activations are quantized with
round(v / scale) (steps 1-3; INT4 concept entry, section 4.1; hnwysp.cn
article, section 2.1), and the int32 result is dequantized with
(input_scale * per_channel_kernel_scale) (step 6).  The oracle reads these as
one correctly rounded fp32 quotient followed by round-half-to-even, and as
fl(fl(float(acc)) * fl(sx * sw)) followed by fl(y + bias).

The golden files were derived in exact rational arithmetic
(`golden/make_quotient_goldens.py`, which calls neither the oracle nor the HIP
library), on scales that are not powers of two and values at and next to the
half-integers, where a quotient formed with the rounded reciprocal lands on
the other integer, and on dequantization inputs where the other association
orders, or a fused multiply-add of the bias, change the fp32 result.  Each
check below first re-derives its golden in exact arithmetic, then compares
the oracle with it.  `test_oracle_mutants.py` builds the oracle with each of
those slips and shows that one of these checks fails.
"""
import json
import os
from fractions import Fraction as F

import numpy as np

from exact_fp import add32, clamp, div32, fr, mul32, rn32, rne_int, sub32, unh

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _vals(c):
    return [unh(v) for v in c["values"]]


def _sym_expected(vals, divisor, lo, hi):
    a = max(abs(v) for v in vals)
    s = div32(a, divisor)
    return s, [clamp(rne_int(fr(div32(v, s))), lo, hi) for v in vals]


def _pack_signed(codes):
    """Two codes per byte along K, even k in bits 0-3 (two's complement nibbles)."""
    codes = list(codes) + ([0] if len(codes) % 2 else [])
    return [(codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4) for j in range(len(codes) // 2)]


def check_act(orc):
    d = _load("quotient_ties.json")
    for row in d["act_rows"]:
        vals = _vals(row)
        s, codes = _sym_expected(vals, 127, -128, 127)
        assert s == unh(row["scale"]) and codes == row["codes"]
        assert all(codes[i] != row["codes_if_reciprocal"][i] for i in row["discriminating"])
        Xq, sx = orc.quantize_act(np.array([vals], np.float32))
        assert sx[0] == s, "activation scale"
        assert Xq[0].tolist() == codes, "activation codes"


def check_sym(orc):
    d = _load("quotient_ties.json")
    for col in d["sym_columns"]:
        vals = _vals(col)
        s, codes = _sym_expected(vals, 7, -8, 7)
        assert s == unh(col["scale"]) and codes == col["codes"]
        assert all(codes[i] != col["codes_if_reciprocal"][i] for i in col["discriminating"])
        packed, sw = orc.quantize_weight_sym(np.array(vals, np.float32)[:, None])
        assert sw[0] == s, "int4 weight scale"
        assert packed[0].tolist() == _pack_signed(codes), "int4 weight codes"


def check_w8(orc):
    d = _load("quotient_ties.json")
    for col in d["w8_columns"]:
        vals = _vals(col)
        s, codes = _sym_expected(vals, 127, -128, 127)
        assert s == unh(col["scale"]) and codes == col["codes"]
        assert all(codes[i] != col["codes_if_reciprocal"][i] for i in col["discriminating"])
        Wq, sw = orc.quantize_weight_w8(np.array(vals, np.float32)[:, None])
        assert sw[0] == s, "int8 weight scale"
        assert Wq[0].tolist() == codes, "int8 weight codes"


def _asym(orc, groups, gsize):
    for grp in groups:
        vals = _vals(grp)
        assert len(vals) == gsize
        lo, hi = min(vals), max(vals)
        s = div32(sub32(hi, lo), 15)
        zp = -rne_int(fr(div32(lo, s)))
        codes = [clamp(rne_int(fr(div32(v, s))) + zp, 0, 15) for v in vals]
        assert s == unh(grp["scale"]) and zp == grp["zero_point"] and codes == grp["codes"]
        if grp["kind"] == "zero_point":
            assert zp != grp["zero_point_if_reciprocal"]
        else:
            assert all(codes[i] != grp["codes_if_slip"][i] for i in grp["discriminating"])
        packed, sc, zr = orc.quantize_weight_asym(np.array(vals, np.float32)[:, None], gsize)
        assert sc[0, 0] == s, "group scale"
        assert zr[0, 0] == zp, "group zero point"
        codes2 = codes + ([0] if len(codes) % 2 else [])
        want = [codes2[2 * j] | (codes2[2 * j + 1] << 4) for j in range(len(codes2) // 2)]
        assert packed[0].tolist() == want, "group codes"


def check_asym_codes(orc):
    d = _load("quotient_ties.json")
    _asym(orc, d["asym_code_groups"], d["asym_group_size"])


def check_asym_zero_points(orc):
    d = _load("quotient_ties.json")
    _asym(orc, d["asym_zero_point_groups"], d["asym_group_size"])


def check_step6(orc):
    d = _load("w4a8_step6_order.json")
    x = np.array([[unh(v) for v in r] for r in d["x"]], np.float32)
    W = np.array([[unh(v) for v in r] for r in d["W"]], np.float32)
    b = np.array([unh(v) for v in d["bias"]], np.float32)
    K, N = W.shape
    # re-derive: steps 1-3 by exact quotients, step 5 as an integer sum, step 6 in order
    sx, xq = _sym_expected(list(x[0]), 127, -128, 127)
    assert [sx] == [unh(v) for v in d["sx"]] and [xq] == d["xq"]
    y, yb = [], []
    for n in range(N):
        sw, wq = _sym_expected(list(W[:, n]), 7, -8, 7)
        assert sw == unh(d["sw"][n])
        acc = sum(p * q for p, q in zip(xq, wq))
        assert acc == d["acc"][0][n]
        assert abs(acc) < 2 ** 24  # float(acc) is exact
        yn = rn32(F(acc) * fr(mul32(sx, sw)))
        y.append(yn)
        yb.append(add32(yn, b[n]))
        assert yn != unh(d["y_if_acc_sx_first"][0][n]) and yn != unh(d["y_if_acc_sw_first"][0][n])
        assert yb[-1] != unh(d["y_bias_if_fma"][0][n])
    assert y == [unh(v) for v in d["y"][0]] and yb == [unh(v) for v in d["y_bias"][0]]
    # the oracle: step 6 alone, and the whole forward with and without bias
    acc = np.array(d["acc"], np.int32)
    sxa = np.array([sx], np.float32)
    swa = np.array([unh(v) for v in d["sw"]], np.float32)
    assert orc.dequant(acc, sxa, swa).view(np.uint32).tolist() == \
        [np.array(y, np.float32).view(np.uint32).tolist()], "dequantization order"
    assert orc.dequant(acc, sxa, swa, b).view(np.uint32).tolist() == \
        [np.array(yb, np.float32).view(np.uint32).tolist()], "bias after dequantization"
    packed, sw = orc.quantize_weight_sym(W)
    assert np.array_equal(sw, swa)
    assert orc.w4a8_linear(x, packed, sw).view(np.uint32).tolist() == \
        [np.array(y, np.float32).view(np.uint32).tolist()], "W4A8 forward"
    assert orc.w4a8_linear(x, packed, sw, b).view(np.uint32).tolist() == \
        [np.array(yb, np.float32).view(np.uint32).tolist()], "W4A8 forward with bias"


CHECKS = {
    "act": check_act,
    "sym": check_sym,
    "w8": check_w8,
    "asym_codes": check_asym_codes,
    "asym_zero_points": check_asym_zero_points,
    "step6": check_step6,
}


def test_act_quotient_ties(orc):
    check_act(orc)


def test_sym_weight_quotient_ties(orc):
    check_sym(orc)


def test_w8_weight_quotient_ties(orc):
    check_w8(orc)


def test_asym_code_quotient_ties(orc):
    check_asym_codes(orc)


def test_asym_zero_point_quotient_ties(orc):
    check_asym_zero_points(orc)


def test_step6_association_order_and_bias(orc):
    check_step6(orc)


def test_goldens_discriminate():
    """Every golden case separates the definition from its slip (re-derived
    here, not read from the file): the quotient cases' scales are not powers of
    two, and the slips change the result."""
    d = _load("quotient_ties.json")
    for key, div in (("act_rows", 127), ("sym_columns", 7), ("w8_columns", 127)):
        for c in d[key]:
            s = unh(c["scale"])
            m, _ = np.frexp(s)
            assert m != 0.5
            vals = _vals(c)
            rs = rn32(1 / fr(s))
            for i in c["discriminating"]:
                assert rne_int(fr(div32(vals[i], s))) != rne_int(fr(mul32(vals[i], rs)))
