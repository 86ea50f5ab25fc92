#!/usr/bin/env python3
"""Write quotient_ties.json and w4a8_step6_order.json (run from any directory).

The cases are derived in exact rational arithmetic from the definitions the
pages give (Keras INT4 guide, "How it works", steps 1, 3 and 6; INT4 concept
entry, section 4.1; "4-bit Integer Quantization for LLMs", quantization
principle; hnwysp.cn article, section 2.1):

  code  = clamp(rne(fl(v / s)), lo, hi)          (symmetric weights, activations)
  code  = clamp(rne(fl(v / s)) + zp, 0, 15),  zp = 0 - rne(fl(x_min / s))   (groups)
  y     = fl(fl(float(acc)) * fl(sx * sw)),  then fl(y + bias)              (step 6)

where fl() rounds the exact result once to fp32 (ties to even) and rne()
rounds to an integer, ties to even.  Nothing here calls the oracle or the HIP
library.  The inputs are chosen, by a seeded search, so that the plausible
slips fail: a quotient formed as fl(v * fl(1 / s)) lands on the other side of
a half-integer than fl(v / s) (scales are not powers of two), and the
dequantization's association order or a fused multiply-add changes the fp32
result.  Each case records what the slip would give.
"""
import json
import os
import sys
from fractions import Fraction as F

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from exact_fp import (add32, clamp, div32, fr, h, is_pow2, mul32, rn32, rne_int,  # noqa: E402
                      sub32)

INF = np.float32(np.inf)


def recip_code(v, s):
    """rne of the quotient formed with the rounded reciprocal: fl(v * fl(1/s))."""
    return rne_int(fr(mul32(v, rn32(1 / fr(s)))))


def true_code(v, s):
    return rne_int(fr(div32(v, s)))


def near_ties(s, kmin, kmax, ulps=3):
    """Float32 values at and around (k + 1/2) * s for k in [kmin, kmax)."""
    for k in range(kmin, kmax):
        v0 = rn32(F(2 * k + 1, 2) * fr(s))
        yield v0
        up = dn = v0
        for _ in range(ulps):
            up, dn = np.nextafter(up, INF), np.nextafter(dn, -INF)
            yield up
            yield dn


def explain(v, s):
    q = div32(v, s)
    qr = mul32(v, rn32(1 / fr(s)))
    return (f"v = {h(v)}, s = {h(s)}: v/s = {float(fr(v) / fr(s)):.17g} -> fl(v/s) = {h(q)} "
            f"-> code {true_code(v, s)}; fl(1/s) = {h(rn32(1 / fr(s)))}, fl(v*fl(1/s)) = {h(qr)} "
            f"-> {recip_code(v, s)}")


def symmetric_rows(rng, divisor, nrows, per_row, width, amin, amax):
    """Rows (activation rows or weight columns) with absmax a, scale fl(a / divisor)
    and `per_row` values whose correctly rounded quotient and reciprocal
    quotient round to different integers."""
    rows = []
    while len(rows) < nrows:
        a = np.float32(rng.uniform(amin, amax))
        if rng.integers(2):
            a = np.float32(a * np.float32(2.0) ** int(rng.integers(-6, 6)))
        s = div32(a, divisor)
        if is_pow2(s):
            continue
        found = []
        for v in near_ties(s, -divisor, divisor):
            if abs(v) >= a or any(v == f for f in found):
                continue
            if true_code(v, s) != recip_code(v, s):
                found.append(v)
        ups = [v for v in found if true_code(v, s) > recip_code(v, s)]
        dns = [v for v in found if true_code(v, s) < recip_code(v, s)]
        if len(ups) < per_row // 2 or len(dns) < per_row - per_row // 2:
            continue
        pick = list(rng.choice(ups, per_row // 2, replace=False)) + \
            list(rng.choice(dns, per_row - per_row // 2, replace=False))
        sign = -1 if len(rows) % 2 else 1  # every other row has its absmax negative
        vals = [np.float32(sign * a)] + [np.float32(v) for v in pick]
        while len(vals) < width:
            vals.append(np.float32(rng.uniform(-1, 1) * a))
        order = rng.permutation(width)
        vals = [vals[i] for i in order]
        disc = [int(np.where(order == i)[0][0]) for i in range(1, 1 + per_row)]
        rows.append((a, s, vals, disc))
    return rows


def sym_case(rows, divisor, lo, hi):
    out = []
    for a, s, vals, disc in rows:
        codes = [clamp(true_code(v, s), lo, hi) for v in vals]
        slip = [clamp(recip_code(v, s), lo, hi) for v in vals]
        assert all(codes[i] != slip[i] for i in disc)
        out.append({"values": [h(v) for v in vals], "scale": h(s),
                    "codes": codes, "codes_if_reciprocal": slip, "discriminating": disc,
                    "why": explain(vals[disc[0]], s)})
    return out


def asym_code_groups(rng, n, width):
    """Groups (lo < 0 < hi) holding values whose code changes with the reciprocal quotient."""
    out = []
    while len(out) < n:
        lo = np.float32(-rng.uniform(0.05, 2.0))
        hi = np.float32(rng.uniform(0.05, 2.0))
        s = div32(sub32(hi, lo), 15)
        if is_pow2(s):
            continue
        zp = -rne_int(fr(div32(lo, s)))
        found = []
        for v in near_ties(s, -16, 16):
            if not (lo < v < hi) or any(v == f for f in found):
                continue
            c, c2 = clamp(true_code(v, s) + zp, 0, 15), clamp(recip_code(v, s) + zp, 0, 15)
            if c != c2:
                found.append(v)
        if len(found) < 2:
            continue
        pick = list(rng.choice(found, 2, replace=False))
        vals = [lo, hi] + pick
        while len(vals) < width:
            vals.append(np.float32(rng.uniform(float(lo), float(hi))))
        order = rng.permutation(width)
        vals = [vals[i] for i in order]
        disc = [int(np.where(order == i)[0][0]) for i in (2, 3)]
        out.append(asym_group(vals, disc, "code"))
    return out


def asym_zero_groups(rng, n, width):
    """Groups whose zero point changes with the reciprocal quotient fl(lo * fl(1/s))."""
    out = []
    while len(out) < n:
        j = int(rng.integers(0, 7))
        t = -F(2 * j + 1, 2)                    # lo / s near -(j + 1/2)
        lo = np.float32(-rng.uniform(0.05, 2.0))
        hi0 = rn32(fr(lo) * (1 + 15 / t))       # range = 15 s with s = lo / t
        hi = hi0
        hit = None
        for step in range(200):
            for cand in (hi, np.float32(2 * hi0 - hi)):
                s = div32(sub32(cand, lo), 15)
                if is_pow2(s):
                    continue
                if true_code(lo, s) != recip_code(lo, s):
                    hit = cand
                    break
            if hit is not None:
                break
            hi = np.nextafter(hi, INF)
        if hit is None:
            continue
        vals = [lo, hit]
        while len(vals) < width:
            vals.append(np.float32(rng.uniform(float(lo), float(hit))))
        order = rng.permutation(width)
        vals = [vals[i] for i in order]
        out.append(asym_group(vals, [int(np.where(order == 0)[0][0])], "zero_point"))
    return out


def asym_group(vals, disc, kind):
    lo, hi = min(vals), max(vals)
    s = div32(sub32(hi, lo), 15)
    zp = -rne_int(fr(div32(lo, s)))
    zp_slip = -recip_code(lo, s)
    codes = [clamp(true_code(v, s) + zp, 0, 15) for v in vals]
    if kind == "code":
        slip = [clamp(recip_code(v, s) + zp, 0, 15) for v in vals]
        assert all(codes[i] != slip[i] for i in disc)
        why = explain(vals[disc[0]], s) + f"; zero point {zp}"
    else:
        assert zp != zp_slip
        slip = [clamp(true_code(v, s) + zp_slip, 0, 15) for v in vals]
        why = (f"x_min = {h(lo)}, x_max = {h(hi)}: range fl(x_max - x_min) = {h(sub32(hi, lo))}, "
               f"s = fl(range / 15) = {h(s)}; " + explain(lo, s) +
               f"; zero point {zp} (with the reciprocal: {zp_slip})")
    return {"values": [h(v) for v in vals], "scale": h(s), "zero_point": zp,
            "zero_point_if_reciprocal": zp_slip, "codes": codes, "codes_if_slip": slip,
            "kind": kind, "discriminating": disc, "why": why}


def step6_case(rng, K, N):
    """One activation row and N weight columns (int4, per channel) whose outputs
    change with (acc*sx)*sw or (acc*sw)*sx, and whose biased outputs change
    with a fused multiply-add."""
    while True:
        x = [np.float32(v) for v in rng.standard_normal(K) * rng.uniform(0.5, 3.0)]
        ax = max(abs(v) for v in x)
        sx = div32(ax, 127)
        xq = [clamp(true_code(v, sx), -128, 127) for v in x]
        cols, accs, sws, ys, biases, ybs = [], [], [], [], [], []
        for n in range(N):
            for _ in range(400):
                w = [np.float32(v) for v in rng.standard_normal(K) * rng.uniform(0.01, 0.2)]
                aw = max(abs(v) for v in w)
                sw = div32(aw, 7)
                wq = [clamp(true_code(v, sw), -8, 7) for v in w]
                acc = sum(a * b for a, b in zip(xq, wq))
                if acc == 0:
                    continue
                s = mul32(sx, sw)
                y = rn32(F(acc) * fr(s))
                alt1 = mul32(mul32(np.float32(acc), sx), sw)
                alt2 = mul32(mul32(np.float32(acc), sw), sx)
                if y == alt1 or y == alt2:
                    continue
                b = None
                for _ in range(400):
                    bb = np.float32(rng.uniform(-1, 1) * abs(float(y)))
                    if add32(y, bb) != rn32(F(acc) * fr(s) + fr(bb)):
                        b = bb
                        break
                if b is None:
                    continue
                cols.append(w), accs.append(acc), sws.append(sw), ys.append(y)
                biases.append(b), ybs.append(add32(y, b))
                break
            else:
                break
        if len(cols) == N:
            break
    W = [[h(cols[n][k]) for n in range(N)] for k in range(K)]
    alt1 = [h(mul32(mul32(np.float32(a), sx), sw)) for a, sw in zip(accs, sws)]
    alt2 = [h(mul32(mul32(np.float32(a), sw), sx)) for a, sw in zip(accs, sws)]
    fma = [h(rn32(F(a) * fr(mul32(sx, sw)) + fr(b))) for a, sw, b in zip(accs, sws, biases)]
    s0 = mul32(sx, sws[0])
    why = (f"column 0: acc = {accs[0]}, sx = {h(sx)}, sw = {h(sws[0])}; fl(sx*sw) = {h(s0)}, "
           f"fl(acc*fl(sx*sw)) = {h(ys[0])}; fl(fl(acc*sx)*sw) = {alt1[0]}; "
           f"fl(fl(acc*sw)*sx) = {alt2[0]}; bias {h(biases[0])}: fl(y + b) = {h(ybs[0])}, "
           f"fma = {fma[0]}")
    return {"x": [[h(v) for v in x]], "W": W, "bias": [h(b) for b in biases],
            "sx": [h(sx)], "xq": [xq], "sw": [h(v) for v in sws], "acc": [accs],
            "y": [[h(v) for v in ys]], "y_bias": [[h(v) for v in ybs]],
            "y_if_acc_sx_first": [alt1], "y_if_acc_sw_first": [alt2], "y_bias_if_fma": [fma],
            "why": why}


def main():
    rng = np.random.default_rng(20251014)
    act = symmetric_rows(rng, 127, nrows=4, per_row=4, width=12, amin=0.5, amax=40.0)
    sym = symmetric_rows(rng, 7, nrows=4, per_row=2, width=10, amin=0.005, amax=0.5)
    w8 = symmetric_rows(rng, 127, nrows=4, per_row=4, width=12, amin=0.005, amax=0.5)
    quot = {
        "source": ("Keras INT4 guide, 'How it works', steps 1-3 (per-channel int4 weights, "
                   "per-row int8 activations, scale = absmax / 7 and / 127); INT4 concept entry, "
                   "section 4.1 (x_q = round(x / scale) + zero_point; symmetric scale "
                   "max|x| / (2^(b-1) - 1), asymmetric (x_max - x_min) / (2^b - 1)); hnwysp.cn "
                   "article, section 2.1 (Q = round(clamp(v / s, -8, 7))); '4-bit Integer "
                   "Quantization for LLMs', quantization principle (groups, scale and zero point)."),
        "derivation": ("Written by make_quotient_goldens.py in exact rational arithmetic: "
                       "fl(v / s) is the exact quotient rounded once to fp32 (ties to even), the "
                       "code its round-half-to-even integer.  Values sit at or next to the "
                       "half-integers (k + 1/2) * s of scales that are not powers of two, where "
                       "fl(v * fl(1 / s)) rounds to the other integer ('*_if_reciprocal')."),
        "float_encoding": "C99 hexadecimal float text of each fp32 value (Python float.fromhex)",
        "act_rows": sym_case(act, 127, -128, 127),
        "sym_columns": sym_case(sym, 7, -8, 7),
        "w8_columns": sym_case(w8, 127, -128, 127),
        "asym_group_size": 8,
        "asym_code_groups": asym_code_groups(rng, 4, 8),
        "asym_zero_point_groups": asym_zero_groups(rng, 4, 8),
    }
    with open(os.path.join(HERE, "quotient_ties.json"), "w") as f:
        json.dump(quot, f, indent=1)
        f.write("\n")
    step6 = step6_case(rng, K=8, N=4)
    step6.update({
        "source": ("Keras INT4 guide, 'How it works', step 6: the int32 result is dequantized "
                   "with (input_scale * per_channel_kernel_scale), i.e. the parenthesised "
                   "product first, then one multiply with the accumulator; the Dense bias is "
                   "added afterwards."),
        "derivation": ("Written by make_quotient_goldens.py in exact rational arithmetic: "
                       "sx = fl(max|x| / 127), sw = fl(max|w| / 7), codes as in steps 1-3, acc the "
                       "exact integer sum, y = fl(acc * fl(sx * sw)), y_bias = fl(y + b).  The "
                       "'*_if_*' entries are what the other association orders and a fused "
                       "multiply-add of the bias would give; each differs from y."),
        "float_encoding": "C99 hexadecimal float text of each fp32 value (Python float.fromhex)",
    })
    with open(os.path.join(HERE, "w4a8_step6_order.json"), "w") as f:
        json.dump(step6, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
