"""Exhaustive CPU checks of two division- and branch-free identities the fused
activation quantizers use in place of the textbook operations (Keras INT4
guide, "How it works", step 3: scale = absmax / 127, code = round(x / scale)).

1. The row scale fl(a / 127) without a division: with y = fl(1/127),
   q = fl(a * y), r = fma(-q, 127, a) (exact), s = fma(r, y, q) is the
   correctly rounded quotient (Markstein's theorem for round-to-nearest),
   checked for every float32 a in [2^-100, 2^128).
2. Round-half-to-even of a quotient t with |t| <= 127.5 by one fp32 add:
   t + 1.5 * 2^23 lies in [2^23, 2^24), where the fp32 spacing is 1, so the
   add rounds t to the nearest integer with ties to even, and the low byte of
   the sum's bit pattern is that integer as an int8 (two's complement), since
   the bit pattern of 1.5 * 2^23 ends in a zero byte; checked for every
   float32 t with |t| <= 127.5.

The checks run as a small C program (gcc, fmaf, no contraction) on the host.
"""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
int main(void) {
    const float y = 1.0f / 127.0f;
    long bad = 0, n = 0;
    for (uint32_t e = 127 - 100; e < 255; ++e)           /* a in [2^-100, 2^128) */
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float a = f((e << 23) | m);
            const float q = a * y, r = fmaf(-q, 127.0f, a), s = fmaf(r, y, q);
            const float t = a / 127.0f;
            ++n;
            if (u(s) != u(t)) { if (bad++ < 3) printf("scale %a: %a vs %a\n", a, s, t); }
        }
    printf("scale: %ld values, %ld mismatches\n", n, bad);
    long bad2 = 0, n2 = 0;
    for (uint32_t sign = 0; sign < 2; ++sign)
        for (uint32_t bits = 0; bits <= 0x42FF0000u; ++bits) {  /* |t| <= 127.5 */
            const float t = f(bits | (sign << 31));
            const uint32_t b = u(t + 12582912.0f);
            const int8_t code = (int8_t)(b & 0xFFu);
            const int8_t want = (int8_t)nearbyintf(t);
            ++n2;
            if (code != want) { if (bad2++ < 3) printf("round %a: %d vs %d\n", t, code, want); }
        }
    printf("round: %ld values, %ld mismatches\n", n2, bad2);
    return (bad || bad2) ? 1 : 0;
}
"""


@pytest.mark.slow
def test_division_free_scale_and_add_rounding(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is needed")
    c = tmp_path / "ident.c"
    exe = tmp_path / "ident"
    c.write_text(SRC)
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                        str(c), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatches" in r.stdout.splitlines()[0] and "0 mismatches" in r.stdout.splitlines()[1]
