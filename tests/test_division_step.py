"""The division step of the rounding-mode attention (host CPU, no GPU).

The matrix-core prefill attention's second pass in the rounding mode weights V
with f16(e / L), each probability e = e^(s - M) divided by its row's span sum L
("What a Llama model computes, and why", section 8). The kernel takes the
quotient from the correctly rounded reciprocal r = 1/L, computed once per row:
q = e r, then q + (e - q L) r with the residual from a fused multiply-add
(Markstein's division step), and rounds that fp32 value to binary16. This
test checks, in IEEE fp32 on the host (C, fused multiply-add, no contraction
elsewhere), that the step equals the correctly rounded quotient for random
pairs from the softmax's range (0 <= e <= 1 <= L) wherever the quotient is
2^-100 or more (below about 2^-120 the residual underflows and the step can be
an ulp off), and that every difference lies below 2^-25, where both values
round to the same binary16 value (0).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t xr(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(void) {
    long bad_normal = 0, bad_f16 = 0, n = 0;
    for (long it = 0; it < 20000000; it++) {
        const float L = 1.f + (float)(xr() % 4096000000ull) / 1000000.f;
        float e;
        switch (xr() % 4) {
            case 0: e = (float)(xr() >> 40) / (float)(1ull << 24); break;
            case 1: e = ldexpf((float)(xr() >> 40) / (float)(1ull << 24), -(int)(xr() % 120)); break;
            case 2: e = 1.f; break;
            default: { const uint32_t b = (uint32_t)(xr() & 0x3f7fffffu); memcpy(&e, &b, 4); }
        }
        const float r = 1.f / L;
        const float q0 = e * r;
        const float q = fmaf(fmaf(-q0, L, e), r, q0);
        const float want = e / L;
        n++;
        /* exact wherever the residual e - q L (about 2^-24 of e) is a normal
           number, which holds for quotients of 2^-100 and more */
        if (q != want && fabsf(want) >= 0x1p-100f) bad_normal++;
        /* a difference anywhere must sit below half of binary16's smallest
           subnormal (2^-24), where both round to 0 in binary16 */
        if (q != want && fmaxf(fabsf(q), fabsf(want)) >= 0x1p-25f) bad_f16++;
    }
    printf("%ld %ld %ld\n", n, bad_normal, bad_f16);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_step_matches_the_quotient():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div.c"), os.path.join(d, "div")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
        n, bad_normal, bad_f16 = map(int, subprocess.run([exe], check=True, capture_output=True,
                                                          text=True).stdout.split())
    assert n == 20000000
    assert bad_normal == 0, f"{bad_normal} quotients of 2^-100 or more differ"
    assert bad_f16 == 0, f"{bad_f16} binary16 probabilities differ"
