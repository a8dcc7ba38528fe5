"""The prologue divides without divide instructions; these checks run the same
float32/float64 steps on the CPU (IEEE fma, round to nearest) against IEEE
division.

- h / s: q0 = h * r, q = fma(fma(-s, q0, h), r, q0) with r = RN(1/s), for s in
  [2^-100, 2^100] (tokens outside that range take a divide instruction).
- s = amax / qmax: the same correction of amax * RN(1/qmax), for every finite
  amax >= 0 (sampled here; a one-off run over all 2^31 of them found no
  mismatch for qmax = 127 or 7).
- the RMSNorm mean ss / K in float64: the correction of ss * RN(1/K).

Markstein's correction step (one fma for the exact remainder, one to correct
the product) gives the correctly rounded quotient when the reciprocal is
correctly rounded; the vla.cpp FoldQuant page's SYCL commit is why the
divides must be correctly rounded (the codes depend on them)."""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
int main(void) {
    long bad_s = 0, n_s = 0, bad_q = 0, n_q = 0, bad_m = 0, n_m = 0;
    const int qs[2] = {127, 7};
    for (int qi = 0; qi < 2; ++qi) {
        const float q = (float)qs[qi];
        volatile float one = 1.0f;
        const float rq = one / q;
        for (uint64_t u = 0; u <= 0x7f7fffffull; u += 97) {          /* every 97th finite amax >= 0 */
            const float a = f_of((uint32_t)u), s0 = a * rq;
            const float s = fmaf(fmaf(-s0, q, a), rq, s0);
            bad_s += u_of(s) != u_of(a / q); ++n_s;
        }
        for (int e = -126; e < 128; ++e)                             /* around every power of two */
            for (int d = -64; d <= 64; ++d) {
                const float a = f_of(u_of(ldexpf(1.0f, e)) + d);
                if (!(a >= 0.0f) || isinf(a)) continue;
                const float s0 = a * rq, s = fmaf(fmaf(-s0, q, a), rq, s0);
                bad_s += u_of(s) != u_of(a / q); ++n_s;
            }
        /* h / s for tokens in the fast range: random and next to the rounding ties */
        for (long i = 0; i < 4000000; ++i) {
            const uint64_t x = next();
            const float s = ldexpf(1.0f + (float)(x & 0xffffff) * 0x1p-24f, (int)((x >> 24) % 201) - 100);
            volatile float onev = 1.0f;
            const float r = onev / s;
            float h;
            if (i & 1) {
                h = ldexpf((float)((int64_t)(x >> 32) % (1 << 24)), -24) * q * s;   /* |h| <= qmax s */
            } else {
                const float k = (float)((int)((x >> 32) % (2 * qs[qi] + 1)) - qs[qi]);
                h = f_of(u_of((k + 0.5f) * s) + (int)((x >> 56) % 5) - 2);       /* near a tie */
            }
            const float q0 = h * r, qq = fmaf(fmaf(-s, q0, h), r, q0);
            bad_q += u_of(qq) != u_of(h / s); ++n_q;
        }
    }
    const int Ks[] = {64, 256, 2048, 3000, 3584, 16384, 18944, 32768, 65536};
    for (int ki = 0; ki < 9; ++ki) {
        const double K = Ks[ki];
        volatile double one = 1.0;
        const double rk = one / K;
        for (long i = 0; i < 400000; ++i) {
            const uint64_t x = next();
            uint64_t bits = (x & 0x000fffffffffffffull) | ((uint64_t)(723 + (x >> 52) % 600) << 52);
            double ss;
            memcpy(&ss, &bits, 8);
            if (i % 3 == 0) ss = (double)((x >> 20) % 100000000) * 0x1p-16;
            const double q0 = ss * rk, m = fma(fma(-q0, K, ss), rk, q0);
            bad_m += memcmp(&m, &(double){ss / K}, 8) != 0; ++n_m;
        }
    }
    printf("%ld %ld %ld %ld %ld %ld\n", bad_s, n_s, bad_q, n_q, bad_m, n_m);
    return 0;
}
"""


def test_markstein_divides_match_ieee_division():
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "mk.c"), os.path.join(d, "mk")
        with open(src, "w") as f:
            f.write(C_SRC)
        flags = ["-O2", "-ffp-contract=off", "-fno-fast-math"]
        r = subprocess.run([cc, *flags, "-mfma", src, "-o", exe, "-lm"], capture_output=True, text=True)
        if r.returncode:  # no hardware fma flag: libm's fma is exact too, only slower
            r = subprocess.run([cc, *flags, src, "-o", exe, "-lm"], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        out = subprocess.run([exe], capture_output=True, text=True, timeout=300).stdout.split()
    bad_s, n_s, bad_q, n_q, bad_m, n_m = map(int, out)
    print(f"scale {n_s} cases, quotient {n_q}, float64 mean {n_m}")
    assert n_s > 40_000_000 and n_q == 8_000_000 and n_m == 3_600_000
    assert (bad_s, bad_q, bad_m) == (0, 0, 0)
