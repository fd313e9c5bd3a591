/* Host check of the activation quantisation's quotient (quant_div in the
 * device code): for a token with amax = max |x| and s = fl32(amax / 448),
 * r = fl32(1 / s), the value copysign(fma(fma(-q0, s, x), r, q0), x) with
 * q0 = fl32(x * r) must have the same E4M3 code (round to nearest even,
 * saturating at 448) as the correctly rounded quotient fl32(x / s).
 * Checked for every positive normal bf16 amax >= 2^-64 (smaller ones take the
 * division on the device) taken with the given stride, and every bf16 x with
 * 0 <= x <= amax; a negative x mirrors a positive one.
 *   usage: quant_div_check [amax stride, default 1 = every amax]
 * Prints the counts; exits 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t bits)
{
    const uint32_t u = bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* the E4M3 value v rounds to, exactly (as a double): steps of 2^(e-3) in the
 * binade [2^e, 2^(e+1)), 2^-9 below 2^-6, saturating at 448 */
static double e4m3_round(float v)
{
    double a = fabs((double)v);
    if (a > 448.0) a = 448.0;
    int e;
    frexp(a, &e);
    const double step = (a < 0x1p-6) ? 0x1p-9 : ldexp(1.0, e - 4);
    const double r = rint(a / step) * step;
    return v < 0 ? -r : r;
}

int main(int argc, char** argv)
{
    const unsigned stride = argc > 1 ? (unsigned)atoi(argv[1]) : 1u;
    long long pairs = 0, bad = 0;
    for (uint32_t ab = 0x0080; ab < 0x7F80; ab += stride) {
        volatile float amax = bf16(ab);
        if (!(amax >= 0x1p-64f)) continue;
        volatile float s = amax / 448.0f;
        volatile float r = 1.0f / s;
        for (uint32_t xb = 0; xb <= ab; ++xb) {
            volatile float x = bf16(xb);
            volatile float y = x / s;
            volatile float q0 = x * r;
            volatile float e = fmaf(-q0, s, x);
            volatile float q = copysignf(fmaf(e, r, q0), x);
            ++pairs;
            if (e4m3_round(q) != e4m3_round(y)) {
                if (bad < 5) printf("amax %a x %a: x/s %a, quant_div %a\n", (double)amax, (double)x, (double)y, (double)q);
                ++bad;
            }
        }
    }
    printf("pairs %lld mismatches %lld\n", pairs, bad);
    return bad != 0;
}
