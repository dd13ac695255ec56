/* Exhaustive host check of the bf16 quotient the quantise kernels use.
 *
 * The kernels quantise x to E4M3FN as the code of the float quotient x / scale
 * (scale = amax / 448, both float divisions correctly rounded).  For bf16 x
 * they form the quotient without a division per element: r = 1 / scale
 * (correctly rounded), q0 = x * r, then the FMA correction step of Markstein's
 * division, q = q0 + r * (x - q0 * scale) (two fused multiply-adds), with the
 * sign of x.  This program checks, for every positive finite bf16 amax whose
 * scale lies in [2^-100, 2^126] and every finite bf16 x with |x| <= amax, that
 * q equals the correctly rounded x / scale bit for bit wherever either value is
 * at least 2^-11 in magnitude (below 2^-10 the E4M3FN code is a signed zero)
 * and has its sign elsewhere.  Exit status 0 when no pair fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t float_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(void) {
    long long pairs = 0, failures = 0, scales = 0;
#pragma omp parallel for reduction(+ : pairs, failures, scales) schedule(dynamic, 64)
    for (int ab = 1; ab < 0x7F80; ++ab) { /* positive finite bf16 amax */
        const float amax = bf16_value((uint16_t)ab);
        const float scale = amax / 448.0f;
        if (!(scale >= 0x1p-100f && scale <= 0x1p+126f)) continue;
        ++scales;
        const float r = 1.0f / scale;
        for (int sign = 0; sign < 2; ++sign) {
            for (int xb = 0; xb <= ab; ++xb) { /* every finite bf16 with |x| <= amax */
                const float x = bf16_value((uint16_t)(xb | (sign << 15)));
                const float exact = x / scale;
                const float q0 = x * r;
                const float q = copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);
                ++pairs;
                const int big = fabsf(q) >= 0x1p-11f || fabsf(exact) >= 0x1p-11f;
                const int ok = big ? float_bits(q) == float_bits(exact) : signbit(q) == signbit(exact);
                if (!ok) {
                    if (failures < 8) printf("x=%a scale=%a quotient=%a kernel=%a\n", x, scale, exact, q);
                    ++failures;
                }
            }
        }
    }
    printf("scales %lld pairs %lld failures %lld\n", scales, pairs, failures);
    return failures != 0;
}
