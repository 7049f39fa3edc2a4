/*
 * Exhaustive check of the fp8 kernels' fast quotient (test helper, CPU only).
 *
 * The fp8 dispatch kernels divide each element x of a 128-element group by
 * the group scale s = fl(amax / 448) without an element-wise division when
 * amax >= 2^-96: with y = fl(1 / s) (correctly rounded), they compute
 * q0 = fl(x * y), r = fma(-q0, s, x) and q = fma(r, y, q0) (Markstein's
 * correction step), keeping the sign of x = +-0 explicitly.  The definition
 * is e4m3fn_rne(clamp(fl(x / s), -448, 448)).
 *
 * x is bf16 and amax is a bf16 value with |x| <= amax, so the inputs form a
 * finite set.  This program walks all of it (about 1.06e9 pairs) and counts
 * the pairs whose e4m3fn code differs between the two quotients (codes from
 * the oracle's codec), separately for amax >= 2^-96 and below.
 * Exit status 0 iff no pair with amax >= 2^-96 differs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t oracle_e4m3fn_rne(float v);

static float bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float clampq(float v) { return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v); }

int main(void)
{
    const float threshold = 0x1p-96f;
    long long pairs = 0, bad_fast = 0, bad_below = 0;
    for (uint32_t ab = 1; ab < 0x7F80; ++ab) {          /* every positive finite bf16 amax */
        const float a = bf((uint16_t)ab);
        volatile float s = a / 448.0f;
        volatile float y = 1.0f / s;
        for (uint32_t xb = 0; xb <= ab; ++xb) {           /* every bf16 0 <= x <= amax */
            const float x = bf((uint16_t)xb);
            for (int sg = 0; sg < 2; ++sg) {
                const float xx = sg ? -x : x;
                const float exact = xx / s;
                const float q0 = xx * y;
                float q = fmaf(fmaf(-q0, s, xx), y, q0);
                if (xx == 0.0f)
                    q = xx;
                ++pairs;
                if (oracle_e4m3fn_rne(clampq(exact)) != oracle_e4m3fn_rne(clampq(q))) {
                    if (a >= threshold)
                        ++bad_fast;
                    else
                        ++bad_below;
                }
            }
        }
    }
    printf("pairs %lld: e4m3 code differs for %lld with amax >= 2^-96 and %lld below\n", pairs,
           bad_fast, bad_below);
    return bad_fast == 0 ? 0 : 1;
}
