/*
 * Exhaustive check of the fp8 kernels' fast group arithmetic (test helper,
 * CPU only).
 *
 * For a 128-element group with amax >= 2^-96 the fp8 dispatch kernels avoid
 * every division:
 *   scale      s = fl(amax / 448): with t = amax * 2^-6 (exact) and
 *              c = fl(1/7), q0 = fl(t * c), r = fma(-q0, 7, t) (exact),
 *              s = fma(r, c, q0);
 *   reciprocal y = fl(1 / s): from v_rcp_f32's result r0 (within 1 ulp of
 *              1/s, so one of the two binary32 neighbours of 1/s),
 *              e = fma(-s, r0, 1), y = fma(e, r0, r0);
 *   quotient   q = fma(-fma(q0, s, -x), y, q0) with q0 = fl(x * y)
 *              (Markstein's correction step with the residual negated: the
 *              exact residual q0*s - x is computed, and its negation enters
 *              the second fma as a source modifier; for x = +-0 the
 *              residual is +0 and the result keeps the sign of x);
 *   code       the kernels convert q without clamping it: the conversion
 *              instruction rounds every magnitude up to 464 to 448 (NaN
 *              only above 464), which equals e4m3fn_rne(clamp(q)) as long
 *              as |q| <= 464.  This program checks that bound (the largest
 *              |q| is printed) and compares e4m3fn_rne(clamp(q)).
 * The definitions are s = fl(amax / 448), y = fl(1 / s) and
 * e4m3fn_rne(clamp(fl(x / s), -448, 448)).
 *
 * amax and x are bf16 with |x| <= amax, so the inputs form a finite set.
 * This program walks all of it: every positive finite bf16 amax for the scale
 * and the reciprocal (both neighbours of 1/s as the rcp result), and every
 * pair (x, amax), about 1.06e9, comparing e4m3fn codes (from the oracle's
 * codec), counted separately for amax >= 2^-96 and below.
 * Exit status 0 iff nothing differs for amax >= 2^-96.
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

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float clampq(float v) { return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v); }

static float fast_scale(float a)
{
    const float c = 1.0f / 7.0f;
    const float t = a * 0x1p-6f;
    const float q0 = t * c;
    return fmaf(fmaf(-q0, 7.0f, t), c, q0);
}

static float corrected_rcp(float s, float r0) { return fmaf(fmaf(-s, r0, 1.0f), r0, r0); }

int main(void)
{
    const float threshold = 0x1p-96f;
    long long pairs = 0, bad_fast = 0, bad_below = 0, bad_scale = 0, bad_rcp = 0, groups = 0;
    float qmax = 0.0f;                 /* largest |q| with amax >= 2^-96 */
    for (uint32_t ab = 1; ab < 0x7F80; ++ab) {          /* every positive finite bf16 amax */
        const float a = bf((uint16_t)ab);
        volatile float s = a / 448.0f;
        volatile float y = 1.0f / s;
        if (a >= threshold) {
            ++groups;
            if (bits(fast_scale(a)) != bits(s))
                ++bad_scale;
            /* 1/s lies strictly between y and the neighbour on the side the
               residual points to: both are possible v_rcp_f32 results */
            const float res = fmaf(-s, y, 1.0f);
            const float other = nextafterf(y, res > 0.0f ? INFINITY : 0.0f);
            if (bits(corrected_rcp(s, y)) != bits(y) ||
                (res != 0.0f && bits(corrected_rcp(s, other)) != bits(y)))
                ++bad_rcp;
        }
        for (uint32_t xb = 0; xb <= ab; ++xb) {           /* every bf16 0 <= x <= amax */
            const float x = bf((uint16_t)xb);
            for (int sg = 0; sg < 2; ++sg) {
                const float xx = sg ? -x : x;
                const float exact = xx / s;
                const float q0 = xx * y;
                /* the residual through a volatile: the compiler must not
                   fold the negation back into the first fma (which would
                   change the sign of a zero residual) */
                volatile float r = fmaf(q0, s, -xx);
                const float q = fmaf(-r, y, q0);
                ++pairs;
                if (a >= threshold && fabsf(q) > qmax)
                    qmax = fabsf(q);
                if (oracle_e4m3fn_rne(clampq(exact)) != oracle_e4m3fn_rne(clampq(q))) {
                    if (a >= threshold)
                        ++bad_fast;
                    else
                        ++bad_below;
                }
            }
        }
    }
    printf("groups %lld with amax >= 2^-96: scale differs for %lld, reciprocal for %lld\n", groups,
           bad_scale, bad_rcp);
    printf("pairs %lld: e4m3 code differs for %lld with amax >= 2^-96 and %lld below\n", pairs,
           bad_fast, bad_below);
    printf("largest |q| with amax >= 2^-96: %.9g (448 + 2^-15 = %.9g)\n", qmax, 448.0 + 0x1p-15);
    return bad_fast == 0 && bad_scale == 0 && bad_rcp == 0 && qmax <= 464.0f ? 0 : 1;
}
