/* Exhaustive check of the FP8 quantiser's quotient (CPU, plain C).
 *
 * The pack kernel computes x / scale, with scale = RN(amax / 448) per
 * 128-channel block, as q1 = copysign(fma(fma(-q0, scale, x), r, q0), x) with
 * q0 = RN(x * r) and r = RN(1 / scale) when amax >= 2^-64, and then encodes q1
 * as OCP E4M3 with round-to-nearest-even and saturation.  The method's
 * definition encodes RN(x / scale) instead.  This program walks every positive
 * finite bf16 amax in [lo_bits, hi_bits) and every bf16 x with 0 <= x <= amax
 * and counts the pairs whose E4M3 codes differ.  For x != 0 the encoding and
 * both quotients are odd in x (RN and fma are odd), so negative x follow; at
 * x = -0 the fma's +0 + -0 = +0 breaks that, so both zeros are checked for
 * every amax, bit for bit.  The encoder here is written from the format:
 * bias 7, 3 significand bits, subnormal step 2^-9, largest 448.
 *
 * usage: quotient_check LO_BITS HI_BITS   -> prints "checked N mismatches M"
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* E4M3 code of v >= 0, nearest with ties to the even code, saturating at 448. */
static int e4m3_code(float v) {
    const double d = v;
    if (d >= 464.0) return 0x7E;                      /* 464 is the midpoint of 448 and the first non-finite step */
    if (d < 0x1p-6) return (int)nearbyint(d * 512.0);  /* subnormals (and 2^-6 itself when it rounds up) */
    int e = (int)floor(log2(d));
    if (ldexp(1.0, e) > d) e--;
    if (ldexp(1.0, e + 1) <= d) e++;
    int m = (int)nearbyint((d / ldexp(1.0, e) - 1.0) * 8.0);
    if (m == 8) {
        e++;
        m = 0;
    }
    const int c = ((e + 7) << 3) | m;
    return c > 0x7E ? 0x7E : c;
}

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    const int lo = atoi(argv[1]), hi = atoi(argv[2]);
    long long checked = 0, mismatches = 0;
    for (int ab = lo; ab < hi; ++ab) {
        const float amax = from_bf16((uint16_t)ab);
        if (!(amax >= 0x1p-64f) || isinf(amax) || isnan(amax)) continue;
        volatile float scale = amax / 448.0f;
        volatile float r = 1.0f / scale;
        for (int xb = 0; xb <= ab; ++xb) {
            const float x = from_bf16((uint16_t)xb);
            const float q = x / scale;
            const float q0 = x * r;
            const float q1 = copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);
            ++checked;
            if (bits_of(q1) != bits_of(q) && e4m3_code(q1) != e4m3_code(q)) ++mismatches;
        }
        for (int zb = 0; zb < 2; ++zb) {            /* +0 and -0: the sign decides the code */
            const float x = from_bf16((uint16_t)(zb ? 0x8000 : 0x0000));
            const float q = x / scale;
            const float q0 = x * r;
            const float q1 = copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);
            ++checked;
            if (bits_of(q1) != bits_of(q)) ++mismatches;
        }
    }
    printf("checked %lld mismatches %lld\n", checked, mismatches);
    return 0;
}
