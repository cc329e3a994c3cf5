/* Exhaustive check of the FP8 quantiser's scale and quotient (CPU, plain C).
 *
 * The method's definition: scale = RN(amax / 448) per 128-channel block, and
 * each channel's code is the OCP E4M3 encoding (round to nearest even,
 * saturating) of RN(x / scale).  The pack kernel, for blocks with
 * amax >= 2^-64, computes instead
 *   scale = fma(fma(-s0, 448, amax), c, s0),  s0 = RN(amax * c),  c = RN(1/448),
 *   q1    = fma(fma(-q0, scale, x), r, q0),   q0 = RN(x * r),     r = RN(1/scale),
 * and encodes q1 with the sign bit of x ORed into the code.  This program
 * walks every positive finite bf16 amax in [lo_bits, hi_bits): it counts the
 * amax whose scale differs from RN(amax / 448) in any bit, then, for every
 * bf16 x with 0 <= x <= amax, the pairs whose E4M3 codes differ.  For x != 0
 * the encoding and both quotients are odd in x (RN and fma are odd, and x's
 * sign is the quotient's), so negative x follow; at x = -0 the fma's
 * +0 + -0 = +0 breaks that, which the ORed sign repairs, so both zeros are
 * checked for every amax, code for code.  The encoder here is written from the
 * format: bias 7, 3 significand bits, subnormal step 2^-9, largest 448.
 *
 * usage: quotient_check LO_BITS HI_BITS
 *        -> prints "checked N mismatches M scale_mismatches S"
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

/* The kernel's code of channel x: the encoding of q1 with x's sign bit. */
static int kernel_code(float q1, float x) { return e4m3_code(fabsf(q1)) | (signbit(x) ? 0x80 : 0); }

/* The definition's code: the encoding of the correctly rounded quotient q. */
static int exact_code(float q) { return e4m3_code(fabsf(q)) | (signbit(q) ? 0x80 : 0); }

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    const int lo = atoi(argv[1]), hi = atoi(argv[2]);
    long long checked = 0, mismatches = 0, scale_mismatches = 0;
    for (int ab = lo; ab < hi; ++ab) {
        const float amax = from_bf16((uint16_t)ab);
        if (!(amax > 0.0f) || isinf(amax) || isnan(amax)) continue;
        volatile float c = 1.0f / 448.0f;
        const float s0 = amax * c;
        const float scale = fmaf(fmaf(-s0, 448.0f, amax), c, s0);
        volatile float exact_scale = amax / 448.0f;
        if (bits_of(scale) != bits_of(exact_scale)) ++scale_mismatches;
        if (!(amax >= 0x1p-64f)) continue;        /* smaller blocks divide in the kernel */
        volatile float r = 1.0f / scale;
        for (int xb = 0; xb <= ab; ++xb) {
            const float x = from_bf16((uint16_t)xb);
            const float q = x / exact_scale;
            const float q0 = x * r;
            const float q1 = fmaf(fmaf(-q0, scale, x), r, q0);
            ++checked;
            if (bits_of(q1) != bits_of(q) && kernel_code(q1, x) != exact_code(q)) ++mismatches;
        }
        for (int zb = 0; zb < 2; ++zb) {            /* +0 and -0: the sign decides the code */
            const float x = from_bf16((uint16_t)(zb ? 0x8000 : 0x0000));
            const float q = x / exact_scale;
            const float q0 = x * r;
            const float q1 = fmaf(fmaf(-q0, scale, x), r, q0);
            ++checked;
            if (kernel_code(q1, x) != exact_code(q)) ++mismatches;
        }
    }
    printf("checked %lld mismatches %lld scale_mismatches %lld\n", checked, mismatches, scale_mismatches);
    return 0;
}
