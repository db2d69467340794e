/* Build-time generator of the bf16 GELU-tanh lookup table used by the GPU
 * kernels (65536 entries, one per bf16 bit pattern).
 *
 * GELU, tanh form (Hendrycks & Gimpel, "Gaussian Error Linear Units"):
 *     g(z) = z/2 * (1 + tanh(u)),   u = sqrt(2/pi) * (z + 0.044715 z^3).
 *
 * The table holds GELU as evaluated in binary64 and rounded once to bf16
 * (round to nearest even), the same value the device's own evaluation gives.
 * For |z| >= 2^-100 that value is the correctly rounded one: the generator
 * evaluates z / (1 + exp(-2u)) in binary128 (__float128, libquadmath) and
 * checks that the result is far enough from the bf16 rounding midpoint for
 * the rounding to be certain (relative distance above 2^-90, against an
 * evaluation error below 2^-100); an entry that fails the check is printed
 * and the generator exits non-zero, which fails the build.  For |z| < 2^-100,
 * |2u| < 2^-99, so binary64 rounds 1 + exp(-2u) to exactly 2 and the value is
 * z/2 exactly; for the 256 inputs with |z| < 2^-125 that is a bf16 rounding
 * midpoint and goes to the even neighbour (the exact GELU lies within a
 * relative 2e-38 of it, on the side of larger magnitude for z > 0).
 *
 * Non-finite inputs (not valid kernel inputs) map to the limits: NaN -> quiet
 * NaN, +inf -> +inf, -inf -> -0.
 *
 * Usage: gen_gelu_table OUT.inc   (writes 65536 comma-separated hex values)
 */
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t float_bits_hi(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Rounds the non-negative binary128 value v to bf16 (nearest, ties to even).
 * Unless v is exact, sets *certain to 0 if v lies within a relative 2^-90 of a
 * rounding midpoint. */
static uint16_t round_to_bf16(__float128 v, int exact, int* certain) {
    *certain = 1;
    if (v == 0) return 0;
    int e;
    frexpq(v, &e); /* v = m * 2^e, m in [0.5, 1) */
    /* bf16: 8 significant bits for normal values (e - 1 >= -126); fixed
     * spacing 2^-133 below that. */
    int qexp = (e - 1 >= -126) ? e - 8 : -133;
    __float128 n = ldexpq(v, -qexp); /* exact: a power-of-two scaling */
    __float128 fl = floorq(n);
    __float128 frac = n - fl;
    __float128 dist = fabsq(frac - 0.5Q);
    if (!exact && dist <= ldexpq(n, -90)) *certain = 0;
    __float128 r;
    if (frac > 0.5Q) r = fl + 1;
    else if (frac < 0.5Q) r = fl;
    else r = (fmodq(fl, 2.0Q) == 0) ? fl : fl + 1;
    /* r * 2^qexp has at most 9 significant bits and is a float exactly
     * (or overflows to +inf past the largest bf16, which z/(1+e) never does) */
    float f = (float)ldexpq(r, qexp);
    return float_bits_hi(f);
}

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT.inc\n", argv[0]);
        return 2;
    }
    FILE* out = fopen(argv[1], "w");
    if (!out) {
        perror(argv[1]);
        return 2;
    }
    const __float128 k = sqrtq(2.0Q / M_PIq);
    int bad = 0;
    for (uint32_t h = 0; h < 65536; ++h) {
        const float zf = bf16_to_float((uint16_t)h);
        const uint16_t sign = (uint16_t)(h & 0x8000u);
        uint16_t y;
        if (isnan(zf)) {
            y = (uint16_t)(h | 0x0040u);
        } else if (isinf(zf)) {
            y = sign ? 0x8000u : 0x7f80u;
        } else {
            const __float128 z = (__float128)zf;
            const __float128 u = k * (z + 0.044715Q * z * z * z);
            const __float128 t = -2 * u;
            __float128 g;
            int exact = 0;
            if (fabsq(z) < 0x1p-100Q) {
                g = z / 2; /* binary64: 1 + exp(-2u) == 2 exactly */
                exact = 1;
            } else if (t > 20000) {
                /* exp(-2u) overflows binary128: |g| < |z| e^-20000, far
                 * below the smallest bf16 subnormal */
                g = 0;
            } else {
                g = z / (1 + expq(t));
            }
            int certain = 1;
            y = (uint16_t)(sign | round_to_bf16(fabsq(g), exact, &certain));
            if (!certain) {
                char buf[64];
                quadmath_snprintf(buf, sizeof buf, "%.36Qe", g);
                fprintf(stderr, "gelu table: rounding of input 0x%04x (g = %s) not certain\n",
                        (unsigned)h, buf);
                bad = 1;
            }
        }
        fprintf(out, "0x%04x,%s", (unsigned)y, (h % 16 == 15) ? "\n" : "");
    }
    if (fclose(out) != 0) {
        perror(argv[1]);
        return 2;
    }
    return bad;
}
