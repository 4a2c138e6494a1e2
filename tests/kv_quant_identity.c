/* The int8 KV codes without a division per value: for every binary16 v and
 * every non-negative binary16 a (the vector's max |v|, +Inf included), with
 * s = RN(a / 127) and y = RN(1 / s), compare
 *     rint(v / s)                                   (the definition)
 *     rint(fma(fma(-q0, s, v), y, q0)), q0 = RN(v * y)  (the kernel's form)
 * each clamped to [-127, 127]; a zero or infinite s takes the division in
 * both.  Prints the pairs compared and the mismatches where |v| <= a or v is
 * NaN (the only pairs a vector can produce); exits 1 if there is any. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

static float half_to_float(uint16_t h) {
    const uint32_t sign = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    float f;
    if (e == 0) f = ldexpf((float)m, -24);
    else if (e == 31) f = m ? NAN : INFINITY;
    else f = ldexpf((float)(m | 1024u), (int)e - 25);
    return sign ? -f : f;
}

static int clamp_code(float c) { return (int)fminf(fmaxf(c, -127.0f), 127.0f); }

static int by_division(float v, float s) { return clamp_code(s != 0.0f ? rintf(v / s) : 0.0f); }

static int by_reciprocal(float v, float s, float y) {
    if (!(s != 0.0f && s < INFINITY)) return by_division(v, s);
    volatile float q0 = v * y;   /* rounded on its own, never fused */
    const float r = fmaf(-q0, s, v);
    return clamp_code(rintf(fmaf(r, y, q0)));
}

int main(void) {
    long pairs = 0, bad = 0;
#pragma omp parallel for reduction(+ : pairs, bad) schedule(dynamic, 64)
    for (int a = 0; a <= 0x7C00; ++a) {
        const float amax = half_to_float((uint16_t)a);
        const float s = amax / 127.0f, y = 1.0f / s;
        for (int b = 0; b < 65536; ++b) {
            const float v = half_to_float((uint16_t)b);
            if (!(fabsf(v) <= amax) && !isnan(v)) continue;
            ++pairs;
            if (by_division(v, s) != by_reciprocal(v, s, y)) ++bad;
        }
    }
    printf("pairs %ld mismatches %ld\n", pairs, bad);
    return bad != 0;
}
