/* kv_oracle.c -- CPU oracle for the FP16 <-> INT8 KV-cache convert.
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.
 *
 * The genie-ai-runtime README ("Project layout") lists an FP16<->INT8 KV
 * convert among its kernels, and its "At a glance" section says the KV cache
 * is INT8 by default with FP16-ULP-bounded drift.  The pages give no scheme.
 * The reading implemented here (plain symmetric absmax quantisation, one
 * scale per KV vector, i.e. per token and head):
 *
 *   a    = max_i |v_i|                  (fp16 -> fp32 is exact; max is exact)
 *   s    = a / 127                      (fp32, IEEE division, round to nearest)
 *   q_i  = rint(v_i / s)                (fp32 IEEE division, then round half
 *                                        to even; |q_i| <= 127), q_i = 0 if s = 0
 *   v'_i = fp16(fp32(q_i * s))          (the product rounded to fp32, then to
 *                                        fp16 by round-to-nearest-even)
 *
 * Every step is a single IEEE operation, so the codes, the scale and the
 * dequantised values are fixed bit for bit.  Non-finite inputs are outside
 * the contract.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* binary16 bit pattern -> float (exact): sign, 5-bit exponent, 10-bit
 * fraction; exponent 0 is a subnormal (f * 2^-24), 31 is Inf/NaN. */
static float half_bits_to_float(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* float -> binary16 bit pattern, round to nearest, ties to even, written
 * from the definition: find the binary16 neighbours of |x| and pick the
 * nearer (the even one on a tie).  Overflow beyond the largest finite value
 * rounds to infinity once |x| >= 65520 (the midpoint between 65504 and
 * 2^16). */
uint16_t oracle_float_to_half_rne(float x) {
    if (isnan(x)) return 0x7E00;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);            /* exact */
    if (a >= 65520.0) return sign | 0x7C00;
    /* spacing of binary16 values around a: 2^-24 below 2^-14, else
     * 2^(floor(log2 a) - 10) */
    double ulp;
    if (a < ldexp(1.0, -14)) {
        ulp = ldexp(1.0, -24);
    } else {
        int e;
        frexp(a, &e);                      /* a = m * 2^e, 0.5 <= m < 1 */
        ulp = ldexp(1.0, e - 1 - 10);
    }
    double lo = floor(a / ulp) * ulp;      /* exact in double */
    double hi = lo + ulp;
    double pick;
    if (a - lo < hi - a)
        pick = lo;
    else if (a - lo > hi - a)
        pick = hi;
    else
        pick = fmod(lo / ulp, 2.0) == 0.0 ? lo : hi;
    /* encode pick (a binary16 value, possibly 65504 + ulp = 2^16 -> Inf) */
    if (pick >= 65536.0) return sign | 0x7C00;
    if (pick < ldexp(1.0, -14)) return sign | (uint16_t)(pick / ldexp(1.0, -24));
    int e;
    double m = frexp(pick, &e);            /* pick = m * 2^e */
    const int exp16 = e - 1 + 15;
    const int frac = (int)((m * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(exp16 << 10) | (uint16_t)frac;
}

float oracle_half_to_float(uint16_t h) { return half_bits_to_float(h); }

/* Quantise nvec vectors of dim binary16 values (v, row-major) to int8 codes
 * q (same layout) and one fp32 scale per vector. */
void oracle_kv_quant(const uint16_t* v, long nvec, int dim, int8_t* q, float* scale) {
    for (long r = 0; r < nvec; ++r) {
        const uint16_t* vr = v + r * (long)dim;
        float amax = 0.0f;
        for (int i = 0; i < dim; ++i) {
            const float x = fabsf(half_bits_to_float(vr[i]));
            if (x > amax) amax = x;
        }
        const float s = amax / 127.0f;
        scale[r] = s;
        for (int i = 0; i < dim; ++i) {
            float c = 0.0f;
            if (s != 0.0f) c = rintf(half_bits_to_float(vr[i]) / s);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            q[r * (long)dim + i] = (int8_t)c;
        }
    }
}

/* Dequantise: v'_i = fp16(fp32(q_i * s)). */
void oracle_kv_dequant(const int8_t* q, const float* scale, long nvec, int dim, uint16_t* v) {
    for (long r = 0; r < nvec; ++r) {
        const float s = scale[r];
        for (int i = 0; i < dim; ++i) {
            const float p = (float)q[r * (long)dim + i] * s;
            v[r * (long)dim + i] = oracle_float_to_half_rne(p);
        }
    }
}
