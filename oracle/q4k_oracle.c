/*
 * q4k_oracle.c -- plain, slow, obviously-correct CPU oracle for the Q4_K
 * weight-only matmul  Y = X . Wdq^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library; its format knowledge is written out here on
 * its own.
 *
 * What it follows.  The genie-ai-runtime README ("At a glance") says the
 * engine loads GGUF models only and is validated on Qwen3-4B-Q4_K_M, and that
 * its hot kernels are an INT4 dequant-fused GEMV and a "tensor-core MMQ Q4_K
 * prefill" matmul.  The pages never define Q4_K itself; this file states the
 * public GGUF Q4_K super-block and its dequantisation rule:
 *
 *   one block = 256 weights in 144 bytes
 *     bytes   0..1   d      (IEEE binary16, little-endian)
 *     bytes   2..3   dmin   (IEEE binary16, little-endian)
 *     bytes   4..15  scales (eight 6-bit sub-block scales sc_j and eight 6-bit
 *                            sub-block mins m_j, packed as in unpack_scale_min)
 *     bytes  16..143 qs     (256 unsigned 4-bit quants q_i, see quant_at)
 *   weight i of the block lies in sub-block s = i / 32 and is
 *     w_i = d * sc_s * q_i - dmin * m_s.
 *
 * Precision.  w is produced in fp32 (one correct rounding of the exact value),
 * then the contraction is accumulated in fp64, and so is A = sum |w * x|,
 * which scales the per-element tolerance.
 *
 * Special values: a d or dmin that is Inf/NaN propagates per IEEE through
 * double arithmetic; finite inputs take the exact integer route.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 256          /* weights per super-block                  */
#define BLOCK_BYTES 144 /* 2 + 2 + 12 + 128                           */

/* ---------------------------------------------------------------- scalars */

/* IEEE 754 binary16 bit pattern -> double, from the format definition:
 * sign bit 15, 5-bit biased exponent (bias 15) in bits 10..14, 10-bit
 * fraction.  Exponent 0 encodes zero/subnormals f * 2^-24, exponent 31
 * encodes Inf (f == 0) or NaN.  Every binary16 value is exact in double. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
float oracle_bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even, from the definition:
 * keep the upper 16 bits, and look at the 16 bits dropped.  NaN stays a
 * (quiet) NaN with its sign. */
uint16_t oracle_float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t trunc = u >> 16;      /* candidate nearer to zero           */
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u)
        return (uint16_t)(trunc + 1);   /* above the midpoint: away      */
    if (dropped < 0x8000u)
        return (uint16_t)trunc;         /* below the midpoint: toward    */
    return (uint16_t)(trunc + (trunc & 1u)); /* tie: the even candidate  */
}

/* ------------------------------------------------------------ block format */

/* The 6-bit scale and min of sub-block j (0..7) from the 12 scale bytes.
 * Sub-blocks 0..3 keep both fields whole in the low six bits of bytes j and
 * j+4.  Sub-blocks 4..7 keep their low four bits in byte j+4 (scale in the low
 * nibble, min in the high nibble) and their top two bits in the otherwise
 * unused bits 6..7 of bytes j-4 (scale) and j (min). */
static void unpack_scale_min(const uint8_t *s, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* The 4-bit quant of weight i (0..255).  Each run of 64 weights uses 32
 * bytes of qs: the first 32 weights of the run in the low nibbles, the next
 * 32 in the high nibbles, byte by byte. */
static int quant_at(const uint8_t *qs, int i) {
    uint8_t byte = qs[32 * (i / 64) + (i % 32)];
    return ((i / 32) % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
}

static uint16_t load_u16le(const uint8_t *p) {
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* Exposed for the tests: every field of every block. */
void oracle_unpack_fields(const uint8_t *blocks, long nblocks, uint8_t *q,
                          uint8_t *sc, uint8_t *m, uint16_t *d_bits,
                          uint16_t *dmin_bits) {
    for (long b = 0; b < nblocks; ++b) {
        const uint8_t *blk = blocks + b * BLOCK_BYTES;
        if (d_bits) d_bits[b] = load_u16le(blk);
        if (dmin_bits) dmin_bits[b] = load_u16le(blk + 2);
        for (int j = 0; j < 8; ++j) {
            int s, mm;
            unpack_scale_min(blk + 4, j, &s, &mm);
            sc[b * 8 + j] = (uint8_t)s;
            m[b * 8 + j] = (uint8_t)mm;
        }
        for (int i = 0; i < QK; ++i)
            q[b * QK + i] = (uint8_t)quant_at(blk + 16, i);
    }
}

/* One weight, rounded once to fp32.
 * Every finite binary16 value is an integer multiple of 2^-24, so
 * d*sc*q - dmin*m == (D*sc*q - DM*m) * 2^-24 exactly, with D = d*2^24 and
 * DM = dmin*2^24 integers below 2^40; the integer difference is below 2^51
 * in magnitude and fits int64 exactly.  Converting that integer to float
 * rounds once (round-to-nearest-even), and the scaling by 2^-24 is exact
 * (results are 0 or at least 2^-24 in magnitude, far above the binary32
 * normal range floor), so the result is RN_fp32 of the exact value. */
static float dequant_one(double d, double dmin, int sc, int q, int m) {
    if (!isfinite(d) || !isfinite(dmin))
        return (float)(d * sc * q - dmin * m);
    int64_t D = (int64_t)ldexp(d, 24);
    int64_t DM = (int64_t)ldexp(dmin, 24);
    int64_t exact = D * sc * q - DM * m;
    return ldexpf((float)exact, -24);
}

static void dequant_block(const uint8_t *blk, float *w) {
    double d = oracle_half_to_double(load_u16le(blk));
    double dmin = oracle_half_to_double(load_u16le(blk + 2));
    for (int i = 0; i < QK; ++i) {
        int sc, m;
        unpack_scale_min(blk + 4, i / 32, &sc, &m);
        w[i] = dequant_one(d, dmin, sc, quant_at(blk + 16, i), m);
    }
}

/* w[256 * nblocks] in fp32. */
void oracle_dequant_f32(const uint8_t *blocks, long nblocks, float *w) {
#pragma omp parallel for schedule(static)
    for (long b = 0; b < nblocks; ++b)
        dequant_block(blocks + b * BLOCK_BYTES, w + b * QK);
}

/* bf16 of the fp32 weight: the value a bf16 tile of the weight holds. */
void oracle_dequant_bf16(const uint8_t *blocks, long nblocks, uint16_t *w) {
#pragma omp parallel for schedule(static)
    for (long b = 0; b < nblocks; ++b) {
        float tmp[QK];
        dequant_block(blocks + b * BLOCK_BYTES, tmp);
        for (int i = 0; i < QK; ++i)
            w[b * QK + i] = oracle_float_to_bf16_rne(tmp[i]);
    }
}

/* ------------------------------------------------------------ contraction */

/* Y[m][n] = sum_k w32[n][k] * x[m][k]   and   A[m][n] = sum_k |w32 * x|,
 * both accumulated in fp64 in increasing k.
 *   W: N rows of K/256 blocks (row n = output feature n), contiguous.
 *   X: M x K bfloat16 bit patterns, row-major.
 *   Y, A: M x N doubles, row-major (A may be NULL).
 * Rows of W are independent; threads split them.  Returns 0, or -1 when K is
 * not a positive multiple of 256 or a buffer cannot be allocated. */
int oracle_gemm(const uint8_t *W, const uint16_t *X, double *Y, double *A,
                long M, long N, long K) {
    if (K <= 0 || K % QK) return -1;
    long nb = K / QK;
    float *xf = (float *)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xf) return -1;
    for (long i = 0; i < M * K; ++i) xf[i] = oracle_bf16_to_float(X[i]);
    int failed = 0;
#pragma omp parallel
    {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)K);
        if (!wrow) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (long n = 0; n < N; ++n) {
            if (!wrow) continue;
            for (long b = 0; b < nb; ++b)
                dequant_block(W + (n * nb + b) * BLOCK_BYTES, wrow + b * QK);
            for (long mi = 0; mi < M; ++mi) {
                const float *x = xf + mi * K;
                double acc = 0.0, aacc = 0.0;
                for (long k = 0; k < K; ++k) {
                    double p = (double)wrow[k] * (double)x[k];
                    acc += p;
                    aacc += fabs(p);
                }
                Y[mi * N + n] = acc;
                if (A) A[mi * N + n] = aacc;
            }
        }
        free(wrow);
    }
    free(xf);
    return failed ? -1 : 0;
}

/* Threads an OpenMP region of the oracle uses (for the CPU baseline). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
