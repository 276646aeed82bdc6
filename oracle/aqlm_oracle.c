/*
 * aqlm_oracle.c -- plain CPU oracle for the additive-quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it; it shares no source, header, table or helper with the GPU library.
 *
 * What it computes (page "AQLM (Additive Quantization for LLMs)", section
 * "Niveau intermediaire"): every row of the weight matrix is cut into groups of
 * 8 consecutive input columns (page "AQLM -- ...", section "Kak eto rabotaet
 * tekhnicheski?": groups of 8, in_group_size), and each group is approximated
 * by the sum of one 8-wide vector taken from each of K codebooks:
 *
 *     w(o, 8j .. 8j+7)  =  C_1[i_1] + C_2[i_2] + ... + C_K[i_K].
 *
 * A codebook is a (number of entries) x (group size) matrix; with B-bit codes
 * it has 2^B entries.  The bitrate is K * log2(entries) / group_size bits per
 * weight (same section, with the worked examples K=2, 65536 entries -> 4 bits
 * and K=2, 256 entries -> 2 bits).
 *
 * Readings taken where the pages are silent (each one is exercised by a test):
 *  - layout: codes [out][in/8][K] row-major, one byte (B=8) or one unsigned
 *    16-bit little-endian word (B=16) per code; codebooks [K][2^B][8] fp16;
 *    x [batch][in] fp16; y [batch][out];
 *  - one set of K codebooks per weight matrix, no scales, no bias;
 *  - the decoded weight is the fp32 left fold  w = C_0 ; w = w + C_k (k = 1..K-1),
 *    starting from C_0's value (so -0 + -0 stays -0);
 *  - y[b][o] = sum over i ascending of (double)W[o][i] * (double)x[b][i], in
 *    double, left unrounded.
 *
 * fp16 <-> fp32 conversions are written from the IEEE 754 binary16 definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0 is
 * subnormal, exponent 31 is Inf/NaN), not taken from any library.
 *
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math).
 * OpenMP splits rows only; each row is computed by one thread in a fixed order,
 * so results do not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 8

/* ORACLE_MUTANT is defined only by the pin-sensitivity test, which compiles a
 * deliberately broken copy of this file to show that the pins catch it. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* ---------------------------------------------------------------- formats */

/* Bits per weight = K * log2(2^B) / group  (page 2, "Niveau intermediaire"). */
double oracle_bits_per_weight(int K, int B, int group)
{
    return (double)K * (double)B / (double)group;
}

/* Bytes of code storage for one out x in matrix: out * (in/8) groups, K codes each. */
int64_t oracle_codes_bytes(int64_t out_features, int64_t in_features, int K, int B)
{
    return out_features * (in_features / ORACLE_GROUP) * (int64_t)K * (int64_t)(B / 8);
}

/* binary16 bit pattern -> float, by the definition of the format. */
float oracle_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);            /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    }
    return (float)(sign ? -v : v);               /* every binary16 value is exact in float */
}

/* float -> binary16 bit pattern, round to nearest, ties to even. */
uint16_t oracle_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0)                             /* halfway between 65504 and 2^16 */
        return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                                 /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                                       /* a in [2^e, 2^(e+1)) */
    if (e < -14)
        e = -14;                                  /* subnormal range shares 2^-24 spacing */
    double q = ldexp(1.0, e - 10);                /* spacing of binary16 values near a */
    double n = a / q;                             /* exact: q is a power of two */
    double fl = floor(n);
    double rem = n - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    double r = fl * q;                            /* rounded magnitude */
    if (r < ldexp(1.0, -14))                      /* subnormal (or smallest normal reached) */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int re;
    double rm = frexp(r, &re);                    /* r = rm * 2^re, rm in [0.5, 1) */
    int biased = re - 1 + 15;
    int frac = (int)(rm * 2048.0) - 1024;
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)frac);
}

/* ----------------------------------------------------------------- decode */

static inline uint32_t code_at(const void *codes, int B, int64_t idx)
{
    if (B == 8)
        return ((const uint8_t *)codes)[idx];
    return ((const uint16_t *)codes)[idx];
}

static int check_args(int64_t out_features, int64_t in_features, int K, int B)
{
    if (out_features < 0 || in_features < 0 || in_features % ORACLE_GROUP)
        return 1;
    if (K < 1 || K > 16 || (B != 8 && B != 16))
        return 1;
    return 0;
}

/* Decode one row o into w[0 .. in-1] (fp32 left fold in codebook order). */
static void decode_row(const void *codes, const uint16_t *codebooks, float *w,
                       int64_t o, int64_t in_features, int K, int B)
{
    const int64_t G = in_features / ORACLE_GROUP;
    const int64_t entries = (int64_t)1 << B;
    for (int64_t j = 0; j < G; ++j) {
        for (int t = 0; t < ORACLE_GROUP; ++t) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
#if ORACLE_MUTANT == 2
                /* planted mistake: the code of group j is read from group j+1 */
                int64_t jj = (j + 1 < G) ? j + 1 : j;
                uint32_t c = code_at(codes, B, (o * G + jj) * K + k);
#else
                uint32_t c = code_at(codes, B, (o * G + j) * K + k);
#endif
#if ORACLE_MUTANT == 3
                /* planted mistake: the 8 entries of a codebook vector reversed */
                uint16_t h = codebooks[((int64_t)k * entries + c) * ORACLE_GROUP + (ORACLE_GROUP - 1 - t)];
#else
                uint16_t h = codebooks[((int64_t)k * entries + c) * ORACLE_GROUP + t];
#endif
                float v = oracle_half_to_float(h);
#if ORACLE_MUTANT == 1
                /* planted mistake: only the first codebook contributes */
                if (k > 0)
                    v = 0.0f * v;
#endif
#if ORACLE_MUTANT == 4
                /* planted mistake: the second codebook is subtracted */
                if (k == 1)
                    v = -v;
#endif
                acc = (k == 0) ? v : acc + v;
            }
            w[j * ORACLE_GROUP + t] = acc;
        }
    }
}

/* Dense fp32 W [out][in] from codes and codebooks.  Returns 0 on success. */
int oracle_decode(const void *codes, const uint16_t *codebooks, float *W,
                  int64_t out_features, int64_t in_features, int K, int B, int nthreads)
{
    if (check_args(out_features, in_features, K, B))
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t o = 0; o < out_features; ++o)
        decode_row(codes, codebooks, W + o * in_features, o, in_features, K, B);
    (void)nthreads;
    return 0;
}

/* Y[b][o] = sum_i W[o][i] * x[b][i] in double, i ascending.  x is fp16 bits. */
int oracle_matvec(const float *W, const uint16_t *x, double *Y,
                  int64_t out_features, int64_t in_features, int64_t batch, int nthreads)
{
    if (out_features < 0 || in_features < 0 || batch < 0)
        return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t o = 0; o < out_features; ++o) {
        const float *w = W + o * in_features;
        for (int64_t b = 0; b < batch; ++b) {
            const uint16_t *xb = x + b * in_features;
            double acc = 0.0;
            for (int64_t i = 0; i < in_features; ++i) {
#if ORACLE_MUTANT == 5
                /* planted mistake: activations read one column off */
                int64_t ii = (i + 1 < in_features) ? i + 1 : i;
                acc += (double)w[i] * (double)oracle_half_to_float(xb[ii]);
#else
                acc += (double)w[i] * (double)oracle_half_to_float(xb[i]);
#endif
            }
            Y[b * out_features + o] = acc;
        }
    }
    (void)nthreads;
    return 0;
}

/*
 * Decode + matvec for a chosen list of rows only, for spot checks at sizes
 * where the dense W would be large.  Yrows[b][r] is the double dot product of
 * decoded row rows[r] with x[b] -- the same arithmetic as oracle_decode
 * followed by oracle_matvec, one row at a time.
 */
int oracle_gemv_rows(const void *codes, const uint16_t *codebooks, const uint16_t *x,
                     const int64_t *rows, int64_t nrows, double *Yrows,
                     int64_t out_features, int64_t in_features, int K, int B,
                     int64_t batch, float *scratch_row, int nthreads)
{
    if (check_args(out_features, in_features, K, B) || nrows < 0 || batch < 0)
        return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= out_features)
            return 1;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t r = 0; r < nrows; ++r) {
#ifdef _OPENMP
        float *w = scratch_row + (int64_t)omp_get_thread_num() * in_features;
#else
        float *w = scratch_row;
#endif
        decode_row(codes, codebooks, w, rows[r], in_features, K, B);
        for (int64_t b = 0; b < batch; ++b) {
            const uint16_t *xb = x + b * in_features;
            double acc = 0.0;
            for (int64_t i = 0; i < in_features; ++i)
                acc += (double)w[i] * (double)oracle_half_to_float(xb[i]);
            Yrows[b * nrows + r] = acc;
        }
    }
    (void)nthreads;
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
