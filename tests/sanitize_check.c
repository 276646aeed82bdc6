/*
 * Host-side checks of libaqlm_mi355x built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on its host code, with the oracle built the same way
 * (tests/test_sanitizers.py builds and runs it).  No device is touched:
 *   1. argument validation: invalid calls are refused before any device work;
 *   2. the kernel-choice and workspace logic over many shapes, batches, schemes and
 *      workspace sizes (aqlm_workspace_bytes / aqlm_grouped_workspace_bytes /
 *      aqlm_selected_variant / aqlm_variant_supported), with the rule that a workspace of
 *      the queried size selects a kernel and one byte less (when positive) is refused;
 *   3. the host-core kernel (aqlm_cpu_gemv) on small random problems against the
 *      oracle's decode + double matvec (per-token bar 2e-3, the decode rule of page
 *      "AQLM (Additive Quantization for LLMs)", section "Niveau intermediaire").
 * Exit status 0 when every check holds; the sanitizers abort the run on a finding.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "aqlm_mi355x.h"

int oracle_decode(const void *codes, const uint16_t *codebooks, float *W, int64_t out_features,
                  int64_t in_features, int K, int B, int nthreads);
int oracle_matvec(const float *W, const uint16_t *x, double *Y, int64_t out_features,
                  int64_t in_features, int64_t batch, int nthreads);
uint16_t oracle_float_to_half(float f);
double oracle_bits_per_weight(int K, int B, int group);

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

/* fake, well-separated device addresses: nothing here is dereferenced */
#define FAKE(i) ((void *)(uintptr_t)(0x100000000ull * (uint64_t)(i)))

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) {
    /* xorshift64* (Vigna 2016) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545f4914f6cdd1dull;
}
static double next_normal(void) {
    const double u1 = ((next_u64() >> 11) + 1.0) / 9007199254740993.0;
    const double u2 = (next_u64() >> 11) / 9007199254740992.0;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static void check_validation(void) {
    void *c = FAKE(1), *cb = FAKE(2), *x = FAKE(3), *y = FAKE(4), *ws = FAKE(5);
    CHECK(aqlm_gemv(NULL, cb, x, y, 16, 64, 2, 8, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT, "null codes");
    CHECK(aqlm_gemv(c, cb, x, y, 16, 60, 2, 8, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT, "in %% 8");
    CHECK(aqlm_gemm(c, cb, x, y, 16, 64, 9, 8, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT, "K > 8");
    CHECK(aqlm_gemm(c, cb, x, y, 16, 64, 2, 12, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT, "B");
    CHECK(aqlm_gemv(c, cb, x, y, INT64_C(1) << 62, INT64_C(1) << 40, 2, 8, 1, NULL, 0, NULL) ==
              AQLM_ERR_INVALID_ARGUMENT, "overflow");
    CHECK(aqlm_gemv(c, cb, x, c, 16, 64, 2, 8, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT, "y overlaps codes");
    CHECK(aqlm_gemv(c, cb, x, y, 11008, 4096, 2, 8, 1, ws, 64, NULL) == AQLM_ERR_INVALID_ARGUMENT,
          "workspace too small");
    CHECK(strstr(aqlm_last_error(), "too small") != NULL, "message: %s", aqlm_last_error());
    CHECK(aqlm_gemv(c, cb, x, y, 11008, 4096, 2, 8, 1, (char *)ws + 8, 1 << 20, NULL) ==
              AQLM_ERR_INVALID_ARGUMENT, "misaligned workspace");
    CHECK(aqlm_gemv(c, cb, x, y, 11008, 4096, 2, 8, 1, y, 1 << 20, NULL) == AQLM_ERR_INVALID_ARGUMENT,
          "workspace overlaps y");
    CHECK(aqlm_gemv_packed(c, cb, x, y, 4096, 4096, 1, 16, 1, NULL, 0, NULL) == AQLM_ERR_INVALID_ARGUMENT,
          "packed without workspace");
    CHECK(aqlm_gemv_packed_noalloc(c, cb, x, y, 28672, 8192, 2, 8, 2, NULL) == AQLM_ERR_INVALID_ARGUMENT,
          "noalloc beyond its scratch");
    CHECK(aqlm_dequantize(c, cb, y, 2, 16, 64, 2, 8, NULL) == AQLM_ERR_INVALID_ARGUMENT, "w dtype");
    CHECK(aqlm_pack_codebooks(cb, (char *)cb + 64, 1, 16, NULL) == AQLM_ERR_INVALID_ARGUMENT, "overlap");
    CHECK(aqlm_codes_bytes(11008, 4096, 2, 8) == 11272192, "codes bytes");
    CHECK(aqlm_bits_per_weight(2, 16, 8) == 4.0 && oracle_bits_per_weight(2, 16, 8) == 4.0, "bitrate");
    const void *gc[4] = {FAKE(10), FAKE(11), FAKE(12), FAKE(13)};
    const void *gcb[4] = {FAKE(20), FAKE(21), FAKE(22), FAKE(23)};
    void *gy[4] = {FAKE(30), FAKE(31), FAKE(32), FAKE(33)};
    const int64_t outs[4] = {4096, 4096, 4096, 0};
    CHECK(aqlm_gemv_grouped(4, gc, gcb, x, gy, outs, 4096, 2, 8, 1, NULL, 0, NULL) ==
              AQLM_ERR_INVALID_ARGUMENT, "empty grouped matrix");
    CHECK(aqlm_grouped_workspace_bytes(AQLM_OP_GEMV, 5, gc, gcb, x, gy, outs, 4096, 2, 8, 1) == -1,
          "more than 4 matrices");
}

static void check_choice_logic(void) {
    static const int64_t shapes[][2] = {{1, 8},     {17, 24},    {65, 520},   {300, 4104},
                                        {4096, 4096}, {11008, 4096}, {4096, 11008}, {28672, 8192}};
    static const int KB[][2] = {{1, 8}, {2, 8}, {4, 8}, {8, 8}, {3, 8}, {1, 16}, {2, 16}, {3, 16}};
    static const int batches[] = {1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 64, 128, 256, 1024, 2048};
    void *c = FAKE(1), *cb = FAKE(2), *x = FAKE(3), *y = FAKE(4);
    int n = 0;
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (size_t k = 0; k < sizeof KB / sizeof KB[0]; ++k)
            for (size_t b = 0; b < sizeof batches / sizeof batches[0]; ++b) {
                const int64_t out = shapes[s][0], in = shapes[s][1];
                const int K = KB[k][0], B = KB[k][1], batch = batches[b];
                for (int op = AQLM_OP_GEMV; op <= AQLM_OP_GEMV_PACKED; ++op) {
                    const int64_t need = aqlm_workspace_bytes(op, AQLM_VARIANT_AUTO, c, cb, x, y, out,
                                                              in, K, B, batch);
                    CHECK(need >= 0, "need %lld op %d %lldx%lld %dx%d b%d", (long long)need, op,
                          (long long)out, (long long)in, K, B, batch);
                    if (op == AQLM_OP_GEMV_PACKED) {
                        CHECK(need > 0, "a packed product always needs a workspace");
                        continue;
                    }
                    const int gemm = op == AQLM_OP_GEMM;
                    const int v_full = aqlm_selected_variant(gemm, c, cb, x, y, out, in, K, B, batch, need);
                    const int v_none = aqlm_selected_variant(gemm, c, cb, x, y, out, in, K, B, batch, 0);
                    CHECK(v_full > 0 && v_none > 0, "choice %d / %d", v_full, v_none);
                    if (need > 0)
                        CHECK(aqlm_selected_variant(gemm, c, cb, x, y, out, in, K, B, batch, need - 1) == -1,
                              "one byte short must be refused");
                    CHECK(aqlm_variant_supported(v_full, c, cb, x, y, out, in, K, B, batch, need) == 1,
                          "chosen variant supported");
                    CHECK(aqlm_variant_supported(AQLM_VARIANT_GENERIC, c, cb, x, y, out, in, K, B, batch, 0) == 1,
                          "generic always");
                    for (int v = 1; v <= 7; ++v) {
                        const int64_t nv = aqlm_workspace_bytes(AQLM_OP_GEMV, v, c, cb, x, y, out, in, K, B, batch);
                        CHECK(nv >= 0, "variant %d need", v);
                    }
                    ++n;
                }
                /* grouped: the shape split in up to four matrices */
                if (out >= 4) {
                    const void *gc[4] = {FAKE(10), FAKE(11), FAKE(12), FAKE(13)};
                    const void *gcb[4] = {FAKE(20), FAKE(21), FAKE(22), FAKE(23)};
                    void *gy[4] = {FAKE(30), FAKE(31), FAKE(32), FAKE(33)};
                    const int64_t q = out / 4;
                    const int64_t outs[4] = {q, q, q, out - 3 * q};
                    for (int op = AQLM_OP_GEMV; op <= AQLM_OP_GEMV_PACKED; ++op)
                        for (int m = 1; m <= 4; ++m)
                            CHECK(aqlm_grouped_workspace_bytes(op, m, gc, gcb, x, gy, outs, in, K, B, batch) >= 0,
                                  "grouped need");
                }
            }
    printf("choice logic: %d calls checked\n", n);
}

static void check_cpu_kernel(void) {
    if (strcmp(aqlm_cpu_isa(), "none") == 0) {
        printf("cpu kernel: no AVX2 on this host, skipped\n");
        return;
    }
    static const int KB[][2] = {{1, 8}, {2, 8}, {4, 8}, {1, 16}, {2, 16}, {3, 16}};
    const int64_t out = 37, in = 200;
    for (size_t k = 0; k < sizeof KB / sizeof KB[0]; ++k)
        for (int batch = 1; batch <= 5; batch += 2) {
            const int K = KB[k][0], B = KB[k][1];
            const int64_t ncodes = out * (in / 8) * K, nent = (int64_t)K << B;
            void *codes = malloc((size_t)(ncodes * (B / 8)));
            uint16_t *cbk = malloc((size_t)nent * 8 * 2), *x = malloc((size_t)(batch * in) * 2);
            uint16_t *y = malloc((size_t)(batch * out) * 2);
            float *W = malloc((size_t)(out * in) * 4);
            double *Y = malloc((size_t)(batch * out) * 8);
            for (int64_t i = 0; i < ncodes; ++i) {
                const uint64_t r = next_u64() >> (64 - B);
                if (B == 8) ((uint8_t *)codes)[i] = (uint8_t)r;
                else ((uint16_t *)codes)[i] = (uint16_t)r;
            }
            for (int64_t i = 0; i < nent * 8; ++i) cbk[i] = oracle_float_to_half((float)(0.02 * next_normal()));
            for (int64_t i = 0; i < batch * in; ++i) x[i] = oracle_float_to_half((float)next_normal());
            CHECK(aqlm_cpu_gemv(codes, cbk, x, y, out, in, K, B, batch, 2) == AQLM_OK, "cpu gemv %dx%d", K, B);
            CHECK(oracle_decode(codes, cbk, W, out, in, K, B, 1) == 0, "oracle decode");
            CHECK(oracle_matvec(W, x, Y, out, in, batch, 1) == 0, "oracle matvec");
            for (int b = 0; b < batch; ++b) {
                double mx = 0, err = 0;
                for (int64_t o = 0; o < out; ++o) mx = fmax(mx, fabs(Y[b * out + o]));
                for (int64_t o = 0; o < out; ++o) {
                    const uint16_t h = y[b * out + o];
                    /* fp16 bits -> value (normal and subnormal; y never holds inf or nan here) */
                    const int e = (h >> 10) & 31, m = h & 1023;
                    double v = e ? ldexp(1024 + m, e - 25) : ldexp(m, -24);
                    if (h & 0x8000) v = -v;
                    err = fmax(err, fabs(v - Y[b * out + o]));
                }
                CHECK(err / (mx + 1e-6) <= 2e-3, "cpu kernel %dx%d batch %d token %d: %.3e", K, B, batch, b,
                      err / (mx + 1e-6));
            }
            free(codes);
            free(cbk);
            free(x);
            free(y);
            free(W);
            free(Y);
        }
    printf("cpu kernel: checked against the oracle (%s)\n", aqlm_cpu_isa());
}

int main(void) {
    check_validation();
    check_choice_logic();
    check_cpu_kernel();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitized host checks ok\n");
    return 0;
}
