// Additive-quantized GEMV on the host cores (token generation on the CPU).
//
// Same product as aqlm_gemv (page "AQLM (Additive Quantization for LLMs)", section
// "Niveau intermediaire": each 8-wide group of a row is the sum of K codebook
// vectors), computed in fp32 from host memory:
// * decode (16-bit codes with K in {1, 2}; 8-bit codes with K = 1): the codebook vectors
//   of two groups (AVX2: one) are converted to fp32 (F16C), summed over k and
//   multiplied with x (FMA); a 1 MiB codebook is served by the core's L2.
// * 8-bit codes with K = 2: a group's two code bytes, read as one little-endian 16-bit
//   index c0 + 256*c1, select an entry of the pair codebook P[c0 + 256*c1] =
//   C_0[c0] + C_1[c1] rounded once to fp16 (the fold the matrix-core kernels use),
//   built per call (1 MiB); the product then runs as the 16-bit K = 1 decode.  Gathers
//   are slow on some hosts; this needs one 16-byte load per group instead.
// * 8-bit codes with K > 2: a row's codes, read in memory order, form the element
//   sequence e = j*K + k (group j, codebook k).  Per token, the table of element e holds
//   C_k[c] . x[8j .. 8j+7] for the 256 codes c (fp32, built once by all threads); a
//   row's product is then the sum over its elements of T[e][code[e]]: 16 lookups per
//   AVX-512 gather (AVX2: 8).  Rows are walked in blocks whose codes stay in L2, and
//   within a block slice by slice along e, so a slice's tables (kSliceElems KiB) stay
//   in L1 while the block's rows read them.
// * 16-bit codes with K > 2: plain scalar code, the fp32 fold then the dot.
// The host needs AVX2, FMA and F16C (AVX-512 F/BW/VL is used where present).  Each row's
// sum is accumulated in an order fixed by the row alone, so the result does not depend
// on the thread count.  y is rounded once to fp16.
#include <immintrin.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "aqlm_mi355x.h"

namespace {

enum Isa { kNone, kAvx2, kAvx512 };

// Before the target pragma below: runs on any x86-64.  AQLM_CPU_ISA=avx2 (read on each
// call) keeps an AVX-512 host on the AVX2 kernels.
Isa detect() {
    static const Isa host = [] {
        __builtin_cpu_init();
        if (!(__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
              __builtin_cpu_supports("f16c")))
            return kNone;
        if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
            __builtin_cpu_supports("avx512vl"))
            return kAvx512;
        return kAvx2;
    }();
    const char *cap = getenv("AQLM_CPU_ISA");
    if (host == kAvx512 && cap && strcmp(cap, "avx2") == 0) return kAvx2;
    return host;
}

}  // namespace

// The kernels below use AVX2, FMA and F16C (AVX-512 ones say so themselves); they run only
// after detect().  gcc takes a target region, clang an attribute applied to each function.
#if defined(__clang__)
#pragma clang attribute push(__attribute__((target("avx2,fma,f16c"))), apply_to = function)
#else
#pragma GCC push_options
#pragma GCC target("avx2,fma,f16c")
#endif

namespace {

constexpr int kGroup = 8;
constexpr int64_t kSliceElems = 32;   // elements per table slice: 32 x 1 KiB of fp32 tables
constexpr int64_t kRowAlign = 16;     // thread row ranges start on multiples of this

float h2f(uint16_t h) { return _cvtsh_ss(h); }
uint16_t f2h(float f) { return _cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT); }

float hsum256(__m256 v) {
    __m128 h = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
    h = _mm_add_ps(h, _mm_movehl_ps(h, h));
    h = _mm_add_ss(h, _mm_shuffle_ps(h, h, 1));
    return _mm_cvtss_f32(h);
}

// Contiguous row range of thread `tid` out of `nt` (ranges start on kRowAlign rows).
void thread_rows(int64_t out, int nt, int tid, int64_t *o0, int64_t *o1) {
    const int64_t units = (out + kRowAlign - 1) / kRowAlign;
    const int64_t per = (units + nt - 1) / nt;
    *o0 = std::min(out, tid * per * kRowAlign);
    *o1 = std::min(out, (tid + 1) * per * kRowAlign);
}

// ------------------------------------------------------------------ scalar (16-bit, K > 2)
float row_dot_scalar(const uint16_t *codes, const uint16_t *cb, const float *xf, int64_t G, int K,
                     int64_t o) {
    float acc = 0.0f;
    for (int64_t j = 0; j < G; ++j) {
        float w[8] = {};
        for (int k = 0; k < K; ++k) {
            const uint16_t *v = cb + ((int64_t(k) << 16) + codes[(o * G + j) * K + k]) * kGroup;
            for (int t = 0; t < 8; ++t) w[t] += h2f(v[t]);
        }
        for (int t = 0; t < 8; ++t) acc += w[t] * xf[j * kGroup + t];
    }
    return acc;
}

// ------------------------------------------------------------------ 8-bit codes: tables
// cbt[k][t][c] = C_k[c][t] in fp32 (transposed once per call)
void transpose_cb8(const uint16_t *cb, int K, float *cbt) {
    for (int k = 0; k < K; ++k)
        for (int c = 0; c < 256; ++c)
            for (int t = 0; t < 8; ++t) cbt[(k * 8 + t) * 256 + c] = h2f(cb[(k * 256 + c) * 8 + t]);
}

// tables of elements e0 .. e1-1 (T points at element 0)
__attribute__((target("avx512f")))
void tables_avx512(const float *cbt, const float *xf, int K, int64_t e0, int64_t e1, float *T) {
    for (int64_t e = e0; e < e1; ++e) {
        const int64_t j = e / K;
        const int k = int(e % K);
        for (int c = 0; c < 256; c += 16) {
            __m512 a = _mm512_setzero_ps();
            for (int t = 0; t < 8; ++t)
                a = _mm512_fmadd_ps(_mm512_loadu_ps(cbt + (k * 8 + t) * 256 + c),
                                    _mm512_set1_ps(xf[j * kGroup + t]), a);
            _mm512_storeu_ps(T + e * 256 + c, a);
        }
    }
}

void tables_avx2(const float *cbt, const float *xf, int K, int64_t e0, int64_t e1, float *T) {
    for (int64_t e = e0; e < e1; ++e) {
        const int64_t j = e / K;
        const int k = int(e % K);
        for (int c = 0; c < 256; c += 8) {
            __m256 a = _mm256_setzero_ps();
            for (int t = 0; t < 8; ++t)
                a = _mm256_fmadd_ps(_mm256_loadu_ps(cbt + (k * 8 + t) * 256 + c),
                                    _mm256_set1_ps(xf[j * kGroup + t]), a);
            _mm256_storeu_ps(T + e * 256 + c, a);
        }
    }
}

// Rows of one token in blocks of `rb` rows (their codes, rb x E bytes, stay in the core's
// L2): within a block the element axis is walked slice by slice, every row of the block
// reading the slice's tables from L1, while the next block's codes are prefetched (one
// 32-byte step per row and slice covers the block).  Each row keeps a vector of lane
// sums (lane = element mod the vector width) across the slices in vacc, reduced once
// at the end.

int64_t lut_block_rows(int64_t E) {
    const int64_t r = (int64_t(256) << 10) / E / kRowAlign * kRowAlign;
    return std::max<int64_t>(kRowAlign, std::min<int64_t>(256, r));
}

// AVX-512: the element tail of a row is a masked gather.
__attribute__((target("avx512f,avx512bw,avx512vl")))
void rows_lut_avx512(const uint8_t *codes, int64_t E, int64_t o0, int64_t o1, const float *T,
                     float *vacc, float *acc) {
    const __m512i lane = _mm512_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    const int64_t rb = lut_block_rows(E);
    for (int64_t b0 = o0; b0 < o1; b0 += rb) {
        const int64_t b1 = std::min(o1, b0 + rb);
        const uint8_t *next = codes + b1 * E, *next_end = codes + o1 * E;
        for (int64_t o = b0; o < b1; ++o) _mm512_storeu_ps(vacc + (o - b0) * 16, _mm512_setzero_ps());
        for (int64_t e0 = 0; e0 < E; e0 += kSliceElems) {
            const int64_t e1 = std::min(E, e0 + kSliceElems);
            for (int64_t o = b0; o < b1; ++o) {
                if (next < next_end) _mm_prefetch(reinterpret_cast<const char *>(next), _MM_HINT_T1);
                next += 32;
                const uint8_t *cr = codes + o * E;
                float *va = vacc + (o - b0) * 16;
                __m512 a = _mm512_loadu_ps(va);
                for (int64_t e = e0; e < e1; e += 16) {
                    const __mmask16 m = e + 16 <= e1 ? __mmask16(0xFFFF)
                                                     : __mmask16((1u << (e1 - e)) - 1u);
                    const __m512i c = _mm512_cvtepu8_epi32(_mm_maskz_loadu_epi8(m, cr + e));
                    const __m512i idx = _mm512_add_epi32(
                        _mm512_slli_epi32(_mm512_add_epi32(lane, _mm512_set1_epi32(int(e))), 8), c);
                    a = _mm512_add_ps(a, _mm512_mask_i32gather_ps(_mm512_setzero_ps(), m, idx, T, 4));
                }
                _mm512_storeu_ps(va, a);
            }
        }
        for (int64_t o = b0; o < b1; ++o)
            acc[o] = _mm512_reduce_add_ps(_mm512_loadu_ps(vacc + (o - b0) * 16));
    }
}

// AVX2: 8 lanes; the elements past the last multiple of 8 are added after the reduction.
void rows_lut_avx2(const uint8_t *codes, int64_t E, int64_t o0, int64_t o1, const float *T,
                   float *vacc, float *acc) {
    const __m256i lane = _mm256_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7);
    const int64_t Ev = E / 8 * 8;
    const int64_t rb = lut_block_rows(E);
    for (int64_t b0 = o0; b0 < o1; b0 += rb) {
        const int64_t b1 = std::min(o1, b0 + rb);
        const uint8_t *next = codes + b1 * E, *next_end = codes + o1 * E;
        for (int64_t o = b0; o < b1; ++o) _mm256_storeu_ps(vacc + (o - b0) * 8, _mm256_setzero_ps());
        for (int64_t e0 = 0; e0 < Ev; e0 += kSliceElems) {
            const int64_t e1 = std::min(Ev, e0 + kSliceElems);
            for (int64_t o = b0; o < b1; ++o) {
                if (next < next_end) _mm_prefetch(reinterpret_cast<const char *>(next), _MM_HINT_T1);
                next += 32;
                const uint8_t *cr = codes + o * E;
                float *va = vacc + (o - b0) * 8;
                __m256 a = _mm256_loadu_ps(va);
                for (int64_t e = e0; e < e1; e += 8) {
                    const __m256i c = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i *>(cr + e)));
                    const __m256i idx = _mm256_add_epi32(
                        _mm256_slli_epi32(_mm256_add_epi32(lane, _mm256_set1_epi32(int(e))), 8), c);
                    a = _mm256_add_ps(a, _mm256_i32gather_ps(T, idx, 4));
                }
                _mm256_storeu_ps(va, a);
            }
        }
        for (int64_t o = b0; o < b1; ++o) {
            float s = hsum256(_mm256_loadu_ps(vacc + (o - b0) * 8));
            for (int64_t e = Ev; e < E; ++e) s += T[e * 256 + codes[o * E + e]];
            acc[o] = s;
        }
    }
}

// ------------------------------------------------------------------ 16-bit codes: decode
// Row o: two groups per step into one 16-lane fp32 vector; two accumulators (even and
// odd steps) hide the FMA latency, added at the end; an odd last group is scalar.
// groups j and j+1 of the row whose codes (type C, codebooks of `entries` vectors)
// start at cr, folded, as 16 fp32 lanes
template <int K, typename C>
__attribute__((target("avx512f"), always_inline)) inline
__m512 dec_pair(const C *cr, const uint16_t *cb, int64_t entries, int64_t j) {
    __m512 v = _mm512_setzero_ps();
    for (int k = 0; k < K; ++k) {
        const __m128i a = _mm_loadu_si128(reinterpret_cast<const __m128i *>(
            cb + (k * entries + cr[j * K + k]) * kGroup));
        const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i *>(
            cb + (k * entries + cr[(j + 1) * K + k]) * kGroup));
        v = _mm512_add_ps(v, _mm512_cvtph_ps(_mm256_inserti128_si256(_mm256_castsi128_si256(a), b, 1)));
    }
    return v;
}

// NB tokens of one row at once: each decoded group pair is used for every token
// (xf holds the tokens' activations `in` apart); per token the sums are formed exactly
// as with one token.
template <int K, int NB, typename C>
__attribute__((target("avx512f")))
void row_dec_avx512(const C *codes, const uint16_t *cb, int64_t entries, const float *xf, int64_t G,
                    int64_t o, float *s) {
    const C *cr = codes + o * G * K;
    const int64_t in = G * kGroup;
    __m512 acc0[NB], acc1[NB];
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = _mm512_setzero_ps();
    int64_t j = 0;
    for (; j + 4 <= G; j += 4) {
        const __m512 v0 = dec_pair<K>(cr, cb, entries, j), v1 = dec_pair<K>(cr, cb, entries, j + 2);
        for (int b = 0; b < NB; ++b) {
            acc0[b] = _mm512_fmadd_ps(v0, _mm512_loadu_ps(xf + b * in + j * kGroup), acc0[b]);
            acc1[b] = _mm512_fmadd_ps(v1, _mm512_loadu_ps(xf + b * in + (j + 2) * kGroup), acc1[b]);
        }
    }
    if (j + 2 <= G) {
        const __m512 v0 = dec_pair<K>(cr, cb, entries, j);
        for (int b = 0; b < NB; ++b)
            acc0[b] = _mm512_fmadd_ps(v0, _mm512_loadu_ps(xf + b * in + j * kGroup), acc0[b]);
        j += 2;
    }
    for (int b = 0; b < NB; ++b) s[b] = _mm512_reduce_add_ps(_mm512_add_ps(acc0[b], acc1[b]));
    if (j < G) {
        float w[8] = {};
        for (int k = 0; k < K; ++k) {
            const uint16_t *v = cb + (k * entries + cr[j * K + k]) * kGroup;
            for (int t = 0; t < 8; ++t) w[t] += h2f(v[t]);
        }
        for (int b = 0; b < NB; ++b)
            for (int t = 0; t < 8; ++t) s[b] += w[t] * xf[b * in + j * kGroup + t];
    }
}

template <int K, int NB, typename C>
void row_dec_avx2(const C *codes, const uint16_t *cb, int64_t entries, const float *xf, int64_t G,
                  int64_t o, float *s) {
    const C *cr = codes + o * G * K;
    const int64_t in = G * kGroup;
    auto one = [&](int64_t j) {
        __m256 v = _mm256_setzero_ps();
        for (int k = 0; k < K; ++k)
            v = _mm256_add_ps(v, _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(
                                     cb + (k * entries + cr[j * K + k]) * kGroup))));
        return v;
    };
    __m256 acc0[NB], acc1[NB];
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = _mm256_setzero_ps();
    int64_t j = 0;
    for (; j + 2 <= G; j += 2) {
        const __m256 v0 = one(j), v1 = one(j + 1);
        for (int b = 0; b < NB; ++b) {
            acc0[b] = _mm256_fmadd_ps(v0, _mm256_loadu_ps(xf + b * in + j * kGroup), acc0[b]);
            acc1[b] = _mm256_fmadd_ps(v1, _mm256_loadu_ps(xf + b * in + (j + 1) * kGroup), acc1[b]);
        }
    }
    if (j < G) {
        const __m256 v0 = one(j);
        for (int b = 0; b < NB; ++b)
            acc0[b] = _mm256_fmadd_ps(v0, _mm256_loadu_ps(xf + b * in + j * kGroup), acc0[b]);
    }
    for (int b = 0; b < NB; ++b) s[b] = hsum256(_mm256_add_ps(acc0[b], acc1[b]));
}

// ------------------------------------------------------------------ 2x8: pair codebook
// P[c0 + 256*c1][t] = fp16(C_0[c0][t] + C_1[c1][t]) for the c1 of c1_begin .. c1_end-1
void pair_codebook(const uint16_t *cb, int c1_begin, int c1_end, uint16_t *P) {
    for (int c1 = c1_begin; c1 < c1_end; ++c1) {
        const __m256 b = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(cb + (256 + c1) * kGroup)));
        for (int c0 = 0; c0 < 256; ++c0) {
            const __m256 a = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(cb + c0 * kGroup)));
            _mm_storeu_si128(reinterpret_cast<__m128i *>(P + (int64_t(c1) * 256 + c0) * kGroup),
                             _mm256_cvtps_ph(_mm256_add_ps(a, b), _MM_FROUND_TO_NEAREST_INT));
        }
    }
}

template <int K, int NB, typename C>
void row_dec_nb(Isa isa, const C *codes, const uint16_t *cb, int64_t entries, const float *xf,
                int64_t G, int64_t o, float *s) {
    if (isa == kAvx512) row_dec_avx512<K, NB>(codes, cb, entries, xf, G, o, s);
    else row_dec_avx2<K, NB>(codes, cb, entries, xf, G, o, s);
}

// nb (1..kDecTokens) tokens of row o
constexpr int kDecTokens = 4;
template <int K, typename C>
void row_dec(Isa isa, const C *codes, const uint16_t *cb, int64_t entries, const float *xf, int64_t G,
             int64_t o, int nb, float *s) {
    switch (nb) {
        case 1: row_dec_nb<K, 1>(isa, codes, cb, entries, xf, G, o, s); break;
        case 2: row_dec_nb<K, 2>(isa, codes, cb, entries, xf, G, o, s); break;
        case 3: row_dec_nb<K, 3>(isa, codes, cb, entries, xf, G, o, s); break;
        default: row_dec_nb<K, 4>(isa, codes, cb, entries, xf, G, o, s); break;
    }
}

aqlm_status_t cpu_gemv(const void *codes_, const void *codebooks_, const void *x_, void *y_,
                       int64_t out, int64_t in, int K, int B, int batch, int threads) {
    if (!codes_ || !codebooks_ || !x_ || !y_ || out < 1 || in < kGroup || in % kGroup || K < 1 ||
        K > 8 || (B != 8 && B != 16) || batch < 1)
        return AQLM_ERR_INVALID_ARGUMENT;
    const int64_t G = in / kGroup;
    if (out > (int64_t(1) << 40) / G || int64_t(batch) * in > (int64_t(1) << 40))
        return AQLM_ERR_INVALID_ARGUMENT;
    const int64_t E = G * K;   // elements (codes) per row
    if (B == 8 && E >= (int64_t(1) << 23)) return AQLM_ERR_INVALID_ARGUMENT;   // int32 table index
    const uint8_t *codes = static_cast<const uint8_t *>(codes_);
    const uint16_t *c16 = static_cast<const uint16_t *>(codes_);
    const uint16_t *cb = static_cast<const uint16_t *>(codebooks_);
    const uint16_t *x = static_cast<const uint16_t *>(x_);
    uint16_t *y = static_cast<uint16_t *>(y_);
    const Isa isa = detect();
    const int nt = threads > 0 ? threads : omp_get_max_threads();
    const bool lut = B == 8 && K > 2;
    const bool pair = B == 8 && K == 2;
    std::vector<uint16_t> P(pair ? size_t(65536) * kGroup : 0);
    if (pair) {
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int c1 = 0; c1 < 256; c1 += 16) pair_codebook(cb, c1, c1 + 16, P.data());
    }

    // the decode paths take up to kDecTokens tokens per pass over the codes; the table
    // and scalar paths one
    const bool dec = !lut && !(B == 16 && K > 2);
    const int tb = dec ? kDecTokens : 1;
    std::vector<float> xf(size_t(tb) * size_t(in));
    std::vector<float> cbt(lut ? size_t(K) * 8 * 256 : 0);
    if (lut) transpose_cb8(cb, K, cbt.data());
    std::vector<float> T(lut ? size_t(E) * 256 : 0);
    std::vector<float> acc(size_t(tb) * size_t(out));
    // per-thread lane sums of one row block
    const size_t vacc_rows = lut ? size_t(lut_block_rows(E)) : 0;
    std::vector<float> vacc(size_t(nt) * vacc_rows * 16);
    for (int b0 = 0; b0 < batch; b0 += tb) {
        const int nb = std::min(tb, batch - b0);
        for (int64_t i = 0; i < int64_t(nb) * in; ++i) xf[i] = h2f(x[int64_t(b0) * in + i]);
#pragma omp parallel num_threads(nt)
        {
            const int tid = omp_get_thread_num(), nth = omp_get_num_threads();
            int64_t o0, o1;
            thread_rows(out, nth, tid, &o0, &o1);
            if (lut) {
                const int64_t per = (E + nth - 1) / nth;
                const int64_t e0 = std::min(E, tid * per), e1 = std::min(E, e0 + per);
                if (isa == kAvx512) tables_avx512(cbt.data(), xf.data(), K, e0, e1, T.data());
                else tables_avx2(cbt.data(), xf.data(), K, e0, e1, T.data());
#pragma omp barrier
                float *va = vacc.data() + size_t(tid) * vacc_rows * 16;
                if (o0 < o1) {
                    if (isa == kAvx512) rows_lut_avx512(codes, E, o0, o1, T.data(), va, acc.data());
                    else rows_lut_avx2(codes, E, o0, o1, T.data(), va, acc.data());
                }
            } else {
                for (int64_t o = o0; o < o1; ++o) {
                    float sb[kDecTokens];
                    if (pair)   // the two code bytes of a group as one 16-bit index
                        row_dec<1>(isa, c16, P.data(), 65536, xf.data(), G, o, nb, sb);
                    else if (B == 8)
                        row_dec<1>(isa, codes, cb, 256, xf.data(), G, o, nb, sb);
                    else if (K == 1)
                        row_dec<1>(isa, c16, cb, 65536, xf.data(), G, o, nb, sb);
                    else if (K == 2)
                        row_dec<2>(isa, c16, cb, 65536, xf.data(), G, o, nb, sb);
                    else
                        sb[0] = row_dot_scalar(c16, cb, xf.data(), G, K, o);
                    for (int b = 0; b < nb; ++b) acc[size_t(b) * out + o] = sb[b];
                }
            }
        }
        for (int b = 0; b < nb; ++b)
            for (int64_t o = 0; o < out; ++o)
                y[int64_t(b0 + b) * out + o] = f2h(acc[size_t(b) * out + o]);
    }
    return AQLM_OK;
}

}  // namespace

#if defined(__clang__)
#pragma clang attribute pop
#else
#pragma GCC pop_options
#endif

extern "C" {

const char *aqlm_cpu_isa(void) {
    switch (detect()) {
        case kAvx512: return "avx512";
        case kAvx2: return "avx2";
        default: return "none";
    }
}

aqlm_status_t aqlm_cpu_gemv(const void *codes, const void *codebooks, const void *x, void *y,
                            int64_t out, int64_t in, int K, int B, int batch, int threads) {
    if (detect() == kNone) return AQLM_ERR_UNSUPPORTED;   // needs AVX2, FMA and F16C
    return cpu_gemv(codes, codebooks, x, y, out, in, K, B, batch, threads);
}

}  // extern "C"
