// C ABI of libaqlm_mi355x: argument checks, kernel choice, launch, error mapping.
// The operation and layouts are documented in include/aqlm_mi355x.h.
#include "aqlm_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "kernels.hpp"

namespace {

constexpr int kGroup = 8;
// Batch from which aqlm_gemm takes the matrix cores.  Measured on MI355X (7B layer,
// grouped, us, gather kernels -> matrix cores): 2x8 b2 80 -> 42, b8 260 -> 48; 1x16 b2
// 129 -> 123, b8 323 -> 131; 4x8 b2 104 -> 89; 2x16 b8 340 -> 244; 8x8 b2 147 -> 184
// (the fp32 fold of 8 codebooks per group), b8 335 -> 185.
constexpr int kMfmaMinBatch = 2;
constexpr int kMfmaMinBatch8Codebooks = 4;
// Canonical 16-bit codes at small batches: the split kernel, its codebook packed into the
// workspace on every call, against the L2-gather kernel and the matrix cores (1x16 7B
// layer, grouped / separate calls, us: batch 3 split 123.9 / 149.5 against matrix cores
// 123.6 / 132.4; batch 4 131.8 / 157.7 against 124.9 / 134.4).
constexpr int kSplitMaxBatch = 4;
constexpr int kSplitMaxBatchGemm = 2;
// Measured on MI355X (7B layer linears, canonical weights): the prefill path overtakes the
// matrix-core kernels at batch 256 for 16-bit codes (decoding a 1 MiB codebook through
// L2 per token tile costs more) and at 1024 for 8-bit codes with K <= 2.
constexpr int kPrefillMinBatch16 = 256;
constexpr int kPrefillMinBatch8 = 1024;

thread_local char g_last_error[256] = "";

void set_error(const char *what, hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
}

bool log_enabled() {
    static const bool on = [] {
        const char *v = std::getenv("AQLM_LOG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

int forced_variant() {
    const char *v = std::getenv("AQLM_FORCE_VARIANT");
    if (!v || !*v) return AQLM_VARIANT_AUTO;
    if (!std::strcmp(v, "generic")) return AQLM_VARIANT_GENERIC;
    if (!std::strcmp(v, "lds")) return AQLM_VARIANT_LDS;
    if (!std::strcmp(v, "lut")) return AQLM_VARIANT_LUT;
    if (!std::strcmp(v, "l2")) return AQLM_VARIANT_L2;
    if (!std::strcmp(v, "mfma")) return AQLM_VARIANT_MFMA;
    if (!std::strcmp(v, "split")) return AQLM_VARIANT_SPLIT;
    if (!std::strcmp(v, "prefill")) return AQLM_VARIANT_PREFILL;
    return AQLM_VARIANT_AUTO;
}

// batch from which aqlm_gemm decodes W once and runs one library GEMM
// (AQLM_PREFILL_MIN_BATCH overrides)
int prefill_min_batch(const aqlm::Problem &p) {
    const int def = (p.B == 16 || p.K >= 4) ? kPrefillMinBatch16 : kPrefillMinBatch8;
    const char *v = std::getenv("AQLM_PREFILL_MIN_BATCH");
    if (!v || !*v) return def;
    const int n = std::atoi(v);
    return n >= 1 ? n : def;
}

int mfma_min_batch(int K) {
    const int def = K >= 8 ? kMfmaMinBatch8Codebooks : kMfmaMinBatch;
    const char *v = std::getenv("AQLM_MFMA_MIN_BATCH");
    if (!v || !*v) return def;
    const int n = std::atoi(v);
    return n >= 1 ? n : def;
}

// [a, a+na) and [b, b+nb) overlap?
bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + uint64_t(nb) && y < x + uint64_t(na);
}

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }

struct Sizes {
    int64_t codes, codebooks, x, y;
};

// Validates shape arguments and computes byte sizes; false on any error.
bool check_shape(int64_t out, int64_t in, int K, int B, int64_t batch, Sizes *s) {
    if (out < 1 || in < 1 || batch < 1) return false;
    if (in % kGroup) return false;
    if (K < 1 || K > 8) return false;
    if (B != 8 && B != 16) return false;
    int64_t t;
    if (!mul_ok(out, in / kGroup, &t) || !mul_ok(t, int64_t(K) * (B / 8), &s->codes)) return false;
    s->codebooks = int64_t(K) * (int64_t(1) << B) * kGroup * 2;
    if (!mul_ok(batch, in, &t) || !mul_ok(t, 2, &s->x)) return false;
    if (!mul_ok(batch, out, &t) || !mul_ok(t, 2, &s->y)) return false;
    return true;
}

aqlm_status_t check_args(const void *codes, const void *cb, const void *x, const void *y,
                         int64_t out, int64_t in, int K, int B, int batch, Sizes *s) {
    if (!codes || !cb || !x || !y) return AQLM_ERR_INVALID_ARGUMENT;
    if (!check_shape(out, in, K, B, batch, s)) return AQLM_ERR_INVALID_ARGUMENT;
    // element alignment: 2-byte codes for B = 16, fp16 data everywhere
    const uintptr_t a = reinterpret_cast<uintptr_t>(cb) | reinterpret_cast<uintptr_t>(x) |
                        reinterpret_cast<uintptr_t>(y) |
                        (B == 16 ? reinterpret_cast<uintptr_t>(codes) : 0);
    if (a & 1u) return AQLM_ERR_INVALID_ARGUMENT;
    if (overlaps(y, s->y, codes, s->codes) || overlaps(y, s->y, cb, s->codebooks) ||
        overlaps(y, s->y, x, s->x))
        return AQLM_ERR_INVALID_ARGUMENT;
    return AQLM_OK;
}

aqlm::Problem make_problem(const void *codes, const void *cb, const void *x, void *y, int64_t out,
                           int64_t in, int K, int B, int batch, void *stream) {
    aqlm::Problem p{codes, cb, x, y, out, in, K, B, batch, static_cast<hipStream_t>(stream), {}};
    p.segs.n = 1;
    p.segs.row0[0] = 0;
    p.segs.row0[1] = int(out);          // callers keep out <= 2^30 for the tuned kernels
    p.segs.codes[0] = codes;
    p.segs.cb[0] = cb;
    p.segs.y[0] = y;
    return p;
}

// Matrix m of a grouped problem as a problem of its own.
aqlm::Problem segment(const aqlm::Problem &p, int m) {
    return make_problem(p.segs.codes[m], p.segs.cb[m], p.x, p.segs.y[m],
                        p.segs.row0[m + 1] - p.segs.row0[m], p.in, p.K, p.B, p.batch, p.stream);
}

// Packed codes: tiles of 8 rows x 64 groups for 2x8 (the lookup-table kernel's
// layout), the canonical layout (a plain copy) for every other (K, B).
bool tiled_codes(int K, int B) { return K == 2 && B == 8; }

int64_t packed_codes_size(int64_t out, int64_t in, int K, int B) {
    Sizes s;
    if (!check_shape(out, in, K, B, 1, &s)) return -1;
    if (!tiled_codes(K, B)) return s.codes;
    if (out > (int64_t(1) << 30) || in > (int64_t(1) << 30)) return -1;
    return aqlm::lut_packed_codes_bytes(out, in);
}

// f holds for the whole problem and for each of its matrices
template <class F>
bool all_segments(const aqlm::Problem &p, F f) {
    if (!f(p)) return false;
    for (int m = 0; p.segs.n > 1 && m < p.segs.n; ++m)
        if (!f(segment(p, m))) return false;
    return true;
}

bool supported_one(int variant, const aqlm::Problem &p);

bool supported(int variant, const aqlm::Problem &p) {
    return all_segments(p, [variant](const aqlm::Problem &q) { return supported_one(variant, q); });
}

bool supported_one(int variant, const aqlm::Problem &p) {
    switch (variant) {
        case AQLM_VARIANT_GENERIC: return true;
        case AQLM_VARIANT_LDS: return p.B == 8 && aqlm::gather_supported(p);
        case AQLM_VARIANT_LUT: return aqlm::lut_supported(p);
        case AQLM_VARIANT_L2: return aqlm::l2_supported(p);
        case AQLM_VARIANT_MFMA: return aqlm::mfma_supported(p);
        case AQLM_VARIANT_PREFILL: return aqlm::mfma_supported(p);
        case AQLM_VARIANT_SPLIT: return aqlm::ds_supported(p);
        default: return false;
    }
}

int choose(bool gemm, const aqlm::Problem &p) {
    const int forced = forced_variant();
    if (forced != AQLM_VARIANT_AUTO && supported(forced, p)) return forced;
    if (gemm && p.batch >= prefill_min_batch(p) && supported(AQLM_VARIANT_PREFILL, p))
        return AQLM_VARIANT_PREFILL;
    // 16-bit codes: the split kernel (codebook packed per call) up to batch 4, or 2 where
    // the matrix cores are allowed
    if (p.batch <= (gemm ? kSplitMaxBatchGemm : kSplitMaxBatch) && supported(AQLM_VARIANT_SPLIT, p))
        return AQLM_VARIANT_SPLIT;
    if (gemm && p.batch >= mfma_min_batch(p.K) && supported(AQLM_VARIANT_MFMA, p))
        return AQLM_VARIANT_MFMA;
    if (supported(AQLM_VARIANT_LUT, p)) return AQLM_VARIANT_LUT;
    if (supported(AQLM_VARIANT_LDS, p)) return AQLM_VARIANT_LDS;
    if (supported(AQLM_VARIANT_L2, p)) return AQLM_VARIANT_L2;
    return AQLM_VARIANT_GENERIC;
}

// Split-slice partial sums of the lookup-table kernel live in one workspace per
// (device, stream), grown on demand and kept until the process exits.  Calls on
// one stream are ordered, so they can share it.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Returns the stream's workspace of at least `bytes`.  A stream that is being
// captured into a graph cannot allocate: if it has no large enough workspace
// yet, *out is left null (the caller then picks a kernel that needs none).
hipError_t get_workspace(hipStream_t stream, size_t bytes, void **out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
        (void)hipGetLastError();  // a stream that cannot be queried is not capturing
        cap = hipStreamCaptureStatusNone;
    }
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[std::make_pair(dev, stream)];
    if (w.bytes < bytes) {
        if (cap != hipStreamCaptureStatusNone) return hipSuccess;
        if (w.ptr) {
            e = hipStreamSynchronize(stream);  // earlier launches may still use it
            if (e != hipSuccess) return e;
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        size_t nb = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
        e = hipMalloc(&w.ptr, nb);
        if (e != hipSuccess) return e;
        w.bytes = nb;
    }
    *out = w.ptr;
    return hipSuccess;
}

// Packs or unpacks codebooks; shared argument checks.
aqlm_status_t pack_common(const void *src, void *dst, int K, int B, void *stream, bool pack) {
    if (!src || !dst || K < 1 || K > 8 || (B != 8 && B != 16)) return AQLM_ERR_INVALID_ARGUMENT;
    const int64_t bytes = int64_t(K) * (int64_t(1) << B) * kGroup * 2;
    // 16-bit codes are packed as 32-bit position pairs
    const uintptr_t align = B == 16 ? 3u : 1u;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & align) ||
        overlaps(src, bytes, dst, bytes))
        return AQLM_ERR_INVALID_ARGUMENT;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = pack ? aqlm::launch_pack_codebooks(src, dst, K, B, s)
                              : aqlm::launch_unpack_codebooks(src, dst, K, B, s);
    if (e != hipSuccess) {
        set_error(pack ? "pack_codebooks" : "unpack_codebooks", e);
        return AQLM_ERR_HIP;
    }
    return AQLM_OK;
}

aqlm_status_t run(int variant, const aqlm::Problem &p) {
    hipError_t e = hipSuccess;
    if (log_enabled())
        std::fprintf(stderr, "[aqlm] %s out=%lld in=%lld K=%d B=%d batch=%d\n",
                     aqlm_variant_name(variant), (long long)p.out, (long long)p.in, p.K, p.B,
                     p.batch);
    // kernels without a matrix table run once per matrix
    if (p.segs.n > 1 && (variant == AQLM_VARIANT_LDS || variant == AQLM_VARIANT_GENERIC ||
                         variant == AQLM_VARIANT_PREFILL)) {
        for (int m = 0; m < p.segs.n; ++m) {
            const aqlm_status_t st = run(variant, segment(p, m));
            if (st != AQLM_OK) return st;
        }
        return AQLM_OK;
    }
    switch (variant) {
        case AQLM_VARIANT_LDS: e = aqlm::launch_gather(p); break;
        case AQLM_VARIANT_L2: e = aqlm::launch_l2(p); break;
        case AQLM_VARIANT_LUT: {
            void *ws = nullptr;
            e = get_workspace(p.stream, aqlm::lut_workspace_bytes(p), &ws);
            if (e != hipSuccess) break;
            if (ws) {
                e = aqlm::launch_lut(p, ws);
            } else if (p.segs.n > 1) {
                // capturing stream whose workspace fits the matrices one at a time only
                for (int m = 0; m < p.segs.n; ++m) {
                    const aqlm_status_t st = run(variant, segment(p, m));
                    if (st != AQLM_OK) return st;
                }
                return AQLM_OK;
            } else {
                // capturing stream without a workspace: same product, no workspace needed
                if (log_enabled())
                    std::fprintf(stderr, "[aqlm] lut: no workspace on a capturing stream, "
                                         "using the gather kernel\n");
                for (int m = 0; m < p.segs.n && e == hipSuccess; ++m) {
                    const aqlm::Problem q = segment(p, m);
                    e = aqlm::gather_supported(q) ? aqlm::launch_gather(q) : aqlm::launch_generic(q);
                }
            }
            break;
        }
        case AQLM_VARIANT_MFMA: {
            const size_t need = aqlm::mfma_workspace_bytes(p);
            void *ws = nullptr;
            if (need) {
                e = get_workspace(p.stream, need, &ws);
                if (e != hipSuccess) break;
                if (!ws && p.segs.n > 1) {
                    // capturing stream whose workspace may fit the matrices one at a time
                    for (int m = 0; m < p.segs.n; ++m) {
                        const aqlm_status_t st = run(variant, segment(p, m));
                        if (st != AQLM_OK) return st;
                    }
                    return AQLM_OK;
                }
                if (!ws) {
                    // capturing stream without a workspace: same product, no workspace needed
                    for (int m = 0; m < p.segs.n && e == hipSuccess; ++m)
                        e = aqlm::launch_generic(segment(p, m));
                    break;
                }
            }
            e = aqlm::launch_mfma(p, ws);
            break;
        }
        case AQLM_VARIANT_SPLIT: {
            void *ws = nullptr;
            e = get_workspace(p.stream, aqlm::split_canonical_workspace_bytes(p), &ws);
            if (e != hipSuccess) break;
            if (!ws) {
                // capturing stream without a large enough workspace: the L2-gather kernel
                if (log_enabled())
                    std::fprintf(stderr, "[aqlm] split: no workspace on a capturing stream\n");
                return run(supported(AQLM_VARIANT_L2, p) ? AQLM_VARIANT_L2 : AQLM_VARIANT_GENERIC, p);
            }
            e = aqlm::launch_split_canonical(p, ws);
            break;
        }
        case AQLM_VARIANT_PREFILL: {
            void *ws = nullptr;
            e = get_workspace(p.stream, aqlm::prefill_workspace_bytes(p), &ws);
            if (e != hipSuccess) break;
            if (!ws) {
                // capturing stream without a large enough workspace: the matrix cores
                if (log_enabled())
                    std::fprintf(stderr, "[aqlm] prefill: no workspace on a capturing stream\n");
                return run(AQLM_VARIANT_MFMA, p);
            }
            e = aqlm::launch_prefill(p, ws);
            break;
        }
        default:
            for (int m = 0; m < p.segs.n && e == hipSuccess; ++m) e = aqlm::launch_generic(segment(p, m));
            break;
    }
    if (e != hipSuccess) {
        set_error(aqlm_variant_name(variant), e);
        return AQLM_ERR_HIP;
    }
    return AQLM_OK;
}

// Validates a grouped call and builds its problem (out = the total rows).  packed: the
// codes are in the packed layout of aqlm_pack_codes.
aqlm_status_t grouped_problem(int n, const void *const *codes, const void *const *codebooks,
                              const void *x, void *const *y, const int64_t *out_features,
                              int64_t in, int K, int B, int batch, void *stream, bool packed,
                              aqlm::Problem *out) {
    if (n < 1 || n > aqlm::kMaxSegs || !codes || !codebooks || !y || !out_features)
        return AQLM_ERR_INVALID_ARGUMENT;
    int64_t total = 0, code_bytes[aqlm::kMaxSegs];
    Sizes s{};
    for (int m = 0; m < n; ++m) {
        const aqlm_status_t st =
            check_args(codes[m], codebooks[m], x, y[m], out_features[m], in, K, B, batch, &s);
        if (st != AQLM_OK) return st;
        code_bytes[m] = packed ? packed_codes_size(out_features[m], in, K, B) : s.codes;
        if (code_bytes[m] < 0) return AQLM_ERR_INVALID_ARGUMENT;
        total += out_features[m];
    }
    if (total > (int64_t(1) << 30)) return AQLM_ERR_INVALID_ARGUMENT;
    // no output may overlap any input or another output
    for (int m = 0; m < n; ++m) {
        const int64_t ym = int64_t(batch) * out_features[m] * 2;
        for (int j = 0; j < n; ++j) {
            if (overlaps(y[m], ym, codes[j], code_bytes[j]) ||
                overlaps(y[m], ym, codebooks[j], s.codebooks))
                return AQLM_ERR_INVALID_ARGUMENT;
            if (j != m && overlaps(y[m], ym, y[j], int64_t(batch) * out_features[j] * 2))
                return AQLM_ERR_INVALID_ARGUMENT;
        }
    }
    aqlm::Problem p = make_problem(codes[0], codebooks[0], x, y[0], total, in, K, B, batch, stream);
    p.segs.n = n;
    int r = 0;
    for (int m = 0; m < n; ++m) {
        p.segs.row0[m] = r;
        r += int(out_features[m]);
        p.segs.codes[m] = codes[m];
        p.segs.cb[m] = codebooks[m];
        p.segs.y[m] = y[m];
    }
    p.segs.row0[n] = r;
    *out = p;
    return AQLM_OK;
}

}  // namespace

extern "C" {

aqlm_status_t aqlm_gemv(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *stream) {
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    return run(choose(false, p), p);
}

aqlm_status_t aqlm_gemm(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *stream) {
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    return run(choose(true, p), p);
}

aqlm_status_t aqlm_gemv_variant(int variant, const void *codes, const void *codebooks,
                                const void *x, void *y, int64_t out_features,
                                int64_t in_features, int K, int B, int batch, void *stream) {
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    if (variant == AQLM_VARIANT_AUTO) return run(choose(false, p), p);
    if (!supported(variant, p)) return AQLM_ERR_UNSUPPORTED;
    return run(variant, p);
}

int aqlm_variant_supported(int variant, const void *codes, const void *codebooks, const void *x,
                           const void *y, int64_t out_features, int64_t in_features, int K, int B,
                           int batch) {
    Sizes s;
    if (check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s) != AQLM_OK)
        return 0;
    const aqlm::Problem p = make_problem(codes, codebooks, x, const_cast<void *>(y), out_features,
                                         in_features, K, B, batch, nullptr);
    if (variant == AQLM_VARIANT_AUTO) return 1;
    return supported(variant, p) ? 1 : 0;
}

int aqlm_selected_variant(int gemm, const void *codes, const void *codebooks, const void *x,
                          const void *y, int64_t out_features, int64_t in_features, int K, int B,
                          int batch) {
    Sizes s;
    if (check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s) != AQLM_OK)
        return -1;
    const aqlm::Problem p = make_problem(codes, codebooks, x, const_cast<void *>(y), out_features,
                                         in_features, K, B, batch, nullptr);
    return choose(gemm != 0, p);
}

aqlm_status_t aqlm_dequantize(const void *codes, const void *codebooks, void *W, int w_dtype,
                              int64_t out_features, int64_t in_features, int K, int B,
                              void *stream) {
    if (!codes || !codebooks || !W) return AQLM_ERR_INVALID_ARGUMENT;
    if (w_dtype != 0 && w_dtype != 1) return AQLM_ERR_INVALID_ARGUMENT;
    Sizes s;
    if (!check_shape(out_features, in_features, K, B, 1, &s)) return AQLM_ERR_INVALID_ARGUMENT;
    int64_t wbytes;
    if (!mul_ok(out_features, in_features, &wbytes) || !mul_ok(wbytes, w_dtype ? 2 : 4, &wbytes))
        return AQLM_ERR_INVALID_ARGUMENT;
    const uintptr_t a = reinterpret_cast<uintptr_t>(codebooks) |
                        (B == 16 ? reinterpret_cast<uintptr_t>(codes) : 0);
    if ((a & 1u) || (reinterpret_cast<uintptr_t>(W) & (w_dtype ? 1u : 3u)))
        return AQLM_ERR_INVALID_ARGUMENT;
    if (overlaps(W, wbytes, codes, s.codes) || overlaps(W, wbytes, codebooks, s.codebooks))
        return AQLM_ERR_INVALID_ARGUMENT;
    const aqlm::Problem p = make_problem(codes, codebooks, nullptr, nullptr, out_features,
                                         in_features, K, B, 1, stream);
    const hipError_t e = aqlm::launch_dequantize(p, W, w_dtype);
    if (e != hipSuccess) {
        set_error("dequantize", e);
        return AQLM_ERR_HIP;
    }
    return AQLM_OK;
}

double aqlm_bits_per_weight(int K, int B, int group) {
    if (group < 1) return 0.0;
    return double(K) * double(B) / double(group);
}

int64_t aqlm_codes_bytes(int64_t out_features, int64_t in_features, int K, int B) {
    Sizes s;
    if (!check_shape(out_features, in_features, K, B, 1, &s)) return -1;
    return s.codes;
}

int64_t aqlm_codebooks_bytes(int K, int B) {
    if (K < 1 || K > 8 || (B != 8 && B != 16)) return -1;
    return int64_t(K) * (int64_t(1) << B) * kGroup * 2;
}

const char *aqlm_status_string(aqlm_status_t status) {
    switch (status) {
        case AQLM_OK: return "ok";
        case AQLM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case AQLM_ERR_UNSUPPORTED: return "variant does not support these arguments";
        case AQLM_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char *aqlm_variant_name(int variant) {
    switch (variant) {
        case AQLM_VARIANT_AUTO: return "auto";
        case AQLM_VARIANT_GENERIC: return "generic";
        case AQLM_VARIANT_LDS: return "lds";
        case AQLM_VARIANT_LUT: return "lut";
        case AQLM_VARIANT_L2: return "l2";
        case AQLM_VARIANT_MFMA: return "mfma";
        case AQLM_VARIANT_SPLIT: return "split";
        case AQLM_VARIANT_PREFILL: return "prefill";
        default: return "unknown";
    }
}

aqlm_status_t aqlm_pack_codebooks(const void *codebooks, void *packed, int K, int B,
                                  void *stream) {
    return pack_common(codebooks, packed, K, B, stream, true);
}

aqlm_status_t aqlm_unpack_codebooks(const void *packed, void *codebooks, int K, int B,
                                    void *stream) {
    return pack_common(packed, codebooks, K, B, stream, false);
}

int64_t aqlm_packed_codes_bytes(int64_t out_features, int64_t in_features, int K, int B) {
    return packed_codes_size(out_features, in_features, K, B);
}

static aqlm_status_t pack_codes_common(const void *src, void *dst, int64_t out, int64_t in, int K,
                                       int B, void *stream, bool pack) {
    if (!src || !dst) return AQLM_ERR_INVALID_ARGUMENT;
    const int64_t pbytes = packed_codes_size(out, in, K, B);
    if (pbytes < 0) return AQLM_ERR_INVALID_ARGUMENT;
    const int64_t cbytes = out * (in / kGroup) * K * (B / 8);
    const int64_t sbytes = pack ? cbytes : pbytes, dbytes = pack ? pbytes : cbytes;
    if (overlaps(src, sbytes, dst, dbytes)) return AQLM_ERR_INVALID_ARGUMENT;
    const bool tiled = tiled_codes(K, B);
    if (tiled && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 1u))
        return AQLM_ERR_INVALID_ARGUMENT;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = tiled ? aqlm::launch_pack_codes_lut(src, dst, out, in, pack, s)
                               : aqlm::launch_copy_bytes(src, dst, cbytes, s);
    if (e != hipSuccess) {
        set_error(pack ? "pack_codes" : "unpack_codes", e);
        return AQLM_ERR_HIP;
    }
    return AQLM_OK;
}

aqlm_status_t aqlm_pack_codes(const void *codes, void *packed, int64_t out_features,
                              int64_t in_features, int K, int B, void *stream) {
    return pack_codes_common(codes, packed, out_features, in_features, K, B, stream, true);
}

aqlm_status_t aqlm_unpack_codes(const void *packed, void *codes, int64_t out_features,
                                int64_t in_features, int K, int B, void *stream) {
    return pack_codes_common(packed, codes, out_features, in_features, K, B, stream, false);
}

aqlm_status_t aqlm_gemv_packed(const void *packed_codes, const void *packed_codebooks,
                               const void *x, void *y, int64_t out_features, int64_t in_features,
                               int K, int B, int batch, void *stream) {
    const void *c[1] = {packed_codes}, *cb[1] = {packed_codebooks};
    void *yy[1] = {y};
    const int64_t o[1] = {out_features};
    return aqlm_gemv_packed_grouped(1, c, cb, x, yy, o, in_features, K, B, batch, stream);
}

aqlm_status_t aqlm_gemv_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *stream) {
    aqlm::Problem p;
    const aqlm_status_t st = grouped_problem(n, codes, codebooks, x, y, out_features, in_features,
                                             K, B, batch, stream, false, &p);
    return st != AQLM_OK ? st : run(choose(false, p), p);
}

aqlm_status_t aqlm_gemm_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *stream) {
    aqlm::Problem p;
    const aqlm_status_t st = grouped_problem(n, codes, codebooks, x, y, out_features, in_features,
                                             K, B, batch, stream, false, &p);
    return st != AQLM_OK ? st : run(choose(true, p), p);
}

aqlm_status_t aqlm_gemv_packed_grouped(int n, const void *const *packed_codes,
                                       const void *const *packed_codebooks, const void *x,
                                       void *const *y, const int64_t *out_features,
                                       int64_t in_features, int K, int B, int batch,
                                       void *stream) {
    aqlm::Problem p;
    aqlm_status_t st = grouped_problem(n, packed_codes, packed_codebooks, x, y, out_features,
                                       in_features, K, B, batch, stream, true, &p);
    if (st != AQLM_OK) return st;
    const bool generic = forced_variant() == AQLM_VARIANT_GENERIC;
    const bool tiled = tiled_codes(K, B);
    const bool split = !generic && !tiled &&
                       all_segments(p, [](const aqlm::Problem &q) { return aqlm::ds_supported(q); });
    // batches the LDS-plane dot-product kernel does not take: the same planes on the
    // matrix cores
    const bool splitm = !generic && !tiled && !split &&
                        all_segments(p, [](const aqlm::Problem &q) { return aqlm::dsm_supported(q); });
    const bool lutp = !generic && tiled &&
                      all_segments(p, [](const aqlm::Problem &q) { return aqlm::lut_packed_supported(q); });
    if (!split && !splitm && !lutp && n > 1) {
        // unpacked one matrix at a time through the workspace (stream order keeps them apart)
        for (int m = 0; m < n; ++m) {
            st = aqlm_gemv_packed_grouped(1, packed_codes + m, packed_codebooks + m, x, y + m,
                                          out_features + m, in_features, K, B, batch, stream);
            if (st != AQLM_OK) return st;
        }
        return AQLM_OK;
    }
    const int64_t cbytes = out_features[0] * (in_features / kGroup) * K * (B / 8);
    const int64_t cbbytes = int64_t(K) * (int64_t(1) << B) * kGroup * 2;
    const size_t cb_off = (size_t(cbytes) + 255) / 256 * 256;
    // unpacked operands, then (matrix cores) that kernel's own workspace
    const size_t unpacked = tiled ? cb_off + size_t(cbbytes) : size_t(cbbytes);
    const size_t ops_off = (unpacked + 255) / 256 * 256;
    const bool gemm = !generic && batch >= mfma_min_batch(K);
    size_t mfma_ws = 0;
    if (!split && !splitm && !lutp && gemm) {
        const aqlm::Problem shape = make_problem(p.codes, p.codebooks, p.x, p.y, p.out, p.in, K,
                                                 B, batch, stream);
        // sized on the shape alone (the kernel's own pointers are checked at launch)
        if (aqlm::mfma_supported(shape)) mfma_ws = aqlm::mfma_workspace_bytes(shape);
    }
    const size_t need = split    ? aqlm::ds_workspace_bytes(p)
                        : splitm ? aqlm::dsm_workspace_bytes(p)
                        : lutp   ? aqlm::lut_packed_workspace_bytes(p)
                                 : ops_off + mfma_ws;
    void *ws = nullptr;
    hipError_t e = get_workspace(p.stream, need, &ws);
    if (e != hipSuccess) {
        set_error("workspace", e);
        return AQLM_ERR_HIP;
    }
    if (!ws) return AQLM_ERR_UNSUPPORTED;   // capturing stream without a workspace
    if (log_enabled())
        std::fprintf(stderr, "[aqlm] packed %s n=%d rows=%lld in=%lld K=%d B=%d batch=%d\n",
                     split ? "split" : splitm ? "split-mfma" : lutp ? "lut_packed" : "unpack+auto", n,
                     (long long)p.out,
                     (long long)p.in, K, B, batch);
    if (split || splitm || lutp) {
        e = split ? aqlm::launch_ds(p, ws) : splitm ? aqlm::launch_dsm(p, ws) : aqlm::launch_lut_packed(p, ws);
        if (e != hipSuccess) {
            set_error(split ? "split" : splitm ? "split-mfma" : "lut_packed", e);
            return AQLM_ERR_HIP;
        }
        return AQLM_OK;
    }
    // one matrix: unpack into the workspace and run as aqlm_gemv
    char *wsb = static_cast<char *>(ws);
    if (tiled) {
        e = aqlm::launch_pack_codes_lut(p.codes, wsb, p.out, p.in, false, p.stream);
        if (e != hipSuccess) {
            set_error("unpack_codes", e);
            return AQLM_ERR_HIP;
        }
    }
    void *cbws = tiled ? wsb + cb_off : wsb;
    e = aqlm::launch_unpack_codebooks(p.codebooks, cbws, K, B, p.stream);
    if (e != hipSuccess) {
        set_error("unpack_codebooks", e);
        return AQLM_ERR_HIP;
    }
    aqlm::Problem q = make_problem(tiled ? wsb : p.codes, cbws, p.x, p.y, p.out, p.in, K, B,
                                   batch, stream);
    if (gemm && aqlm::mfma_supported(q) && aqlm::mfma_workspace_bytes(q) <= mfma_ws) {
        // matrix cores, with their partial sums after the unpacked operands
        e = aqlm::launch_mfma(q, mfma_ws ? wsb + ops_off : nullptr);
        if (e != hipSuccess) {
            set_error("mfma", e);
            return AQLM_ERR_HIP;
        }
        return AQLM_OK;
    }
    int v = choose(false, q);
    // the workspace holds the operands: no kernel that needs one of its own
    if (v == AQLM_VARIANT_LUT || v == AQLM_VARIANT_MFMA) v = AQLM_VARIANT_LDS;
    if (v == AQLM_VARIANT_LDS && !supported(v, q)) v = AQLM_VARIANT_GENERIC;
    return run(v, q);
}

const char *aqlm_version(void) { return "0.4.0"; }

const char *aqlm_last_error(void) { return g_last_error; }

}  // extern "C"
