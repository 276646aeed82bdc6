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
constexpr int kMfmaMinBatchDefault = 16;

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
    return AQLM_VARIANT_AUTO;
}

int mfma_min_batch() {
    const char *v = std::getenv("AQLM_MFMA_MIN_BATCH");
    if (!v || !*v) return kMfmaMinBatchDefault;
    const int n = std::atoi(v);
    return n >= 1 ? n : kMfmaMinBatchDefault;
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
    return aqlm::Problem{codes, cb, x, y, out, in, K, B, batch,
                         static_cast<hipStream_t>(stream)};
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

bool supported(int variant, const aqlm::Problem &p) {
    switch (variant) {
        case AQLM_VARIANT_GENERIC: return true;
        case AQLM_VARIANT_LDS: return p.B == 8 && aqlm::gather_supported(p);
        case AQLM_VARIANT_LUT: return aqlm::lut_supported(p);
        case AQLM_VARIANT_L2: return aqlm::l2_supported(p);
        case AQLM_VARIANT_MFMA: return aqlm::mfma_supported(p);
        default: return false;
    }
}

int choose(bool gemm, const aqlm::Problem &p) {
    const int forced = forced_variant();
    if (forced != AQLM_VARIANT_AUTO && supported(forced, p)) return forced;
    if (gemm && p.batch >= mfma_min_batch() && supported(AQLM_VARIANT_MFMA, p))
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
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 1u) ||
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
    switch (variant) {
        case AQLM_VARIANT_LDS: e = aqlm::launch_gather(p); break;
        case AQLM_VARIANT_L2: e = aqlm::launch_l2(p); break;
        case AQLM_VARIANT_LUT: {
            void *ws = nullptr;
            e = get_workspace(p.stream, aqlm::lut_workspace_bytes(p), &ws);
            if (e != hipSuccess) break;
            if (ws) {
                e = aqlm::launch_lut(p, ws);
            } else {
                // capturing stream without a workspace: same product, no workspace needed
                if (log_enabled())
                    std::fprintf(stderr, "[aqlm] lut: no workspace on a capturing stream, "
                                         "using the gather kernel\n");
                e = aqlm::gather_supported(p) ? aqlm::launch_gather(p) : aqlm::launch_generic(p);
            }
            break;
        }
        case AQLM_VARIANT_MFMA: {
            const size_t need = aqlm::mfma_workspace_bytes(p);
            void *ws = nullptr;
            if (need) {
                e = get_workspace(p.stream, need, &ws);
                if (e != hipSuccess) break;
                if (!ws) {
                    // capturing stream without a workspace: same product, no workspace needed
                    e = aqlm::launch_generic(p);
                    break;
                }
            }
            e = aqlm::launch_mfma(p, ws);
            break;
        }
        default: e = aqlm::launch_generic(p); break;
    }
    if (e != hipSuccess) {
        set_error(aqlm_variant_name(variant), e);
        return AQLM_ERR_HIP;
    }
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
    Sizes s;
    aqlm_status_t st = check_args(packed_codes, packed_codebooks, x, y, out_features, in_features,
                                  K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const int64_t pbytes = packed_codes_size(out_features, in_features, K, B);
    if (pbytes < 0 || overlaps(y, s.y, packed_codes, pbytes)) return AQLM_ERR_INVALID_ARGUMENT;
    aqlm::Problem p = make_problem(packed_codes, packed_codebooks, x, y, out_features, in_features,
                                   K, B, batch, stream);
    const bool generic = forced_variant() == AQLM_VARIANT_GENERIC;
    const bool tiled = tiled_codes(K, B);
    int path;  // 0: split kernel, 1: packed lookup-table kernel, 2: unpack into the workspace
    size_t need;
    const size_t cb_off = (size_t(s.codes) + 255) / 256 * 256;
    if (!generic && !tiled && aqlm::ds_supported(p)) {
        path = 0;
        need = aqlm::ds_workspace_bytes(p);
    } else if (!generic && tiled && aqlm::lut_packed_supported(p)) {
        path = 1;
        need = aqlm::lut_packed_workspace_bytes(p);
    } else {
        path = 2;
        need = tiled ? cb_off + size_t(s.codebooks) : size_t(s.codebooks);
    }
    void *ws = nullptr;
    hipError_t e = get_workspace(p.stream, need, &ws);
    if (e != hipSuccess) {
        set_error("workspace", e);
        return AQLM_ERR_HIP;
    }
    if (!ws) return AQLM_ERR_UNSUPPORTED;   // capturing stream without a workspace
    if (log_enabled())
        std::fprintf(stderr, "[aqlm] packed %s out=%lld in=%lld K=%d B=%d batch=%d\n",
                     path == 0 ? "split" : path == 1 ? "lut_packed" : "unpack+auto",
                     (long long)p.out, (long long)p.in, K, B, batch);
    if (path == 0 || path == 1) {
        e = path == 0 ? aqlm::launch_ds(p, ws) : aqlm::launch_lut_packed(p, ws);
        if (e != hipSuccess) {
            set_error(path == 0 ? "split" : "lut_packed", e);
            return AQLM_ERR_HIP;
        }
        return AQLM_OK;
    }
    char *wsb = static_cast<char *>(ws);
    if (tiled) {
        e = aqlm::launch_pack_codes_lut(packed_codes, wsb, out_features, in_features, false,
                                        p.stream);
        if (e != hipSuccess) {
            set_error("unpack_codes", e);
            return AQLM_ERR_HIP;
        }
        p.codes = wsb;
    }
    void *cbws = tiled ? wsb + cb_off : wsb;
    e = aqlm::launch_unpack_codebooks(packed_codebooks, cbws, K, B, p.stream);
    if (e != hipSuccess) {
        set_error("unpack_codebooks", e);
        return AQLM_ERR_HIP;
    }
    p.codebooks = cbws;
    int v = choose(false, p);
    if (v == AQLM_VARIANT_LUT) v = AQLM_VARIANT_LDS;   // the workspace holds the operands
    return run(v, p);
}

const char *aqlm_version(void) { return "0.3.0"; }

const char *aqlm_last_error(void) { return g_last_error; }

}  // extern "C"
