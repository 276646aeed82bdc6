// C ABI of libaqlm_mi355x: argument checks, kernel choice, launch, error mapping.
// The operation and layouts are documented in include/aqlm_mi355x.h.
//
// The library holds no device memory and no per-stream state: every product call
// receives its scratch memory (partial sums, packed or unpacked operands) from the
// caller as `workspace`, and the kernel it runs is a function of its arguments alone
// (shapes, pointer alignment, workspace size, environment overrides read once), so
// an eager call and the same call captured into a HIP graph run the same kernels.
#include "aqlm_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

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
// Measured on MI355X (7B layer, seven separate calls, us, matrix cores against prefill):
// 16-bit codes b256 417 / 542, b512 732 / 576, b1024 1190 / 741 (decoding a 1 MiB codebook
// through L2 per token tile costs more).  8-bit codes with K <= 2 on the tiled kernel
// (inputs not a multiple of 64): b512 429 / 540, b1024 690 / 692, b2048 1387 / 1018.  On
// the kernel with DMA-staged operands (inputs a multiple of 64) the matrix cores stay
// ahead at every batch measured: b1024 584 / 681, b2048 912 / 1013, b4096 1795 / 1881.
constexpr int kPrefillMinBatch16 = 512;
constexpr int kPrefillMinBatch8 = 1024;
constexpr int kPrefillMinBatch8Staged = 1 << 30;
// The workspace is cut into fp32 / 16-byte-vector regions at 256-byte offsets.
constexpr uintptr_t kWorkspaceAlign = 256;
constexpr int64_t kUnlimited = INT64_MAX;

thread_local char g_last_error[256] = "";

void set_error(const char *what, hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
}

void set_message(const char *what) { std::snprintf(g_last_error, sizeof(g_last_error), "%s", what); }

bool log_enabled() {
    static const bool on = [] {
        const char *v = std::getenv("AQLM_LOG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

int forced_variant() {
    static const int forced = [] {
        const char *v = std::getenv("AQLM_FORCE_VARIANT");
        if (!v || !*v) return int(AQLM_VARIANT_AUTO);
        if (!std::strcmp(v, "generic")) return int(AQLM_VARIANT_GENERIC);
        if (!std::strcmp(v, "lds")) return int(AQLM_VARIANT_LDS);
        if (!std::strcmp(v, "lut")) return int(AQLM_VARIANT_LUT);
        if (!std::strcmp(v, "l2")) return int(AQLM_VARIANT_L2);
        if (!std::strcmp(v, "mfma")) return int(AQLM_VARIANT_MFMA);
        if (!std::strcmp(v, "split")) return int(AQLM_VARIANT_SPLIT);
        if (!std::strcmp(v, "prefill")) return int(AQLM_VARIANT_PREFILL);
        return int(AQLM_VARIANT_AUTO);
    }();
    return forced;
}

int env_batch(const char *name, int def) {
    const char *v = std::getenv(name);
    if (!v || !*v) return def;
    const int n = std::atoi(v);
    return n >= 1 ? n : def;
}

// batch from which aqlm_gemm decodes W once and runs one dense GEMM
// (AQLM_PREFILL_MIN_BATCH overrides)
int prefill_min_batch(const aqlm::Problem &p) {
    static const int b16 = env_batch("AQLM_PREFILL_MIN_BATCH", kPrefillMinBatch16);
    static const int b8 = env_batch("AQLM_PREFILL_MIN_BATCH", kPrefillMinBatch8);
    static const int b8s = env_batch("AQLM_PREFILL_MIN_BATCH", kPrefillMinBatch8Staged);
    if (p.B == 16 || p.K >= 4) return b16;
    return p.in % 64 == 0 ? b8s : b8;
}

int mfma_min_batch(int K) {
    static const int any = env_batch("AQLM_MFMA_MIN_BATCH", kMfmaMinBatch);
    static const int k8 = env_batch("AQLM_MFMA_MIN_BATCH", kMfmaMinBatch8Codebooks);
    return K >= 8 ? k8 : any;
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

bool supported_one(int variant, const aqlm::Problem &p) {
    switch (variant) {
        case AQLM_VARIANT_GENERIC: return true;
        case AQLM_VARIANT_LDS: return p.B == 8 && aqlm::gather_supported(p);
        case AQLM_VARIANT_LUT: return aqlm::lut_supported(p);
        case AQLM_VARIANT_L2: return aqlm::l2_supported(p);
        case AQLM_VARIANT_MFMA: return aqlm::mfma_supported(p);
        case AQLM_VARIANT_PREFILL: return aqlm::prefill_supported(p);
        case AQLM_VARIANT_SPLIT: return aqlm::ds_supported(p);
        default: return false;
    }
}

bool supported(int variant, const aqlm::Problem &p) {
    return all_segments(p, [variant](const aqlm::Problem &q) { return supported_one(variant, q); });
}

// Workspace bytes a variant needs for p (0: none).  Kernels without a matrix table
// (lds, generic, prefill) run a grouped problem one matrix at a time, in stream order,
// each reusing the whole workspace.
int64_t variant_need(int variant, const aqlm::Problem &p) {
    switch (variant) {
        case AQLM_VARIANT_LUT: return int64_t(aqlm::lut_workspace_bytes(p));
        case AQLM_VARIANT_MFMA: return int64_t(aqlm::mfma_workspace_bytes(p));
        case AQLM_VARIANT_SPLIT: return int64_t(aqlm::split_canonical_workspace_bytes(p));
        case AQLM_VARIANT_PREFILL: {
            int64_t n = 0;
            for (int m = 0; m < p.segs.n; ++m) {
                const int64_t s = int64_t(aqlm::prefill_workspace_bytes(segment(p, m)));
                n = s > n ? s : n;
            }
            return n;
        }
        default: return 0;
    }
}

// The fastest kernel for p whose workspace fits `ws_bytes` (0 or unlimited).  Without a
// workspace the matrix-core kernel runs unsplit (launch_mfma with a null workspace).
int choose_within(bool gemm, const aqlm::Problem &p, int64_t ws_bytes) {
    auto fits = [&](int v) {
        return supported(v, p) &&
               (variant_need(v, p) <= ws_bytes || (v == AQLM_VARIANT_MFMA && ws_bytes == 0));
    };
    const int forced = forced_variant();
    if (forced != AQLM_VARIANT_AUTO && fits(forced)) return forced;
    if (gemm && p.batch >= prefill_min_batch(p) && fits(AQLM_VARIANT_PREFILL))
        return AQLM_VARIANT_PREFILL;
    // 16-bit codes: the split kernel (codebook packed per call) up to batch 4, or 2 where
    // the matrix cores are allowed
    if (p.batch <= (gemm ? kSplitMaxBatchGemm : kSplitMaxBatch) && fits(AQLM_VARIANT_SPLIT))
        return AQLM_VARIANT_SPLIT;
    if (gemm && p.batch >= mfma_min_batch(p.K) && fits(AQLM_VARIANT_MFMA)) return AQLM_VARIANT_MFMA;
    if (fits(AQLM_VARIANT_LUT)) return AQLM_VARIANT_LUT;
    if (fits(AQLM_VARIANT_LDS)) return AQLM_VARIANT_LDS;
    if (fits(AQLM_VARIANT_L2)) return AQLM_VARIANT_L2;
    return AQLM_VARIANT_GENERIC;
}

// Kernel choice under the workspace rule: no workspace (0 bytes) selects among the
// kernels that need none; any other size must cover the fastest kernel's need.
// Returns the variant, or -1 (message set) when the workspace is too small.
int choose(bool gemm, const aqlm::Problem &p, int64_t ws_bytes) {
    if (ws_bytes == 0) return choose_within(gemm, p, 0);
    const int v = choose_within(gemm, p, kUnlimited);
    const int64_t need = variant_need(v, p);
    if (need > ws_bytes) {
        std::snprintf(g_last_error, sizeof(g_last_error),
                      "workspace of %lld bytes is too small: %s needs %lld (aqlm_workspace_bytes)",
                      (long long)ws_bytes, aqlm_variant_name(v), (long long)need);
        return -1;
    }
    return v;
}

// Checks the caller's workspace: size >= 0, a pointer when the size is positive,
// 256-byte aligned, and disjoint from every operand of p (codes_bytes[m] per matrix).
aqlm_status_t check_workspace(const void *ws, int64_t ws_bytes, const aqlm::Problem &p,
                              const int64_t *codes_bytes) {
    if (ws_bytes < 0 || (ws_bytes > 0 && !ws)) return AQLM_ERR_INVALID_ARGUMENT;
    if (ws_bytes == 0) return AQLM_OK;
    if (reinterpret_cast<uintptr_t>(ws) & (kWorkspaceAlign - 1)) {
        set_message("workspace must be 256-byte aligned");
        return AQLM_ERR_INVALID_ARGUMENT;
    }
    const int64_t cbbytes = int64_t(p.K) * (int64_t(1) << p.B) * kGroup * 2;
    bool clash = overlaps(ws, ws_bytes, p.x, int64_t(p.batch) * p.in * 2);
    for (int m = 0; m < p.segs.n && !clash; ++m) {
        const int64_t rows = p.segs.row0[m + 1] - p.segs.row0[m];
        clash = overlaps(ws, ws_bytes, p.segs.codes[m], codes_bytes[m]) ||
                overlaps(ws, ws_bytes, p.segs.cb[m], cbbytes) ||
                overlaps(ws, ws_bytes, p.segs.y[m], int64_t(p.batch) * rows * 2);
    }
    if (clash) {
        set_message("workspace overlaps an operand");
        return AQLM_ERR_INVALID_ARGUMENT;
    }
    return AQLM_OK;
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

// Launches `variant` for p with the workspace `ws` (at least variant_need bytes).
aqlm_status_t run(int variant, const aqlm::Problem &p, void *ws) {
    hipError_t e = hipSuccess;
    if (log_enabled())
        std::fprintf(stderr, "[aqlm] %s out=%lld in=%lld K=%d B=%d batch=%d n=%d\n",
                     aqlm_variant_name(variant), (long long)p.out, (long long)p.in, p.K, p.B,
                     p.batch, p.segs.n);
    // kernels without a matrix table run once per matrix
    if (p.segs.n > 1 && (variant == AQLM_VARIANT_LDS || variant == AQLM_VARIANT_GENERIC ||
                         variant == AQLM_VARIANT_PREFILL)) {
        for (int m = 0; m < p.segs.n; ++m) {
            const aqlm_status_t st = run(variant, segment(p, m), ws);
            if (st != AQLM_OK) return st;
        }
        return AQLM_OK;
    }
    switch (variant) {
        case AQLM_VARIANT_LDS: e = aqlm::launch_gather(p); break;
        case AQLM_VARIANT_L2: e = aqlm::launch_l2(p); break;
        case AQLM_VARIANT_LUT: e = aqlm::launch_lut(p, ws); break;
        case AQLM_VARIANT_MFMA: e = aqlm::launch_mfma(p, ws); break;   // null: unsplit
        case AQLM_VARIANT_SPLIT: e = aqlm::launch_split_canonical(p, ws); break;
        case AQLM_VARIANT_PREFILL: e = aqlm::launch_prefill(p, ws); break;
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
// codes are in the packed layout of aqlm_pack_codes.  code_bytes (n entries) receives
// each matrix's code bytes.
aqlm_status_t grouped_problem(int n, const void *const *codes, const void *const *codebooks,
                              const void *x, void *const *y, const int64_t *out_features,
                              int64_t in, int K, int B, int batch, void *stream, bool packed,
                              aqlm::Problem *out, int64_t *code_bytes) {
    if (n < 1 || n > aqlm::kMaxSegs || !codes || !codebooks || !y || !out_features)
        return AQLM_ERR_INVALID_ARGUMENT;
    int64_t total = 0;
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

// ---- products from packed weights ----------------------------------------------

enum PackedKind { kPackedSplit, kPackedSplitMfma, kPackedLut, kPackedUnpack };

// How a packed product runs and the workspace it needs.  kPackedUnpack: the packed
// operands of one matrix are unpacked into the workspace (codes at 0 when tiled, the
// codebooks at cb_off), and the matrix-core kernel's partial sums follow at ops_off.
struct PackedPlan {
    PackedKind kind;
    int64_t need;
    bool tiled, gemm;
    size_t cb_off, ops_off, mfma_ws;
};

PackedPlan packed_plan_one(const aqlm::Problem &p) {
    PackedPlan pl{};
    pl.kind = kPackedUnpack;
    pl.tiled = tiled_codes(p.K, p.B);
    const bool generic = forced_variant() == AQLM_VARIANT_GENERIC;
    const int64_t cbytes = p.out * (p.in / kGroup) * p.K * (p.B / 8);
    const int64_t cbbytes = int64_t(p.K) * (int64_t(1) << p.B) * kGroup * 2;
    pl.cb_off = (size_t(cbytes) + 255) / 256 * 256;
    const size_t unpacked = pl.tiled ? pl.cb_off + size_t(cbbytes) : size_t(cbbytes);
    pl.ops_off = (unpacked + 255) / 256 * 256;
    pl.gemm = !generic && p.batch >= mfma_min_batch(p.K);
    if (pl.gemm) {
        // the unpacked operands sit at 256-byte offsets of the workspace: sized on the
        // shape with aligned operands
        const char *base = reinterpret_cast<const char *>(uintptr_t(1) << 40);
        const aqlm::Problem q = make_problem(base, base, p.x, p.y, p.out, p.in, p.K, p.B,
                                             p.batch, p.stream);
        if (aqlm::mfma_supported(q)) pl.mfma_ws = aqlm::mfma_workspace_bytes(q);
    }
    pl.need = int64_t(pl.ops_off + pl.mfma_ws);
    return pl;
}

PackedPlan packed_plan(const aqlm::Problem &p) {
    PackedPlan pl{};
    const bool generic = forced_variant() == AQLM_VARIANT_GENERIC;
    pl.tiled = tiled_codes(p.K, p.B);
    const bool split = !generic && !pl.tiled &&
                       all_segments(p, [](const aqlm::Problem &q) { return aqlm::ds_supported(q); });
    // batches the LDS-plane dot-product kernel does not take: the same planes on the
    // matrix cores
    const bool splitm = !generic && !pl.tiled && !split &&
                        all_segments(p, [](const aqlm::Problem &q) { return aqlm::dsm_supported(q); });
    const bool lutp = !generic && pl.tiled &&
                      all_segments(p, [](const aqlm::Problem &q) { return aqlm::lut_packed_supported(q); });
    if (split || splitm || lutp) {
        pl.kind = split ? kPackedSplit : splitm ? kPackedSplitMfma : kPackedLut;
        pl.need = int64_t(split ? aqlm::ds_workspace_bytes(p)
                          : splitm ? aqlm::dsm_workspace_bytes(p)
                                   : aqlm::lut_packed_workspace_bytes(p));
        return pl;
    }
    if (p.segs.n == 1) return packed_plan_one(p);
    // several matrices unpacked one at a time through the same workspace
    pl.kind = kPackedUnpack;
    for (int m = 0; m < p.segs.n; ++m) {
        const int64_t nm = packed_plan_one(segment(p, m)).need;
        pl.need = nm > pl.need ? nm : pl.need;
    }
    return pl;
}

aqlm_status_t run_packed(const aqlm::Problem &p, const PackedPlan &pl, void *ws) {
    hipError_t e = hipSuccess;
    const char *name = pl.kind == kPackedSplit ? "split" : pl.kind == kPackedSplitMfma ? "split-mfma"
                     : pl.kind == kPackedLut ? "lut_packed" : "unpack+auto";
    if (log_enabled())
        std::fprintf(stderr, "[aqlm] packed %s n=%d rows=%lld in=%lld K=%d B=%d batch=%d\n", name,
                     p.segs.n, (long long)p.out, (long long)p.in, p.K, p.B, p.batch);
    if (pl.kind != kPackedUnpack) {
        e = pl.kind == kPackedSplit ? aqlm::launch_ds(p, ws)
          : pl.kind == kPackedSplitMfma ? aqlm::launch_dsm(p, ws) : aqlm::launch_lut_packed(p, ws);
        if (e != hipSuccess) {
            set_error(name, e);
            return AQLM_ERR_HIP;
        }
        return AQLM_OK;
    }
    if (p.segs.n > 1) {
        // one matrix at a time through the workspace (stream order keeps them apart)
        for (int m = 0; m < p.segs.n; ++m) {
            const aqlm::Problem q = segment(p, m);
            const aqlm_status_t st = run_packed(q, packed_plan_one(q), ws);
            if (st != AQLM_OK) return st;
        }
        return AQLM_OK;
    }
    char *wsb = static_cast<char *>(ws);
    if (pl.tiled) {
        e = aqlm::launch_pack_codes_lut(p.codes, wsb, p.out, p.in, false, p.stream);
        if (e != hipSuccess) {
            set_error("unpack_codes", e);
            return AQLM_ERR_HIP;
        }
    }
    void *cbws = pl.tiled ? wsb + pl.cb_off : wsb;
    e = aqlm::launch_unpack_codebooks(p.codebooks, cbws, p.K, p.B, p.stream);
    if (e != hipSuccess) {
        set_error("unpack_codebooks", e);
        return AQLM_ERR_HIP;
    }
    aqlm::Problem q = make_problem(pl.tiled ? wsb : p.codes, cbws, p.x, p.y, p.out, p.in, p.K, p.B,
                                   p.batch, p.stream);
    if (pl.gemm && aqlm::mfma_supported(q) && aqlm::mfma_workspace_bytes(q) <= pl.mfma_ws) {
        // matrix cores, with their partial sums after the unpacked operands
        e = aqlm::launch_mfma(q, pl.mfma_ws ? wsb + pl.ops_off : nullptr);
        if (e != hipSuccess) {
            set_error("mfma", e);
            return AQLM_ERR_HIP;
        }
        return AQLM_OK;
    }
    // the workspace holds the operands: a kernel that needs no workspace of its own
    return run(choose_within(false, q, 0), q, nullptr);
}

// A product call: checks, kernel choice under the workspace rule, launch.
aqlm_status_t product(bool gemm, const aqlm::Problem &p, const int64_t *code_bytes, void *ws,
                      int64_t ws_bytes) {
    const aqlm_status_t st = check_workspace(ws, ws_bytes, p, code_bytes);
    if (st != AQLM_OK) return st;
    const int v = choose(gemm, p, ws_bytes);
    if (v < 0) return AQLM_ERR_INVALID_ARGUMENT;
    // no workspace: a null pointer, which also keeps the matrix-core kernel unsplit
    return run(v, p, ws_bytes ? ws : nullptr);
}

aqlm_status_t packed_product(const aqlm::Problem &p, const int64_t *code_bytes, void *ws,
                             int64_t ws_bytes) {
    const aqlm_status_t st = check_workspace(ws, ws_bytes, p, code_bytes);
    if (st != AQLM_OK) return st;
    const PackedPlan pl = packed_plan(p);
    if (pl.need > ws_bytes) {
        std::snprintf(g_last_error, sizeof(g_last_error),
                      "workspace of %lld bytes is too small: the packed product needs %lld "
                      "(aqlm_workspace_bytes)", (long long)ws_bytes, (long long)pl.need);
        return AQLM_ERR_INVALID_ARGUMENT;
    }
    return run_packed(p, pl, ws);
}

// Workspace bytes of an (op, variant) call on a validated problem; -1 if the op is unknown.
int64_t workspace_need(int op, int variant, const aqlm::Problem &p) {
    switch (op) {
        case AQLM_OP_GEMV:
        case AQLM_OP_GEMM:
            if (variant == AQLM_VARIANT_AUTO)
                return variant_need(choose_within(op == AQLM_OP_GEMM, p, kUnlimited), p);
            return supported(variant, p) ? variant_need(variant, p) : 0;
        case AQLM_OP_GEMV_PACKED:
            return variant == AQLM_VARIANT_AUTO ? packed_plan(p).need : -1;
        default: return -1;
    }
}

}  // namespace

namespace aqlm {
void set_last_error_message(const char *what) { set_message(what); }
}  // namespace aqlm

extern "C" {

aqlm_status_t aqlm_gemv(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *workspace, int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    return product(false, p, &s.codes, workspace, workspace_bytes);
}

aqlm_status_t aqlm_gemm(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *workspace, int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    return product(true, p, &s.codes, workspace, workspace_bytes);
}

aqlm_status_t aqlm_gemv_variant(int variant, const void *codes, const void *codebooks,
                                const void *x, void *y, int64_t out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    Sizes s;
    aqlm_status_t st = check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s);
    if (st != AQLM_OK) return st;
    const aqlm::Problem p = make_problem(codes, codebooks, x, y, out_features, in_features, K, B,
                                         batch, stream);
    if (variant == AQLM_VARIANT_AUTO) return product(false, p, &s.codes, workspace, workspace_bytes);
    st = check_workspace(workspace, workspace_bytes, p, &s.codes);
    if (st != AQLM_OK) return st;
    if (!supported(variant, p)) return AQLM_ERR_UNSUPPORTED;
    if (variant_need(variant, p) > workspace_bytes) {
        // the matrix-core kernel also runs unsplit without a workspace
        if (variant != AQLM_VARIANT_MFMA || workspace_bytes != 0) return AQLM_ERR_UNSUPPORTED;
        workspace = nullptr;
    }
    return run(variant, p, workspace_bytes ? workspace : nullptr);
}

int aqlm_variant_supported(int variant, const void *codes, const void *codebooks, const void *x,
                           const void *y, int64_t out_features, int64_t in_features, int K, int B,
                           int batch, int64_t workspace_bytes) {
    Sizes s;
    if (check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s) != AQLM_OK)
        return 0;
    const aqlm::Problem p = make_problem(codes, codebooks, x, const_cast<void *>(y), out_features,
                                         in_features, K, B, batch, nullptr);
    if (variant == AQLM_VARIANT_AUTO) return 1;
    if (!supported(variant, p)) return 0;
    return variant_need(variant, p) <= workspace_bytes ||
           (variant == AQLM_VARIANT_MFMA && workspace_bytes == 0);
}

int aqlm_selected_variant(int gemm, const void *codes, const void *codebooks, const void *x,
                          const void *y, int64_t out_features, int64_t in_features, int K, int B,
                          int batch, int64_t workspace_bytes) {
    Sizes s;
    if (check_args(codes, codebooks, x, y, out_features, in_features, K, B, batch, &s) != AQLM_OK ||
        workspace_bytes < 0)
        return -1;
    const aqlm::Problem p = make_problem(codes, codebooks, x, const_cast<void *>(y), out_features,
                                         in_features, K, B, batch, nullptr);
    return choose(gemm != 0, p, workspace_bytes);
}

int64_t aqlm_grouped_workspace_bytes(int op, int n, const void *const *codes,
                                     const void *const *codebooks, const void *x, void *const *y,
                                     const int64_t *out_features, int64_t in_features, int K,
                                     int B, int batch) {
    aqlm::Problem p;
    int64_t cbytes[aqlm::kMaxSegs];
    if (grouped_problem(n, codes, codebooks, x, y, out_features, in_features, K, B, batch, nullptr,
                        op == AQLM_OP_GEMV_PACKED, &p, cbytes) != AQLM_OK)
        return -1;
    return workspace_need(op, AQLM_VARIANT_AUTO, p);
}

int64_t aqlm_workspace_bytes(int op, int variant, const void *codes, const void *codebooks,
                             const void *x, const void *y, int64_t out_features,
                             int64_t in_features, int K, int B, int batch) {
    const void *c[1] = {codes}, *cb[1] = {codebooks};
    void *yy[1] = {const_cast<void *>(y)};
    const int64_t o[1] = {out_features};
    aqlm::Problem p;
    int64_t cbytes[1];
    if (grouped_problem(1, c, cb, x, yy, o, in_features, K, B, batch, nullptr,
                        op == AQLM_OP_GEMV_PACKED, &p, cbytes) != AQLM_OK)
        return -1;
    return workspace_need(op, variant, p);
}

aqlm_status_t aqlm_dequantize(const void *codes, const void *codebooks, void *W, int w_dtype,
                              int64_t out_features, int64_t in_features, int K, int B,
                              void *stream) {
    g_last_error[0] = 0;
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
    g_last_error[0] = 0;
    return pack_common(codebooks, packed, K, B, stream, true);
}

aqlm_status_t aqlm_unpack_codebooks(const void *packed, void *codebooks, int K, int B,
                                    void *stream) {
    g_last_error[0] = 0;
    return pack_common(packed, codebooks, K, B, stream, false);
}

int64_t aqlm_packed_codes_bytes(int64_t out_features, int64_t in_features, int K, int B) {
    return packed_codes_size(out_features, in_features, K, B);
}

static aqlm_status_t pack_codes_common(const void *src, void *dst, int64_t out, int64_t in, int K,
                                       int B, void *stream, bool pack) {
    g_last_error[0] = 0;
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
                               int K, int B, int batch, void *workspace, int64_t workspace_bytes,
                               void *stream) {
    const void *c[1] = {packed_codes}, *cb[1] = {packed_codebooks};
    void *yy[1] = {y};
    const int64_t o[1] = {out_features};
    return aqlm_gemv_packed_grouped(1, c, cb, x, yy, o, in_features, K, B, batch, workspace,
                                    workspace_bytes, stream);
}

aqlm_status_t aqlm_gemv_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    aqlm::Problem p;
    int64_t cbytes[aqlm::kMaxSegs];
    const aqlm_status_t st = grouped_problem(n, codes, codebooks, x, y, out_features, in_features,
                                             K, B, batch, stream, false, &p, cbytes);
    return st != AQLM_OK ? st : product(false, p, cbytes, workspace, workspace_bytes);
}

aqlm_status_t aqlm_gemm_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    aqlm::Problem p;
    int64_t cbytes[aqlm::kMaxSegs];
    const aqlm_status_t st = grouped_problem(n, codes, codebooks, x, y, out_features, in_features,
                                             K, B, batch, stream, false, &p, cbytes);
    return st != AQLM_OK ? st : product(true, p, cbytes, workspace, workspace_bytes);
}

aqlm_status_t aqlm_gemv_packed_grouped(int n, const void *const *packed_codes,
                                       const void *const *packed_codebooks, const void *x,
                                       void *const *y, const int64_t *out_features,
                                       int64_t in_features, int K, int B, int batch,
                                       void *workspace, int64_t workspace_bytes, void *stream) {
    g_last_error[0] = 0;
    aqlm::Problem p;
    int64_t cbytes[aqlm::kMaxSegs];
    const aqlm_status_t st = grouped_problem(n, packed_codes, packed_codebooks, x, y, out_features,
                                             in_features, K, B, batch, stream, true, &p, cbytes);
    return st != AQLM_OK ? st : packed_product(p, cbytes, workspace, workspace_bytes);
}

const char *aqlm_version(void) { return "0.5.0"; }

const char *aqlm_last_error(void) { return g_last_error; }

}  // extern "C"
