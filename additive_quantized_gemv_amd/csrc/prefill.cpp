// Prefill-size batches: W decoded once per call, then one library GEMM.
//
// At a few hundred tokens and more, the matrix-core kernels' per-token-tile decode
// and split partial sums cost more than decoding W once: launch_dequant16 writes the
// dense fp16 W (the bits aqlm_dequantize writes, the fold of the page "AQLM (Additive
// Quantization for LLMs)", section "Niveau intermediaire", rounded once) into the
// workspace, and hipBLASLt multiplies it with x in fp16 with fp32 accumulation, the
// same arithmetic as the matrix-core path.  The dense W lives only in the stream's
// workspace for the duration of the call.
//
// Layouts (hipBLASLt is column-major): y [batch][out] row-major is the column-major
// out x batch matrix Y^T = W x^T, with W [out][in] row-major = column-major in x out
// used transposed, and x [batch][in] row-major = column-major in x batch.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr size_t kGemmScratch = size_t(64) << 20;   // hipBLASLt's own workspace

size_t w_bytes(const Problem &p) {
    return (size_t(p.out) * size_t(p.in) * 2 + 255) / 256 * 256;
}

struct Plan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    bool ok = false;
};

std::mutex g_mutex;
std::map<int, hipblasLtHandle_t> g_handles;                               // per device
std::map<std::tuple<int, int64_t, int64_t, int>, Plan> g_plans;          // (device, out, in, batch)

// The handle of the current device and the cached plan for this shape (made on first use:
// descriptors and the heuristic's first algorithm).  Host work only, so it may run while
// the stream is being captured.
hipError_t plan_for(const Problem &p, hipblasLtHandle_t *handle, const Plan **plan) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mutex);
    auto h = g_handles.find(dev);
    if (h == g_handles.end()) {
        hipblasLtHandle_t nh = nullptr;
        if (hipblasLtCreate(&nh) != HIPBLAS_STATUS_SUCCESS) return hipErrorUnknown;
        h = g_handles.emplace(dev, nh).first;
    }
    *handle = h->second;
    Plan &pl = g_plans[std::make_tuple(dev, p.out, p.in, p.batch)];
    if (!pl.ok) {
        const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
        if (hipblasLtMatmulDescCreate(&pl.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatmulDescSetAttribute(pl.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&pl.a, HIP_R_16F, uint64_t(p.in), uint64_t(p.out), p.in) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&pl.b, HIP_R_16F, uint64_t(p.in), uint64_t(p.batch), p.in) !=
                HIPBLAS_STATUS_SUCCESS ||
            hipblasLtMatrixLayoutCreate(&pl.c, HIP_R_16F, uint64_t(p.out), uint64_t(p.batch), p.out) !=
                HIPBLAS_STATUS_SUCCESS)
            return hipErrorUnknown;
        hipblasLtMatmulPreference_t pref = nullptr;
        if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return hipErrorUnknown;
        const uint64_t ws = kGemmScratch;
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                              sizeof(ws));
        hipblasLtMatmulHeuristicResult_t res[1];
        int found = 0;
        const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(*handle, pl.desc, pl.a, pl.b, pl.c,
                                                                   pl.c, pref, 1, res, &found);
        hipblasLtMatmulPreferenceDestroy(pref);
        if (st != HIPBLAS_STATUS_SUCCESS || found < 1) return hipErrorNotSupported;
        pl.algo = res[0].algo;
        pl.ok = true;
    }
    *plan = &pl;
    return hipSuccess;
}

}  // namespace

size_t prefill_workspace_bytes(const Problem &p) { return w_bytes(p) + kGemmScratch; }

hipError_t launch_prefill(const Problem &p, void *workspace) {
    hipblasLtHandle_t handle = nullptr;
    const Plan *pl = nullptr;
    hipError_t e = plan_for(p, &handle, &pl);
    if (e != hipSuccess) return e;
    char *ws = static_cast<char *>(workspace);
    e = launch_dequant16(p, ws);
    if (e != hipSuccess) return e;
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st =
        hipblasLtMatmul(handle, pl->desc, &alpha, ws, pl->a, p.x, pl->b, &beta, p.y, pl->c, p.y,
                        pl->c, &pl->algo, ws + w_bytes(p), kGemmScratch, p.stream);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace aqlm
