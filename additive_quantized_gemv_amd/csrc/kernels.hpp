// Host-visible launchers of the gfx950 kernels (implemented in the *.hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aqlm {

// Up to kMaxSegs matrices that share x, in, K, B and batch, computed in one launch:
// matrix m owns global rows [row0[m], row0[m+1]) of the concatenated output.  A single
// product is a table of one.  aux0 is scratch for launchers: the first work unit
// (workgroup, row range or tile) of each matrix in the launch's own decomposition.
constexpr int kMaxSegs = 4;
struct Segs {
    int n;
    int row0[kMaxSegs + 1];
    int aux0[kMaxSegs + 1];
    const void *codes[kMaxSegs];
    const void *cb[kMaxSegs];
    void *y[kMaxSegs];
};


struct Problem {
    const void *codes;        // matrix 0 (the only one unless segs.n > 1)
    const void *codebooks;
    const void *x;
    void *y;
    int64_t out;              // total rows over all matrices
    int64_t in;
    int K;
    int B;
    int batch;
    hipStream_t stream;
    Segs segs;
};

// Every launcher returns the hipError_t of its launch (hipSuccess when queued).

// Sets the calling thread's aqlm_last_error() text (defined with the C ABI).
void set_last_error_message(const char *what);

// Generic: any K in 1..8, B in {8,16}, any batch, any in % 8 == 0.
hipError_t launch_generic(const Problem &p);

// Same over matrices: partial is [parts][batch][T] (T = segs.row0[segs.n]); for global row g of
// matrix m, y_m[b][g - row0[m]] = fp16(sum over parts, in order).
hipError_t launch_partial_sum_segs(const float *partial, const Segs &segs, int batch, int parts,
                                   hipStream_t s);
hipError_t launch_copy_bytes(const void *src, void *dst, int64_t n, hipStream_t s);

// Dense W (fp32 when w_fp16 == 0, fp16 otherwise).
hipError_t launch_dequantize(const Problem &p, void *W, int w_fp16);
// dense fp16 W ([out][in], 16-byte aligned) for the prefill path; same bits as
// launch_dequantize with w_fp16
hipError_t launch_dequant16(const Problem &p, void *W);
// prefill: W decoded once into the workspace (out*in fp16), then the dense fp16 GEMM
// kernel with fp32 accumulation
bool prefill_supported(const Problem &p);
size_t prefill_workspace_bytes(const Problem &p);
hipError_t launch_prefill(const Problem &p, void *workspace);

// Gather kernel for 8-bit codes (codebooks staged in LDS), batch <= 8.
bool gather_supported(const Problem &p);
hipError_t launch_gather(const Problem &p);

// Gather kernel for 16-bit codes (codebook through L2), K in {1,2}, batch <= 8.
bool l2_supported(const Problem &p);
hipError_t launch_l2(const Problem &p);

// Lookup-table kernel for K = 2, B = 8, batch 1 (split over input slices).
bool lut_supported(const Problem &p);
size_t lut_workspace_bytes(const Problem &p);
hipError_t launch_lut(const Problem &p, void *workspace);
// 2x8 lookup-table kernel over packed code tiles (8 rows x 64 groups) and plane-major codebooks
int64_t lut_packed_codes_bytes(int64_t out, int64_t in);
bool lut_packed_supported(const Problem &p);
size_t lut_packed_workspace_bytes(const Problem &p);
hipError_t launch_lut_packed(const Problem &p, void *workspace);
hipError_t launch_pack_codes_lut(const void *src, void *dst, int64_t out, int64_t in, bool pack,
                                 hipStream_t s);

// 16-bit codes with the codebook split by vector position (packed planes), batch <= 4.
bool ds_supported(const Problem &p);
size_t ds_workspace_bytes(const Problem &p);
hipError_t launch_ds(const Problem &p, void *workspace);
// the same from canonical codebooks (16-byte aligned): packed into the workspace first
size_t split_canonical_workspace_bytes(const Problem &p);
hipError_t launch_split_canonical(const Problem &p, void *workspace);
bool dsm_supported(const Problem &p);
size_t dsm_workspace_bytes(const Problem &p);
hipError_t launch_dsm(const Problem &p, void *workspace);
hipError_t launch_pack_codebooks(const void *cb, void *planes, int K, int B, hipStream_t s);
hipError_t launch_unpack_codebooks(const void *planes, void *cb, int K, int B, hipStream_t s);

// Decode-to-fp16 fragments + MFMA, K in {1,2}, B in {8,16}, any batch; the input
// axis may be split over workgroups (partial tiles in the workspace of
// mfma_workspace_bytes); with a null workspace it is not split.
bool mfma_supported(const Problem &p);
size_t mfma_workspace_bytes(const Problem &p);
hipError_t launch_mfma(const Problem &p, void *workspace);

}  // namespace aqlm
