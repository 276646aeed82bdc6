/*
 * aqlm_mi355x.h -- C ABI of libaqlm_mi355x: additive-quantized matrix-vector and
 * small-batch matrix-matrix products on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "AQLM (Additive Quantization for LLMs)", section
 * "Niveau intermediaire"; groups of 8 along the input axis from page
 * "AQLM -- ...", section "Kak eto rabotaet tekhnicheski?"):
 *
 *   W is never stored dense.  Row o, input group j (columns 8j .. 8j+7) is
 *       W[o][8j+t] = C_0[i_0(o,j)][t] + C_1[i_1(o,j)][t] + ... + C_{K-1}[i_{K-1}(o,j)][t]
 *   with K codebooks of 2^B entries of 8 fp16 values each, and the product is
 *       Y[b][o] = sum_i W[o][i] * X[b][i].
 *   Storage costs K*B/8 bits per weight (same section, bitrate formula):
 *   scheme 1x16 (K=1, B=16) and 2x8 (K=2, B=8) both give 2 bits per weight.
 *
 * Layouts (all tensors dense, row-major, in device memory, owned by the caller):
 *   codes     [out_features][in_features/8][K]   uint8 when B = 8, 16-bit unsigned
 *                                                (little-endian) when B = 16
 *   codebooks [K][2^B][8]                        fp16 (IEEE binary16)
 *   x         [batch][in_features]               fp16
 *   y         [batch][out_features]              fp16, written (round to nearest even)
 *   W         [out_features][in_features]        fp32 or fp16 (aqlm_dequantize only)
 *
 * Numerics: products are accumulated in fp32.  The decoded weight is the fp32
 * left fold C_0 + C_1 + ... in codebook order; aqlm_dequantize writes it exactly
 * (fp32) or rounded once to fp16 (nearest even).  The batched (MFMA) path feeds
 * that fp16 rounding of W to the matrix cores.
 *
 * Calls are asynchronous: work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and the call returns before it finishes.
 *
 * Ownership and memory: every pointer is caller-owned.  The library allocates no
 * device or host memory in any call, keeps no pointer after a call returns, keeps no
 * per-stream or per-device state and never synchronizes a stream: calls are
 * reentrant and may run concurrently on any streams (aqlm_gemv_packed_noalloc,
 * which works in a fixed device array of its own, is the one exception).  Kernels
 * that add partial results in a second pass, or that
 * re-lay out operands per call, use scratch memory the caller passes as `workspace`
 * (device memory, 256-byte aligned, disjoint from every operand, no initial contents
 * needed) of `workspace_bytes` bytes.  aqlm_workspace_bytes() and
 * aqlm_grouped_workspace_bytes() give the amount a call needs for its fastest
 * kernel, from the same arguments.  The kernel a call runs depends only on its
 * arguments (shapes, pointer alignment, workspace_bytes; the environment overrides
 * named below are read once per process), so a call captured into a HIP graph runs
 * exactly the kernels the same eager call runs.  The rule:
 *   - workspace_bytes == 0 (workspace may be NULL): the fastest kernel that needs
 *     no workspace (the same result within the stated tolerance, slower);
 *   - workspace_bytes >= what the fastest kernel needs: that kernel;
 *   - anything in between: AQLM_ERR_INVALID_ARGUMENT, nothing launched
 *     (aqlm_last_error() names the size needed).
 *   The products from packed weights need a workspace in every case.
 * A workspace may be reused by every call ordered after the previous one on the
 * same stream; calls that may run at the same time need separate workspaces.  A
 * graph that captured a call keeps using that call's workspace on every replay, so
 * the memory must outlive the graph, and graphs that share a workspace must not be
 * replayed concurrently.
 *
 * Errors: argument errors are reported synchronously, before any device work:
 * a null pointer, a size < 1, in_features not a multiple of 8, K outside
 * 1..8, B not 8 or 16, sizes whose byte counts overflow int64, an output
 * buffer that overlaps an input, or a workspace that is misaligned, overlaps an
 * operand or is too small.  A launch failure (no device, no gfx950 code object)
 * returns AQLM_ERR_HIP; aqlm_last_error() then gives the HIP message.  Tuned
 * kernels that cannot take a shape (rows not a multiple of 16 bytes, unaligned
 * operand pointers, too much LDS) are replaced by the next kernel in the library's
 * order that can (at the end, the generic kernel); AQLM_ERR_UNSUPPORTED comes only
 * from aqlm_gemv_variant and from aqlm_cpu_gemv on a host without AVX2.
 *
 * Environment (read once per process): AQLM_FORCE_VARIANT=<name> prefers a named
 * kernel where it can take the call; AQLM_MFMA_MIN_BATCH and AQLM_PREFILL_MIN_BATCH
 * move aqlm_gemm's batch thresholds; AQLM_LOG=1 prints each choice to stderr.
 */
#ifndef AQLM_MI355X_H
#define AQLM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AQLM_OK = 0,
    AQLM_ERR_INVALID_ARGUMENT = 1,
    AQLM_ERR_UNSUPPORTED = 2,
    AQLM_ERR_HIP = 3
} aqlm_status_t;

/* Kernel variants, for aqlm_gemv_variant and aqlm_variant_name. */
typedef enum {
    AQLM_VARIANT_AUTO = 0,    /* library's choice (what aqlm_gemv / aqlm_gemm do)          */
    AQLM_VARIANT_GENERIC = 1, /* any K in 1..8, B in {8,16}, any batch and shape             */
    AQLM_VARIANT_LDS = 2,     /* B = 8: codebooks staged in LDS, gather + fp32 dot, batch<=8 */
    AQLM_VARIANT_LUT = 3,     /* K = 2, B = 8, batch 1: per-group codebook.x lookup tables
                                 (workspace: slice partial sums)                        */
    AQLM_VARIANT_L2 = 4,      /* B = 16: codebook gathered through L2, batch <= 8            */
    AQLM_VARIANT_MFMA = 5,    /* decode to fp16 fragments + fp16 matrix cores, any batch;
                                 K in {1,2}, or K in {4,8} with B = 8; in/8 a multiple of 4
                                 (workspace above batch 32: input-split partial sums)   */
    AQLM_VARIANT_SPLIT = 6,   /* B = 16: a slice of the codebook per CU, batch <= 4
                                 (packed codebooks, or canonical ones packed into the
                                 workspace on each call); aqlm_gemv_packed also at batch
                                 5..16 on the matrix cores                               */
    AQLM_VARIANT_PREFILL = 7  /* prefill-size batches: W decoded once to fp16 in the
                                 workspace (out*in*2 bytes), then the dense fp16 GEMM
                                 kernel with fp32 accumulation; any K, B, in % 8 == 0;
                                 x and codebooks 16-byte aligned                         */
} aqlm_variant_t;

/* The call a workspace query is about (aqlm_workspace_bytes). */
typedef enum {
    AQLM_OP_GEMV = 0,         /* aqlm_gemv, aqlm_gemv_variant, aqlm_gemv_grouped          */
    AQLM_OP_GEMM = 1,         /* aqlm_gemm, aqlm_gemm_grouped                             */
    AQLM_OP_GEMV_PACKED = 2   /* aqlm_gemv_packed, aqlm_gemv_packed_grouped               */
} aqlm_op_t;

/*
 * y = W x for a batch of activation rows (token generation): the product the page
 * "AQLM (Additive Quantization for LLMs)", section "Niveau intermediaire", defines
 * through its codes and codebooks.  Picks a gather/lookup kernel for the
 * (K, B, batch, shape, workspace); never the matrix cores.  With a workspace,
 * 16-bit codes with K in {1,2} at batch <= 4 (aligned as AQLM_VARIANT_SPLIT needs)
 * take the codebook-split kernel (the codebooks packed into position pairs in the
 * workspace on each call, K MiB per matrix), and 2x8 at batch 1 the lookup-table
 * kernel; without one, the L2-gather and LDS-gather kernels.  From batch 2 aqlm_gemm
 * is faster (MI355X, 7B layer, 2x8: 44 against 116 us at batch 4): it decodes each
 * group once for all tokens on the matrix cores.
 * Arguments: device pointers as laid out above; out_features, in_features >= 1
 * with in_features % 8 == 0; K in 1..8; B in {8, 16}; batch >= 1; workspace and
 * workspace_bytes as in the header's ownership rule.
 */
aqlm_status_t aqlm_gemv(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The same product (page "AQLM (Additive Quantization for LLMs)", section "Niveau
 * intermediaire"; many tokens at once, the batched form the page "Extreme
 * Compression of Large Language Models via Additive Quantization", abstract,
 * compares against fp16) with the same arguments; from batch 2 (4 for eight
 * codebooks, 3 for 16-bit codes, which take the split kernel up to batch 2;
 * AQLM_MFMA_MIN_BATCH overrides the first two) it uses the decode-to-fp16 + MFMA
 * kernels, below that it behaves as aqlm_gemv.  From prefill-size batches (512 for
 * 16-bit codes or K >= 4, 1024 for 8-bit codes with K <= 2 when in_features is not a
 * multiple of 64; AQLM_PREFILL_MIN_BATCH overrides) W is instead decoded once into the
 * workspace as dense fp16 (out*in*2 bytes) and multiplied by one fp16 GEMM with fp32
 * accumulation.  8-bit codes with K <= 2 and in_features a multiple of 64 stay on the
 * matrix-core decode kernels at every batch.
 */
aqlm_status_t aqlm_gemm(const void *codes, const void *codebooks, const void *x, void *y,
                        int64_t out_features, int64_t in_features, int K, int B, int batch,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The product of aqlm_gemv (page "AQLM (Additive Quantization for LLMs)", section
 * "Niveau intermediaire") with a named kernel variant (benchmarks, A/B tests).
 * Returns AQLM_ERR_UNSUPPORTED, with nothing launched, if that variant cannot take
 * the arguments or needs more workspace than workspace_bytes (see
 * aqlm_variant_supported).  AQLM_VARIANT_AUTO behaves as aqlm_gemv.
 */
aqlm_status_t aqlm_gemv_variant(int variant, const void *codes, const void *codebooks,
                                const void *x, void *y, int64_t out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream);

/* 1 if aqlm_gemv_variant(variant, ...) would run for these arguments and a workspace of
 * workspace_bytes, else 0.  No device work. */
int aqlm_variant_supported(int variant, const void *codes, const void *codebooks, const void *x,
                           const void *y, int64_t out_features, int64_t in_features, int K,
                           int B, int batch, int64_t workspace_bytes);

/* The variant aqlm_gemv (gemm = 0) or aqlm_gemm (gemm = 1) would run for these
 * arguments and a workspace of workspace_bytes; -1 on an argument error (including a
 * workspace that is too small).  No device work. */
int aqlm_selected_variant(int gemm, const void *codes, const void *codebooks, const void *x,
                          const void *y, int64_t out_features, int64_t in_features, int K,
                          int B, int batch, int64_t workspace_bytes);

/*
 * Workspace bytes the call `op` (AQLM_OP_*) needs for its fastest kernel with these
 * arguments (0: none needed); `variant` is AQLM_VARIANT_AUTO, or a named variant for
 * aqlm_gemv_variant (0 if that variant cannot take the call).  For
 * AQLM_OP_GEMV_PACKED, `codes` / `codebooks` are the packed operands and variant must
 * be AQLM_VARIANT_AUTO.  The grouped form takes the arguments of the grouped calls.
 * Returns -1 on an argument error.  Host-only, no device work; the size depends on
 * the shapes and on the pointers' alignment only.
 */
int64_t aqlm_workspace_bytes(int op, int variant, const void *codes, const void *codebooks,
                             const void *x, const void *y, int64_t out_features,
                             int64_t in_features, int K, int B, int batch);
int64_t aqlm_grouped_workspace_bytes(int op, int n, const void *const *codes,
                                     const void *const *codebooks, const void *x, void *const *y,
                                     const int64_t *out_features, int64_t in_features, int K,
                                     int B, int batch);

/*
 * Dense W [out][in] from codes and codebooks, the decode rule of page "AQLM (Additive
 * Quantization for LLMs)", section "Niveau intermediaire" (W as the sum of one
 * codebook vector per codebook): w_dtype 0 writes the fp32 fold exactly, 1 writes it
 * rounded once to fp16 (nearest even).  Same argument rules as aqlm_gemv; W must not
 * overlap the inputs.  Needs no workspace.
 */
aqlm_status_t aqlm_dequantize(const void *codes, const void *codebooks, void *W, int w_dtype,
                              int64_t out_features, int64_t in_features, int K, int B,
                              void *stream);

/*
 * Packed codebook layouts (same bytes as the codebooks of page "AQLM (Additive
 * Quantization for LLMs)", section "Niveau intermediaire"; a one-time change of the
 * weights' layout, not part of the product).  B in {8, 16}; `packed` must not
 * overlap `codebooks`; both 2-byte aligned (4-byte for B = 16).
 * - B = 8: plane-major [K][8][256] fp16, packed[k][t][c] = codebooks[k][c][t].
 * - B = 16: position pairs [K][4][65536][2] fp16,
 *   packed[k][q][c][s] = codebooks[k][c][2q + s]: one 32-bit word holds positions
 *   2q and 2q+1 of an entry, so half of the code space of one position pair
 *   (32768 words = 128 KiB) fits the LDS of a CU.
 */
aqlm_status_t aqlm_pack_codebooks(const void *codebooks, void *packed, int K, int B, void *stream);

/* Exact inverse of aqlm_pack_codebooks (same page and section). */
aqlm_status_t aqlm_unpack_codebooks(const void *packed, void *codebooks, int K, int B,
                                    void *stream);

/*
 * Packed code layout (the codes of page "AQLM (Additive Quantization for LLMs)",
 * section "Niveau intermediaire", re-laid out once, like aqlm_pack_codebooks; not
 * part of the product).
 * - K = 2, B = 8: tiles of 8 rows x 64 groups.  With G = in/8, NQ = ceil(out/8)
 *   and S = ceil(G/64), tile (s, q) for s < S, q < NQ is 1024 bytes at byte
 *   offset (s*NQ + q) * 1024; its bytes 16*jl + 2*r and 16*jl + 2*r + 1 are the
 *   codes (codebook 0, codebook 1) of row 8q + r, group 64s + jl.  Rows >= out
 *   and groups >= G hold code 0.  Size S * NQ * 1024 bytes.  codes and packed
 *   must be 2-byte aligned.
 * - every other (K, B): the canonical layout itself (a copy).
 * aqlm_packed_codes_bytes returns the size, or -1 on bad arguments.  `packed`
 * must not overlap `codes`.  Asynchronous on `stream`.
 */
int64_t aqlm_packed_codes_bytes(int64_t out_features, int64_t in_features, int K, int B);
aqlm_status_t aqlm_pack_codes(const void *codes, void *packed, int64_t out_features,
                              int64_t in_features, int K, int B, void *stream);
/* Exact inverse of aqlm_pack_codes (padding is dropped). */
aqlm_status_t aqlm_unpack_codes(const void *packed, void *codes, int64_t out_features,
                                int64_t in_features, int K, int B, void *stream);

/*
 * The product of aqlm_gemv (page "AQLM (Additive Quantization for LLMs)", section
 * "Niveau intermediaire") from packed weights: codes from aqlm_pack_codes, codebooks
 * from aqlm_pack_codebooks.  Same y, same argument rules; a workspace of
 * aqlm_workspace_bytes(AQLM_OP_GEMV_PACKED, ...) bytes is required.
 * - 16-bit codes, K in {1,2}, batch <= 4, in_features <= 32768 / K (and batch x
 *   in_features/8 <= 14336 at batch 3..4): the position-split kernel
 *   (AQLM_VARIANT_SPLIT).  With one codebook at batch 1 (or 2 with in_features <=
 *   4096) each of the 8 workgroups of a row range holds one position pair for one
 *   half of the code space in LDS (codes of the other half read a zero word);
 *   otherwise each of K*8 workgroups holds one position of one codebook.  A second
 *   kernel adds their partial sums (workspace: K*8 x batch x out fp32).
 * - 16-bit codes, batch 5..16 (K = 1) or 5..8 (K = 2), in_features a multiple of 64,
 *   16-byte aligned pointers: the same split on the matrix cores, one position per
 *   workgroup (taken from the pairs while the table is staged; a small kernel first
 *   writes x transposed by position into the workspace).
 * - 2x8, batch 1, 16-byte aligned pointers: the lookup-table kernel reading
 *   the code tiles (1 KiB contiguous per wave load; workspace: slice partial sums).
 * - otherwise the packed operands are unpacked into the workspace and the product
 *   runs as aqlm_gemm does (matrix cores from batch 2, their partial sums after the
 *   operands), else as aqlm_gemv without a workspace.
 */
aqlm_status_t aqlm_gemv_packed(const void *packed_codes, const void *packed_codebooks,
                               const void *x, void *y, int64_t out_features, int64_t in_features,
                               int K, int B, int batch, void *workspace, int64_t workspace_bytes,
                               void *stream);

/*
 * aqlm_gemv_packed without a workspace argument, for callers that cannot allocate or
 * hold scratch memory (code under HIP graph capture without a memory pool of its
 * own, tight serving loops, harnesses that forbid allocation).  Same product,
 * arguments and kernels as aqlm_gemv_packed; the scratch is a fixed device array of
 * the library of aqlm_noalloc_scratch_bytes() = 16 MiB on each GPU, reserved when the
 * library's code is loaded on that GPU and held until the process ends.  Its address
 * is looked up on the first call on each device.  A call whose workspace need
 * (aqlm_workspace_bytes(AQLM_OP_GEMV_PACKED, ...)) exceeds that size returns
 * AQLM_ERR_INVALID_ARGUMENT with nothing launched (aqlm_last_error() gives both
 * sizes).  Every call on one GPU shares the array and leaves its contents behind
 * (the kernels need no initial contents): calls that may run at the same time on one
 * GPU (different streams, or graphs replayed concurrently) race on it and must be
 * ordered by the caller.  No call allocates or frees memory.
 */
aqlm_status_t aqlm_gemv_packed_noalloc(const void *packed_codes, const void *packed_codebooks,
                                       const void *x, void *y, int64_t out_features,
                                       int64_t in_features, int K, int B, int batch,
                                       void *stream);
int64_t aqlm_noalloc_scratch_bytes(void);

/*
 * Several products that read the same activations, in one launch: the linears of a
 * layer that share x (q, k, v; gate, up), each the product of page "AQLM (Additive
 * Quantization for LLMs)", section "Niveau intermediaire", with its own codes and
 * codebooks.  y_m = W_m x for m < n, 1 <= n <= 4, where W_m has out_features[m] rows,
 * codes codes[m] and codebooks codebooks[m]; in_features, K, B and batch are common.
 * codes, codebooks, y and out_features are host arrays of n entries (read during the
 * call only); each y[m] is [batch][out_features[m]] fp16.  Each matrix follows the
 * argument rules of aqlm_gemv; no y[m] may overlap x, any codes, any codebooks or
 * another y; the out_features must add up to at most 2^30.  The result equals n
 * separate calls; launches (and their fixed start-up time) are shared.  One workspace
 * serves the whole call (aqlm_grouped_workspace_bytes).  aqlm_gemv_grouped chooses
 * kernels as aqlm_gemv does, aqlm_gemm_grouped as aqlm_gemm, aqlm_gemv_packed_grouped
 * as aqlm_gemv_packed (packed codes and codebooks).
 */
aqlm_status_t aqlm_gemv_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream);
aqlm_status_t aqlm_gemm_grouped(int n, const void *const *codes, const void *const *codebooks,
                                const void *x, void *const *y, const int64_t *out_features,
                                int64_t in_features, int K, int B, int batch, void *workspace,
                                int64_t workspace_bytes, void *stream);
aqlm_status_t aqlm_gemv_packed_grouped(int n, const void *const *packed_codes,
                                       const void *const *packed_codebooks, const void *x,
                                       void *const *y, const int64_t *out_features,
                                       int64_t in_features, int K, int B, int batch,
                                       void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The same product on the host cores (token generation on the CPU): host pointers in
 * the canonical layouts of aqlm_gemv, y [batch][out] fp16 written by the call, which
 * returns when it is done.  fp32 arithmetic (16-bit codes with K in {1,2} and 8-bit codes
 * with K = 1: F16C decode + FMA; 2x8: the same decode over a per-call pair codebook
 * P[c0 + 256*c1] = C_0[c0] + C_1[c1] rounded once to fp16, as the matrix-core kernels
 * round the fold; 8-bit codes with K > 2: per-group codebook.x lookup tables and AVX-512
 * / AVX2 gathers; 16-bit codes with K > 2: scalar code), y rounded once to fp16; the
 * result meets the same bar against the exact product as the GPU kernels and does not
 * depend on `threads`.  threads <= 0: the OpenMP default.  AQLM_ERR_INVALID_ARGUMENT
 * for a null pointer, a size < 1, in_features not a multiple of 8, K outside 1..8, B
 * not 8 or 16 or out*in/8 or batch*in above 2^40 (no overlap check: y must not alias
 * an input); AQLM_ERR_UNSUPPORTED on a host without AVX2, FMA and F16C.  No device is
 * involved.  Its scratch (the pair codebook or lookup tables) is host memory owned
 * by the call and freed before it returns.
 * (Page "Extreme Compression of Large Language Models via Additive Quantization",
 * abstract: the method's token generation also runs on CPUs.)
 */
aqlm_status_t aqlm_cpu_gemv(const void *codes, const void *codebooks, const void *x, void *y,
                            int64_t out_features, int64_t in_features, int K, int B, int batch,
                            int threads);
/* Instruction set the CPU kernel uses on this host: "avx512", "avx2" or "none".  The
 * environment variable AQLM_CPU_ISA=avx2, read on each call, keeps an AVX-512 host on
 * the AVX2 kernels. */
const char *aqlm_cpu_isa(void);

/* K*B/group bits per weight: the bitrate formula of page "AQLM (Additive
 * Quantization for LLMs)", section "Niveau intermediaire". */
double aqlm_bits_per_weight(int K, int B, int group);

/* Bytes of codes for an out x in matrix, out * (in/8) * K * B/8 (the same formula
 * applied to the matrix's weights); -1 on bad arguments. */
int64_t aqlm_codes_bytes(int64_t out_features, int64_t in_features, int K, int B);

/* Bytes of codebooks, K * 2^B * 8 * 2 (K codebooks of 2^B fp16 vectors of length 8,
 * the codebook shape of the same section); -1 on bad arguments. */
int64_t aqlm_codebooks_bytes(int K, int B);

/* Static strings; never NULL. */
const char *aqlm_status_string(aqlm_status_t status);
const char *aqlm_variant_name(int variant);
const char *aqlm_version(void);

/* Text of the last error seen by this thread's calls: the HIP message after
 * AQLM_ERR_HIP, or what was wrong with a workspace ("" if none).  Each call that
 * launches work clears it first. */
const char *aqlm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AQLM_MI355X_H */
