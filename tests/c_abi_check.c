/*
 * The library called from plain C, with no Python in the process: reads one problem
 * from a file, runs it through aqlm_gemv, aqlm_gemm and (packed) aqlm_gemv_packed on
 * device buffers of its own, and writes the three y to a file for the test to check
 * against the oracle.
 *
 * Input file:  int64 out, in, K, B, batch; then codes (out*in/8*K*B/8 bytes),
 *              codebooks (K*2^B*8 fp16), x (batch*in fp16).
 * Output file: y of aqlm_gemv, then of aqlm_gemm, then of aqlm_gemv_packed
 *              (each batch*out fp16).
 * Exit status: 0 on success; 1 on a usage or I/O error; 2 on an error from the
 * library or the HIP runtime (the message on stderr).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "aqlm_mi355x.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

#define AQLM_OK_(call)                                                                \
    do {                                                                              \
        aqlm_status_t s_ = (call);                                                    \
        if (s_ != AQLM_OK) {                                                          \
            fprintf(stderr, "%s: %s (%s)\n", #call, aqlm_status_string(s_),           \
                    aqlm_last_error());                                               \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

static void *read_all(FILE *f, size_t n) {
    void *p = malloc(n ? n : 1);
    if (p && fread(p, 1, n, f) != n) {
        free(p);
        return NULL;
    }
    return p;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <problem file> <y file>\n", argv[0]);
        return 1;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 1;
    int64_t hdr[5];
    if (fread(hdr, sizeof(int64_t), 5, f) != 5) return 1;
    const int64_t out = hdr[0], in = hdr[1];
    const int K = (int)hdr[2], B = (int)hdr[3], batch = (int)hdr[4];
    const int64_t code_bytes = aqlm_codes_bytes(out, in, K, B);
    const int64_t cb_bytes = aqlm_codebooks_bytes(K, B);
    if (code_bytes < 0 || cb_bytes < 0 || batch < 1) return 1;
    const size_t x_bytes = (size_t)batch * (size_t)in * 2, y_bytes = (size_t)batch * (size_t)out * 2;
    void *codes = read_all(f, (size_t)code_bytes), *cb = read_all(f, (size_t)cb_bytes);
    void *x = read_all(f, x_bytes);
    fclose(f);
    if (!codes || !cb || !x) return 1;

    const int64_t packed_bytes = aqlm_packed_codes_bytes(out, in, K, B);
    void *d_codes, *d_cb, *d_x, *d_y, *d_pcodes, *d_pcb;
    HIP_OK(hipMalloc(&d_codes, (size_t)code_bytes));
    HIP_OK(hipMalloc(&d_cb, (size_t)cb_bytes));
    HIP_OK(hipMalloc(&d_x, x_bytes));
    HIP_OK(hipMalloc(&d_y, y_bytes));
    HIP_OK(hipMalloc(&d_pcodes, (size_t)packed_bytes));
    HIP_OK(hipMalloc(&d_pcb, (size_t)cb_bytes));
    HIP_OK(hipMemcpy(d_codes, codes, (size_t)code_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cb, cb, (size_t)cb_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, x_bytes, hipMemcpyHostToDevice));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void *y = malloc(y_bytes * 3);
    if (!y) return 1;
    /* the caller owns the workspace: one buffer sized for the largest of the three calls */
    AQLM_OK_(aqlm_pack_codes(d_codes, d_pcodes, out, in, K, B, stream));
    AQLM_OK_(aqlm_pack_codebooks(d_cb, d_pcb, K, B, stream));
    const int64_t ws_gemv = aqlm_workspace_bytes(AQLM_OP_GEMV, AQLM_VARIANT_AUTO, d_codes, d_cb,
                                                 d_x, d_y, out, in, K, B, batch);
    const int64_t ws_gemm = aqlm_workspace_bytes(AQLM_OP_GEMM, AQLM_VARIANT_AUTO, d_codes, d_cb,
                                                 d_x, d_y, out, in, K, B, batch);
    const int64_t ws_packed = aqlm_workspace_bytes(AQLM_OP_GEMV_PACKED, AQLM_VARIANT_AUTO,
                                                   d_pcodes, d_pcb, d_x, d_y, out, in, K, B, batch);
    if (ws_gemv < 0 || ws_gemm < 0 || ws_packed <= 0) return 1;
    int64_t ws_bytes = ws_gemv > ws_gemm ? ws_gemv : ws_gemm;
    ws_bytes = ws_packed > ws_bytes ? ws_packed : ws_bytes;
    void *d_ws;
    HIP_OK(hipMalloc(&d_ws, (size_t)ws_bytes));
    AQLM_OK_(aqlm_gemv(d_codes, d_cb, d_x, d_y, out, in, K, B, batch, d_ws, ws_bytes, stream));
    HIP_OK(hipMemcpyAsync(y, d_y, y_bytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    AQLM_OK_(aqlm_gemm(d_codes, d_cb, d_x, d_y, out, in, K, B, batch, d_ws, ws_bytes, stream));
    HIP_OK(hipMemcpyAsync((char *)y + y_bytes, d_y, y_bytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));
    AQLM_OK_(aqlm_gemv_packed(d_pcodes, d_pcb, d_x, d_y, out, in, K, B, batch, d_ws, ws_bytes,
                              stream));
    HIP_OK(hipMemcpyAsync((char *)y + 2 * y_bytes, d_y, y_bytes, hipMemcpyDeviceToHost, stream));
    HIP_OK(hipStreamSynchronize(stream));

    FILE *o = fopen(argv[2], "wb");
    if (!o || fwrite(y, 1, y_bytes * 3, o) != y_bytes * 3) return 1;
    fclose(o);
    printf("c abi ok: %s, %lldx%lld %dx%d batch %d\n", aqlm_version(), (long long)out,
           (long long)in, K, B, batch);
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(d_codes));
    HIP_OK(hipFree(d_cb));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_pcodes));
    HIP_OK(hipFree(d_pcb));
    HIP_OK(hipFree(d_ws));
    free(codes);
    free(cb);
    free(x);
    free(y);
    return 0;
}
