// Generic additive-quantized GEMV and the dequantize kernel (gfx950).
//
// Decode rule (page "AQLM (Additive Quantization for LLMs)", section "Niveau
// intermediaire"): group j of row o is the sum of one 8-wide fp16 vector from
// each of the K codebooks.  Here the sum is the fp32 left fold in codebook
// order, which is also what the dense dequantized W holds.
//
// The generic kernel is the always-correct fallback: one wave per output row,
// lanes striding over the row's groups, codebooks read through the caches,
// fp32 accumulation, DPP wave reduction, one fp16 store per (token, row).
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kGenericTokens = 8;  // tokens accumulated per pass over a row

__device__ __forceinline__ uint32_t read_code(const void *codes, int B, int64_t idx) {
    return B == 8 ? static_cast<uint32_t>(static_cast<const uint8_t *>(codes)[idx])
                  : static_cast<uint32_t>(static_cast<const uint16_t *>(codes)[idx]);
}

// Fold the K codebook vectors of group (o, j) into w[0..7] (fp32, codebook order).
__device__ __forceinline__ void decode_group(const void *codes, const uint16_t *cb, int K, int B,
                                             int64_t G, int64_t o, int64_t j, float w[8]) {
    const int64_t entries = int64_t(1) << B;
    const int64_t base = (o * G + j) * K;
    for (int k = 0; k < K; ++k) {
        const uint32_t c = read_code(codes, B, base + k);
        const uint16_t *v = cb + (k * entries + c) * kGroup;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float f = h2f(v[t]);
            w[t] = (k == 0) ? f : w[t] + f;
        }
    }
}

__global__ void __launch_bounds__(256)
generic_kernel(const void *__restrict__ codes, const uint16_t *__restrict__ cb,
               const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int64_t out,
               int64_t in, int K, int B, int batch) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t o = int64_t(blockIdx.x) * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (o >= out) return;
    const int64_t G = in / kGroup;
    for (int b0 = 0; b0 < batch; b0 += kGenericTokens) {
        const int nb = min(kGenericTokens, batch - b0);
        float acc[kGenericTokens];
#pragma unroll
        for (int b = 0; b < kGenericTokens; ++b) acc[b] = 0.0f;
        for (int64_t j = lane; j < G; j += kWave) {
            float w[8];
            decode_group(codes, cb, K, B, G, o, j, w);
#pragma unroll
            for (int b = 0; b < kGenericTokens; ++b) {
                if (b < nb) {
                    const uint16_t *xv = x + (b0 + b) * in + j * kGroup;
#pragma unroll
                    for (int t = 0; t < 8; ++t) acc[b] = fmaf(w[t], h2f(xv[t]), acc[b]);
                }
            }
        }
#pragma unroll
        for (int b = 0; b < kGenericTokens; ++b) {
            if (b < nb) {
                const float s = wave_sum(acc[b]);
                if (lane == 0) y[(b0 + b) * out + o] = f2h_bits(s);
            }
        }
    }
}

__global__ void __launch_bounds__(256)
dequantize_kernel(const void *__restrict__ codes, const uint16_t *__restrict__ cb, void *W,
                  int64_t out, int64_t in, int K, int B, int w_fp16) {
    const int64_t G = in / kGroup;
    const int64_t n = out * G;
    for (int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < n;
         g += int64_t(gridDim.x) * blockDim.x) {
        const int64_t o = g / G, j = g - o * G;
        float w[8];
        decode_group(codes, cb, K, B, G, o, j, w);
        if (w_fp16) {
            uint16_t *dst = static_cast<uint16_t *>(W) + g * kGroup;
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[t] = f2h_bits(w[t]);
        } else {
            float *dst = static_cast<float *>(W) + g * kGroup;
#pragma unroll
            for (int t = 0; t < 8; ++t) dst[t] = w[t];
        }
    }
}

// y_m[b][g - row0[m]] = fp16(sum over parts, in order, of partial[part][b][g]) for every
// global row g < T of matrix m and token b; partial is [parts][batch][T].
// PMAX > 0 (parts <= PMAX): every part's load is issued before the first add (the part
// index clamped, the value masked after), so a thread waits for memory once whatever the
// number of parts (a 4096 x 11008 2x8 product has 22 slices: measured on MI355X, 7.59
// against 8.27 us per call with loads in rounds of 8); one wave per workgroup.  PMAX = 0:
// any number of parts, in rounds of 8 loads.
template <int NS, int PMAX>
__global__ void __launch_bounds__(PMAX > 0 ? 64 : 256)
partial_sum_segs_kernel(const float *__restrict__ partial, int batch, int parts, const Segs segs) {
    const int T = seg_total<NS>(segs.n, segs.row0);
    const int64_t n = int64_t(batch) * T;
    const int g = blockIdx.x * blockDim.x + threadIdx.x;   // global row; token b = blockIdx.y
    const int b = blockIdx.y;
    if (g >= T) return;
    const int64_t i = int64_t(b) * T + g;
    float s = 0.0f;
    if constexpr (PMAX > 0) {
        float v[PMAX];
#pragma unroll
        for (int q = 0; q < PMAX; ++q) v[q] = partial[int64_t(min(q, parts - 1)) * n + i];
#pragma unroll
        for (int q = 0; q < PMAX; ++q) s += q < parts ? v[q] : 0.0f;
    } else {
        for (int p0 = 0; p0 < parts; p0 += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (p0 + q < parts) ? partial[int64_t(p0 + q) * n + i] : 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) s += v[q];
        }
    }
    const int m = seg_of<NS>(segs.n, segs.row0, g);
    const int out_m = pick(segs.row0, m + 1) - pick(segs.row0, m);
    static_cast<uint16_t *>(pick(segs.y, m))[int64_t(b) * out_m + (g - pick(segs.row0, m))] = f2h_bits(s);
}

// One matrix: y[i] = fp16(sum over parts, in order, of partial[part][i]), i < n = batch * out;
// PMAX as above.
template <int PMAX>
__global__ void __launch_bounds__(PMAX > 0 ? 64 : 256)
partial_sum_kernel(const float *__restrict__ partial, uint16_t *__restrict__ y, int n, int parts) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.0f;
    if constexpr (PMAX > 0) {
        float v[PMAX];
#pragma unroll
        for (int q = 0; q < PMAX; ++q) v[q] = partial[size_t(min(q, parts - 1)) * n + i];
#pragma unroll
        for (int q = 0; q < PMAX; ++q) s += q < parts ? v[q] : 0.0f;
    } else {
        for (int p0 = 0; p0 < parts; p0 += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (p0 + q < parts) ? partial[size_t(p0 + q) * n + i] : 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) s += v[q];
        }
    }
    y[i] = f2h_bits(s);
}

// Batched sums, four consecutive rows of one token per thread (16-byte loads, one 8-byte
// store): with one output per thread the 1.6 M outputs of a batch-128 12288-row sum run as
// ~24,000 waves of two loads each, in several latency-bound rounds.  Needs T, every
// matrix's first row and each y_m 4-element aligned (the launcher checks); parts added in
// order as above.
template <int NS, int PMAX>
__global__ void __launch_bounds__(64)
partial_sum4_kernel(const float *__restrict__ partial, int batch, int parts, const Segs segs) {
    const int T = seg_total<NS>(segs.n, segs.row0);
    const int64_t n = int64_t(batch) * T;
    const int g = (blockIdx.x * blockDim.x + threadIdx.x) * 4;   // first of four global rows
    const int b = blockIdx.y;
    if (g >= T) return;
    const int64_t i = int64_t(b) * T + g;
    float4 v[PMAX];
#pragma unroll
    for (int q = 0; q < PMAX; ++q)
        v[q] = *reinterpret_cast<const float4 *>(partial + int64_t(min(q, parts - 1)) * n + i);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
        const bool in = q < parts;
        s0 += in ? v[q].x : 0.0f;
        s1 += in ? v[q].y : 0.0f;
        s2 += in ? v[q].z : 0.0f;
        s3 += in ? v[q].w : 0.0f;
    }
    const int m = seg_of<NS>(segs.n, segs.row0, g);
    const int out_m = pick(segs.row0, m + 1) - pick(segs.row0, m);
    uint16_t *dst = static_cast<uint16_t *>(pick(segs.y, m)) + int64_t(b) * out_m + (g - pick(segs.row0, m));
    *reinterpret_cast<uint2 *>(dst) = uint2{f2h_bits(s0) | (uint32_t(f2h_bits(s1)) << 16),
                                            f2h_bits(s2) | (uint32_t(f2h_bits(s3)) << 16)};
}

// the four-row form applies: more than one token, and every row range and output row
// 4-element aligned
bool psum4_fits(const float *partial, const Segs &segs, int batch) {
    if (batch < 2 || (reinterpret_cast<uintptr_t>(partial) & 15u)) return false;
    for (int m = 0; m <= segs.n; ++m)
        if (segs.row0[m] % 4) return false;
    for (int m = 0; m < segs.n; ++m)
        if (reinterpret_cast<uintptr_t>(segs.y[m]) & 7u) return false;
    return true;
}

template <int PMAX>
void launch_psum4(const float *partial, const Segs &segs, int batch, int parts, hipStream_t s) {
    const int T = segs.row0[segs.n];
    const dim3 grid(unsigned((T / 4 + 63) / 64), unsigned(batch));
    if (segs.n == 1)
        hipLaunchKernelGGL((partial_sum4_kernel<1, PMAX>), grid, dim3(64), 0, s, partial, batch, parts, segs);
    else
        hipLaunchKernelGGL((partial_sum4_kernel<kMaxSegs, PMAX>), grid, dim3(64), 0, s, partial, batch,
                           parts, segs);
}

template <int PMAX>
void launch_psum(const float *partial, const Segs &segs, int batch, int parts, hipStream_t s) {
    constexpr int TPB = PMAX > 0 ? 64 : 256;
    const int T = segs.row0[segs.n];
    const dim3 grid(unsigned((T + TPB - 1) / TPB), unsigned(batch));
    if (segs.n == 1 && int64_t(batch) * T <= INT32_MAX - TPB) {
        const int n = batch * T;   // [batch][out] is one flat range
        hipLaunchKernelGGL(partial_sum_kernel<PMAX>, dim3(unsigned((n + TPB - 1) / TPB)), dim3(TPB), 0, s,
                           partial, static_cast<uint16_t *>(segs.y[0]), n, parts);
    } else if (segs.n == 1) {
        hipLaunchKernelGGL((partial_sum_segs_kernel<1, PMAX>), grid, dim3(TPB), 0, s, partial, batch,
                           parts, segs);
    } else {
        hipLaunchKernelGGL((partial_sum_segs_kernel<kMaxSegs, PMAX>), grid, dim3(TPB), 0, s, partial,
                           batch, parts, segs);
    }
}

}  // namespace

hipError_t launch_partial_sum_segs(const float *partial, const Segs &segs, int batch, int parts,
                                   hipStream_t s) {
    if (parts <= 32 && psum4_fits(partial, segs, batch)) {
        if (parts <= 2) launch_psum4<2>(partial, segs, batch, parts, s);
        else if (parts <= 4) launch_psum4<4>(partial, segs, batch, parts, s);
        else if (parts <= 8) launch_psum4<8>(partial, segs, batch, parts, s);
        else if (parts <= 16) launch_psum4<16>(partial, segs, batch, parts, s);
        else launch_psum4<32>(partial, segs, batch, parts, s);
        return hipGetLastError();
    }
    if (parts <= 8) launch_psum<8>(partial, segs, batch, parts, s);
    else if (parts <= 16) launch_psum<16>(partial, segs, batch, parts, s);
    else if (parts <= 24) launch_psum<24>(partial, segs, batch, parts, s);
    else if (parts <= 32) launch_psum<32>(partial, segs, batch, parts, s);
    else if (parts <= 64) launch_psum<64>(partial, segs, batch, parts, s);
    else launch_psum<0>(partial, segs, batch, parts, s);
    return hipGetLastError();
}

// byte copy, 16 bytes per thread where both pointers allow it
__global__ void __launch_bounds__(256)
copy_bytes_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool wide = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) == 0;
    const int64_t nw = wide ? n / 16 : 0;
    for (int64_t i = t0; i < nw; i += stride)
        reinterpret_cast<uint4 *>(dst)[i] = reinterpret_cast<const uint4 *>(src)[i];
    for (int64_t i = nw * 16 + t0; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_copy_bytes(const void *src, void *dst, int64_t n, hipStream_t s) {
    const int64_t units = (n + 15) / 16;
    const int blocks = int((units + 255) / 256 < 4096 ? (units + 255) / 256 : 4096);
    hipLaunchKernelGGL(copy_bytes_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), n);
    return hipGetLastError();
}

hipError_t launch_generic(const Problem &p) {
    const int waves_per_block = 4;
    const int64_t blocks = (p.out + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL(generic_kernel, dim3(static_cast<unsigned>(blocks)),
                       dim3(waves_per_block * kWave), 0, p.stream, p.codes,
                       static_cast<const uint16_t *>(p.codebooks),
                       static_cast<const uint16_t *>(p.x), static_cast<uint16_t *>(p.y), p.out,
                       p.in, p.K, p.B, p.batch);
    return hipGetLastError();
}

// Dense fp16 W for the prefill path: one thread per group, the K codebook vectors read as
// 16-byte loads, the fp32 left fold rounded once (the value dequantize_kernel writes with
// w_fp16), one 16-byte store.  W is [out][in] row-major.
template <int B>
__global__ void __launch_bounds__(256)
dequant16_kernel(const void *__restrict__ codes, const uint4 *__restrict__ cb,
                 uint4 *__restrict__ W, int64_t ngroups, int K) {
    for (int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < ngroups;
         g += int64_t(gridDim.x) * blockDim.x) {
        float w[8];
        for (int k = 0; k < K; ++k) {
            const uint32_t c = B == 8 ? uint32_t(static_cast<const uint8_t *>(codes)[g * K + k])
                                      : uint32_t(static_cast<const uint16_t *>(codes)[g * K + k]);
            const uint4 v = cb[(int64_t(k) << B) + c];
            const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float f = h2f(uint16_t(h[t >> 1] >> (16 * (t & 1))));
                w[t] = (k == 0) ? f : w[t] + f;
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = uint32_t(f2h_bits(w[2 * i])) | (uint32_t(f2h_bits(w[2 * i + 1])) << 16);
        W[g] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_dequant16(const Problem &p, void *W) {
    const int64_t n = p.out * (p.in / kGroup);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (p.B == 8)
        hipLaunchKernelGGL(dequant16_kernel<8>, dim3(unsigned(blocks)), dim3(256), 0, p.stream, p.codes,
                           static_cast<const uint4 *>(p.codebooks), static_cast<uint4 *>(W), n, p.K);
    else
        hipLaunchKernelGGL(dequant16_kernel<16>, dim3(unsigned(blocks)), dim3(256), 0, p.stream, p.codes,
                           static_cast<const uint4 *>(p.codebooks), static_cast<uint4 *>(W), n, p.K);
    return hipGetLastError();
}

hipError_t launch_dequantize(const Problem &p, void *W, int w_fp16) {
    const int64_t n = p.out * (p.in / kGroup);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(dequantize_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       p.stream, p.codes, static_cast<const uint16_t *>(p.codebooks), W, p.out,
                       p.in, p.K, p.B, w_fp16);
    return hipGetLastError();
}

}  // namespace aqlm
