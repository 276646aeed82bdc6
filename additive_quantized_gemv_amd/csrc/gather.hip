// Gather GEMV kernel for 8-bit codes, token generation (batch 1..8), gfx950.
//
// y[b][o] = sum_j sum_k C_k[i_k(o,j)] . x[b][8j .. 8j+7]   (distributing the dot
// product over the additive decode of page "AQLM (Additive Quantization for
// LLMs)", section "Niveau intermediaire"; W is never materialised).
//
// All K codebooks (K x 256 x 16 B, 8 KiB for 2x8) are staged in LDS once per
// workgroup; every group-row gathers K 16-byte entries from LDS.
//
// Mapping: a wave owns RPW consecutive rows at a time; lane l reads 16-byte
// chunks l, l+64, ... of each of those rows (one chunk = 16/(K*B/8) groups),
// so each wave load is a contiguous 1 KiB of one row.  The activations are
// staged in LDS when they fit, otherwise read through the caches.  Products are
// v_dot2_f32_f16 (fp16 x fp16 -> fp32), lane partials are reduced with DPP.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kRPW = 4;            // rows per wave per iteration
constexpr int kWavesPerBlock = 4;  // 256 threads
constexpr int kRowsPerTile = kRPW * kWavesPerBlock;
constexpr int kMaxLdsBytes = 160 * 1024;

template <int K, int CB>
__device__ __forceinline__ uint32_t chunk_code(const uint4 &cw, int n) {
    // n-th code of a 16-byte chunk (n is a compile-time constant after unrolling)
    const uint32_t w = (CB == 1) ? ((n >> 2) == 0 ? cw.x : (n >> 2) == 1 ? cw.y
                                    : (n >> 2) == 2 ? cw.z : cw.w)
                                 : ((n >> 1) == 0 ? cw.x : (n >> 1) == 1 ? cw.y
                                    : (n >> 1) == 2 ? cw.z : cw.w);
    return (CB == 1) ? ((w >> ((n & 3) * 8)) & 0xFFu) : ((w >> ((n & 1) * 16)) & 0xFFFFu);
}

template <int K, int BITS, int NB, bool XLDS>
__global__ void __launch_bounds__(kWavesPerBlock * kWave)
gather_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ cb,
              const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int out, int in,
              int batch, int row_tiles) {
    constexpr int CB = BITS / 8;          // bytes per code
    constexpr int GPC = 16 / (K * CB);    // groups per 16-byte chunk
    constexpr int CBE = BITS == 8 ? K * 256 : 0;  // codebook entries held in LDS
    extern __shared__ uint4 smem[];
    const int G = in / kGroup;
    const int NC = G / GPC;               // chunks per row
    uint4 *cbs = smem;
    uint4 *xs = smem + CBE;

    for (int i = threadIdx.x; i < CBE; i += blockDim.x)
        cbs[i] = reinterpret_cast<const uint4 *>(cb)[i];
    if (XLDS) {
        for (int i = threadIdx.x; i < batch * G; i += blockDim.x)
            xs[i] = reinterpret_cast<const uint4 *>(x)[i];
    }
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint4 *cbg = reinterpret_cast<const uint4 *>(cb);

    for (int tile = blockIdx.x; tile < row_tiles; tile += gridDim.x) {
        const int o0 = tile * kRowsPerTile + wave * kRPW;
        if (o0 >= out) continue;
        float acc[kRPW][NB];
#pragma unroll
        for (int r = 0; r < kRPW; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;
        const uint8_t *rowp[kRPW];
#pragma unroll
        for (int r = 0; r < kRPW; ++r)
            rowp[r] = codes + size_t(min(o0 + r, out - 1)) * size_t(NC) * 16u;

        for (int c = lane; c < NC; c += kWave) {
            uint4 cw[kRPW];
#pragma unroll
            for (int r = 0; r < kRPW; ++r) cw[r] = load_stream16(rowp[r] + size_t(c) * 16u);
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                const int j = c * GPC + g;
                uint4 xv[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < batch) {
                        xv[b] = XLDS ? xs[b * G + j]
                                     : *reinterpret_cast<const uint4 *>(x + size_t(b) * in +
                                                                        size_t(j) * kGroup);
                    } else {
                        xv[b] = make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < kRPW; ++r) {
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const uint32_t code = chunk_code<K, CB>(cw[r], g * K + k);
                        const uint4 v = (BITS == 8) ? cbs[k * 256 + code]
                                                    : cbg[(size_t(k) << 16) + code];
#pragma unroll
                        for (int b = 0; b < NB; ++b) acc[r][b] = dot8(v, xv[b], acc[r][b]);
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kRPW; ++r) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float s = wave_sum(acc[r][b]);
                if (lane == 0 && b < batch && o0 + r < out)
                    y[size_t(b) * out + o0 + r] = f2h_bits(s);
            }
        }
    }
}

struct GatherCfg {
    int groups_per_chunk;
    size_t cb_lds;
    size_t x_lds;
};

GatherCfg gather_cfg(const Problem &p) {
    GatherCfg c{};
    const int cbytes = p.K * (p.B / 8);
    c.groups_per_chunk = cbytes <= 16 ? 16 / cbytes : 0;
    c.cb_lds = p.B == 8 ? size_t(p.K) * 256 * 16 : 0;
    c.x_lds = size_t(p.batch) * size_t(p.in) * 2;
    return c;
}

template <int K, int BITS, int NB>
hipError_t launch_nb(const Problem &p) {
    const GatherCfg c = gather_cfg(p);
    const bool xlds = c.cb_lds + c.x_lds <= 64 * 1024;
    const size_t lds = c.cb_lds + (xlds ? c.x_lds : 0);
    const int row_tiles = int((p.out + kRowsPerTile - 1) / kRowsPerTile);
    // enough workgroups to cover the rows, at most ~4 resident per CU
    int blocks_per_cu = int(kMaxLdsBytes / (lds ? lds : 1));
    blocks_per_cu = blocks_per_cu < 1 ? 1 : (blocks_per_cu > 4 ? 4 : blocks_per_cu);
    int grid = 256 * blocks_per_cu;
    if (grid > row_tiles) grid = row_tiles;
    const uint8_t *codes = static_cast<const uint8_t *>(p.codes);
    const uint16_t *cb = static_cast<const uint16_t *>(p.codebooks);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    uint16_t *y = static_cast<uint16_t *>(p.y);
    if (xlds)
        hipLaunchKernelGGL((gather_kernel<K, BITS, NB, true>), dim3(grid),
                           dim3(kWavesPerBlock * kWave), lds, p.stream, codes, cb, x, y,
                           int(p.out), int(p.in), p.batch, row_tiles);
    else
        hipLaunchKernelGGL((gather_kernel<K, BITS, NB, false>), dim3(grid),
                           dim3(kWavesPerBlock * kWave), lds, p.stream, codes, cb, x, y,
                           int(p.out), int(p.in), p.batch, row_tiles);
    return hipGetLastError();
}

template <int K, int BITS>
hipError_t launch_kb(const Problem &p) {
    if (p.batch <= 1) return launch_nb<K, BITS, 1>(p);
    if (p.batch <= 2) return launch_nb<K, BITS, 2>(p);
    if (p.batch <= 4) return launch_nb<K, BITS, 4>(p);
    return launch_nb<K, BITS, 8>(p);
}

}  // namespace

bool gather_supported(const Problem &p) {
    if (p.batch < 1 || p.batch > 8) return false;
    if (p.B != 8 || !(p.K == 1 || p.K == 2 || p.K == 4 || p.K == 8)) return false;
    const GatherCfg c = gather_cfg(p);
    const int64_t G = p.in / kGroup;
    if (c.groups_per_chunk == 0 || G % c.groups_per_chunk) return false;
    if (p.out > INT32_MAX / 2 || p.in > INT32_MAX / 2) return false;
    if (int64_t(p.batch) * G > INT32_MAX) return false;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(p.codes) |
                          reinterpret_cast<uintptr_t>(p.codebooks) |
                          reinterpret_cast<uintptr_t>(p.x);
    if (mis & 15u) return false;
    if (c.cb_lds > 64 * 1024) return false;
    return true;
}

hipError_t launch_gather(const Problem &p) {
    switch (p.K) {
        case 1: return launch_kb<1, 8>(p);
        case 2: return launch_kb<2, 8>(p);
        case 4: return launch_kb<4, 8>(p);
        default: return launch_kb<8, 8>(p);
    }
}

}  // namespace aqlm
