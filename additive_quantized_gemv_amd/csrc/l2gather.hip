// 16-bit-code GEMV (1x16, 2x16) for token generation on gfx950, codebook through L2.
//
// y[b][o] = sum_j sum_k C_k[i_k(o,j)] . x[b][8j .. 8j+7]   (distributed additive
// decode of page "AQLM (Additive Quantization for LLMs)", section "Niveau
// intermediaire").  The 65536 x 16 B codebook (1 MiB per codebook) cannot live
// in LDS, so every group-row gathers one 16-byte entry per codebook from global
// memory; each XCD's 4 MiB L2 keeps a copy of it hot, and the codes, read once,
// are streamed with non-temporal loads so they do not evict it.
//
// What bounds it is the number of gathers in flight, so the kernel is written
// for latency hiding rather than arithmetic:
// * each lane owns 16-byte code chunks (8 codes) of a row; while the gathers of
//   one chunk are outstanding, the codes of the next chunk (same row, or the
//   wave's next row) are already being fetched from HBM;
// * few registers per lane (no multi-row unrolling) so that many waves fit on
//   a SIMD; activations are staged once per workgroup in LDS when they fit.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kL2Waves = 4;

template <int K, int NB, bool XLDS, int NS>
__global__ void __launch_bounds__(kL2Waves * kWave)
l2_kernel(const uint16_t *__restrict__ x, int in, int batch, const Segs segs) {
    constexpr int GPC = 8 / K;                 // groups per 16-byte chunk
    extern __shared__ uint4 xs[];              // [batch][G] when XLDS
    const int G = in / kGroup;
    const int NC = G / GPC;                    // chunks per row
    const int CPL = (NC + kWave - 1) / kWave;  // chunk iterations per row
    if (XLDS) {
        for (int i = threadIdx.x; i < batch * G; i += blockDim.x)
            xs[i] = reinterpret_cast<const uint4 *>(x)[i];
        __syncthreads();
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int nwaves = gridDim.x * kL2Waves;
    const int out = seg_total<NS>(segs.n, segs.row0);         // rows over all matrices
    int o = blockIdx.x * kL2Waves + threadIdx.x / kWave;
    if (o >= out) return;

    // Branch-free (the chunk index is clamped into the row; clamped lanes are masked
    // where the chunk is used): a conditional load would be waited for at once.
    // Global row -> its matrix's codes (wave-uniform).
    auto load_chunk = [&](int row, int it) -> u32x4 {
        const int mi = seg_of<NS>(segs.n, segs.row0, row);
        const uint8_t *codes = static_cast<const uint8_t *>(pick(segs.codes, mi));
        const int c = min(lane + kWave * it, NC - 1);
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            codes + (size_t(row - pick(segs.row0, mi)) * NC + c) * 16u));
    };

    int it = 0;
    u32x4 cur = load_chunk(o, 0);
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;

    while (true) {
        int o_n = o, it_n = it + 1;
        if (it_n == CPL) {
            it_n = 0;
            o_n = o + nwaves;
        }
        const u32x4 nxt = load_chunk(min(o_n, out - 1), it_n);

        const int c = lane + kWave * it;
        const int mi = seg_of<NS>(segs.n, segs.row0, o);
        const uint4 *__restrict__ cb = static_cast<const uint4 *>(pick(segs.cb, mi));
        if (c < NC) {
            uint4 v[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const uint32_t w = cur[n >> 1];
                const uint32_t code = (w >> ((n & 1) * 16)) & 0xFFFFu;
                v[n] = cb[(size_t(n % K) << 16) + code];
            }
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                const int j = c * GPC + g;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < batch) {
                        const uint4 xv = XLDS ? xs[b * G + j]
                                              : *reinterpret_cast<const uint4 *>(
                                                    x + size_t(b) * in + size_t(j) * kGroup);
#pragma unroll
                        for (int k = 0; k < K; ++k) acc[b] = dot8(v[g * K + k], xv, acc[b]);
                    }
                }
            }
        }
        if (it == CPL - 1) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float s = wave_sum(acc[b]);
                if (lane == 0 && b < batch) {
                    const int out_m = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
                    static_cast<uint16_t *>(pick(segs.y, mi))[size_t(b) * out_m + (o - pick(segs.row0, mi))] =
                        f2h_bits(s);
                }
                acc[b] = 0.0f;
            }
        }
        if (o_n >= out) break;
        o = o_n;
        it = it_n;
        cur = nxt;
    }
}

template <int K, int NB>
hipError_t launch_nb(const Problem &p) {
    const size_t xbytes = size_t(p.batch) * size_t(p.in) * 2;
    const bool xlds = xbytes <= 64 * 1024;
    // up to 8 workgroups (32 waves) per CU, fewer when the activations take LDS
    int per_cu = 8;
    if (xlds) {
        const int by_lds = int((160 * 1024) / (xbytes ? xbytes : 1));
        per_cu = by_lds < per_cu ? (by_lds < 1 ? 1 : by_lds) : per_cu;
    }
    const int64_t need = (p.out + kL2Waves - 1) / kL2Waves;
    const int grid = int(need < int64_t(256) * per_cu ? need : int64_t(256) * per_cu);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    const dim3 g(grid), b(kL2Waves * kWave);
    const bool one = p.segs.n == 1;
    if (xlds && one)
        hipLaunchKernelGGL((l2_kernel<K, NB, true, 1>), g, b, xbytes, p.stream, x, int(p.in),
                           p.batch, p.segs);
    else if (xlds)
        hipLaunchKernelGGL((l2_kernel<K, NB, true, kMaxSegs>), g, b, xbytes, p.stream, x,
                           int(p.in), p.batch, p.segs);
    else if (one)
        hipLaunchKernelGGL((l2_kernel<K, NB, false, 1>), g, b, 0, p.stream, x, int(p.in),
                           p.batch, p.segs);
    else
        hipLaunchKernelGGL((l2_kernel<K, NB, false, kMaxSegs>), g, b, 0, p.stream, x,
                           int(p.in), p.batch, p.segs);
    return hipGetLastError();
}

template <int K>
hipError_t launch_k(const Problem &p) {
    if (p.batch <= 1) return launch_nb<K, 1>(p);
    if (p.batch <= 2) return launch_nb<K, 2>(p);
    if (p.batch <= 4) return launch_nb<K, 4>(p);
    return launch_nb<K, 8>(p);
}

}  // namespace

bool l2_supported(const Problem &p) {
    if (p.B != 16 || (p.K != 1 && p.K != 2)) return false;
    if (p.batch < 1 || p.batch > 8) return false;
    const int64_t G = p.in / kGroup;
    if (G % (8 / p.K)) return false;
    if (p.out > (1 << 30) || p.in > (1 << 30) || int64_t(p.batch) * G > INT32_MAX) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks) |
                        reinterpret_cast<uintptr_t>(p.x);
    return (a & 15u) == 0;
}

hipError_t launch_l2(const Problem &p) { return p.K == 1 ? launch_k<1>(p) : launch_k<2>(p); }

}  // namespace aqlm
