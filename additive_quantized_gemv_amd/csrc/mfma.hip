// Batched additive-quantized GEMM on the gfx950 matrix cores.
//
// At batch >= 16 the product is a real dense contraction, so W is decoded to
// fp16 and fed to v_mfma_f32_{16x16x32,32x32x16}_f16 (fp32 accumulation).
// Decode rule: page "AQLM (Additive Quantization for LLMs)", section "Niveau
// intermediaire".  Each lane's A fragment is exactly one 8-wide group of one
// row (8 consecutive k), so a lane decodes one group straight into its MFMA
// operand registers: no dense W tile is written anywhere.
//
// * K = 1: the fragment is the codebook vector itself.  K = 2: v_pk_add_f16 of
//   the two vectors, i.e. the exact sum rounded once to fp16, which equals the
//   fp16 rounding of the fp32 fold because fp32 carries more than 2*11+2 bits
//   (double rounding through fp32 is innocuous for one fp16 addition).
// * B = 8 codebooks are staged in LDS; the B = 16 codebook is read through L2.
// * A workgroup is 4 waves on one tile of MS rows x (MS*NT) tokens; the waves
//   split the input axis four ways and their accumulators are summed in LDS,
//   so a 4096-row layer still yields 256+ workgroups.
// * MFMA operand layout used: A lane l = row (l % MS), k-block (l / MS);
//   B lane l = token (l % MS), same k-block.  Both operands place the same 8
//   inputs in a lane, so the product does not depend on how the hardware orders
//   k inside a block.  Result (16x16): lane l, reg r -> row 4(l/16)+r, token l%16;
//   (32x32): reg r -> row 8(r/4)+4(l/32)+(r%4), token l%32.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kMfmaWaves = 4;

template <int MS> struct Acc;
template <> struct Acc<16> { typedef float4v type; static constexpr int n = 4; };
template <> struct Acc<32> { typedef float16v type; static constexpr int n = 16; };

template <int MS>
__device__ __forceinline__ typename Acc<MS>::type mfma(half8 a, half8 b, typename Acc<MS>::type c) {
    if constexpr (MS == 16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <int MS>
__device__ __forceinline__ int out_row(int lane, int r) {
    if constexpr (MS == 16) return 4 * (lane >> 4) + r;
    else return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// codes of 4 consecutive groups of one row (K*B/8 bytes each)
template <int K, int BITS> struct CodeBlock;
template <> struct CodeBlock<1, 8> { typedef uint32_t type; };
template <> struct CodeBlock<2, 8> { typedef u32x2 type; };
template <> struct CodeBlock<1, 16> { typedef u32x2 type; };
template <> struct CodeBlock<2, 16> { typedef u32x4 type; };

template <int K, int BITS>
__device__ __forceinline__ uint32_t block_code(const typename CodeBlock<K, BITS>::type &cw, int n) {
    // n-th code inside the block (compile-time n after unrolling)
    if constexpr (K * BITS == 8) {
        return (cw >> (8 * n)) & 0xFFu;
    } else if constexpr (K * BITS == 16) {
        const uint32_t w = (n >> (BITS == 8 ? 2 : 1)) ? cw.y : cw.x;
        return BITS == 8 ? (w >> (8 * (n & 3))) & 0xFFu : (w >> (16 * (n & 1))) & 0xFFFFu;
    } else {
        const int wi = n >> 1;
        const uint32_t w = wi == 0 ? cw.x : wi == 1 ? cw.y : wi == 2 ? cw.z : cw.w;
        return (w >> (16 * (n & 1))) & 0xFFFFu;
    }
}

template <int K, int BITS, int MS, int NT>
__global__ void __launch_bounds__(kMfmaWaves * kWave)
mfma_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ cb,
            const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int out, int in, int batch) {
    typedef typename Acc<MS>::type acc_t;
    typedef typename CodeBlock<K, BITS>::type cblock_t;
    constexpr int KB = 64 / MS;            // k-blocks (of 8 inputs) per MFMA
    constexpr int SS = KB * 4;             // groups per super-step (4 MFMA k-steps)
    constexpr int CBE = BITS == 8 ? K * 256 : 0;
    constexpr int NACC = Acc<MS>::n;
    __shared__ uint4 cbs[CBE > 0 ? CBE : 1];
    __shared__ float red[(kMfmaWaves - 1) * NT * NACC * kWave];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < CBE; i += blockDim.x)
        cbs[i] = reinterpret_cast<const uint4 *>(cb)[i];
    if (CBE) __syncthreads();

    const int G = in / kGroup;
    const int row0 = blockIdx.x * MS;
    const int tok0 = blockIdx.y * (MS * NT);
    const int m = lane % MS;
    const int kb = lane / MS;
    const int o = row0 + m;
    const bool row_ok = o < out;
    const cblock_t *crow = reinterpret_cast<const cblock_t *>(codes + size_t(row_ok ? o : 0) *
                                                              size_t(G) * (K * BITS / 8));
    const uint4 *cbg = reinterpret_cast<const uint4 *>(cb);

    acc_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = acc_t{};

    const int nsuper = (G + SS - 1) / SS;
    for (int q = wave; q < nsuper; q += kMfmaWaves) {
        const int jb = q * SS + 4 * kb;    // first of this lane's 4 groups
        const bool blk_ok = row_ok && jb < G;
        cblock_t cw{};
        if (blk_ok) cw = __builtin_nontemporal_load(crow + jb / 4);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int j = jb + s;
            half8 a = {};
            if (blk_ok) {
                uint4 v0;
                const uint32_t c0 = block_code<K, BITS>(cw, s * K);
                v0 = BITS == 8 ? cbs[c0] : cbg[c0];
                if constexpr (K == 1) {
                    a = __builtin_bit_cast(half8, v0);
                } else {
                    const uint32_t c1 = block_code<K, BITS>(cw, s * K + 1);
                    const uint4 v1 = BITS == 8 ? cbs[256 + c1] : cbg[(1u << 16) + c1];
                    a = __builtin_bit_cast(half8, v0) + __builtin_bit_cast(half8, v1);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int n = tok0 + t * MS + m;
                half8 b = {};
                if (n < batch && jb < G)
                    b = *reinterpret_cast<const half8 *>(x + size_t(n) * in + size_t(j) * kGroup);
                acc[t] = mfma<MS>(a, b, acc[t]);
            }
        }
    }

    // sum the four waves' partial tiles
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < NACC; ++r)
                red[(((wave - 1) * NT + t) * NACC + r) * kWave + lane] = acc[t][r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < NACC; ++r) {
            float s = acc[t][r];
#pragma unroll
            for (int w = 1; w < kMfmaWaves; ++w) s += red[(((w - 1) * NT + t) * NACC + r) * kWave + lane];
            const int row = row0 + out_row<MS>(lane, r);
            const int n = tok0 + t * MS + (lane % MS);
            if (row < out && n < batch) y[size_t(n) * out + row] = f2h_bits(s);
        }
    }
}

template <int K, int BITS, int MS, int NT>
hipError_t launch_t(const Problem &p) {
    const int grid_x = int((p.out + MS - 1) / MS);
    const int grid_y = (p.batch + MS * NT - 1) / (MS * NT);
    hipLaunchKernelGGL((mfma_kernel<K, BITS, MS, NT>), dim3(grid_x, grid_y),
                       dim3(kMfmaWaves * kWave), 0, p.stream,
                       static_cast<const uint8_t *>(p.codes),
                       static_cast<const uint16_t *>(p.codebooks),
                       static_cast<const uint16_t *>(p.x), static_cast<uint16_t *>(p.y),
                       int(p.out), int(p.in), p.batch);
    return hipGetLastError();
}

template <int K, int BITS>
hipError_t launch_kb(const Problem &p) {
    if (p.batch <= 16) return launch_t<K, BITS, 16, 1>(p);
    if (p.batch <= 32) return launch_t<K, BITS, 32, 1>(p);
    if (p.batch <= 64) return launch_t<K, BITS, 32, 2>(p);
    return launch_t<K, BITS, 32, 4>(p);
}

}  // namespace

bool mfma_supported(const Problem &p) {
    if (!((p.K == 1 || p.K == 2) && (p.B == 8 || p.B == 16))) return false;
    if (p.batch < 1) return false;
    const int64_t G = p.in / kGroup;
    if (G % 4) return false;
    if (p.out > (1 << 30) || p.in > (1 << 30) || int64_t(p.batch) * p.in > (int64_t(1) << 40))
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks) |
                        reinterpret_cast<uintptr_t>(p.x);
    return (a & 15u) == 0;
}

hipError_t launch_mfma(const Problem &p) {
    if (p.B == 8) return p.K == 1 ? launch_kb<1, 8>(p) : launch_kb<2, 8>(p);
    return p.K == 1 ? launch_kb<1, 16>(p) : launch_kb<2, 16>(p);
}

}  // namespace aqlm
