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
// * Workgroup = 4 waves on 4*MS consecutive rows x (MS*NT) tokens.  Waves own
//   different rows and share the activations: chunks of CHG groups x all tokens
//   are staged in LDS (double-buffered, rows padded by 16 B so the B-fragment
//   reads of one instruction hit different banks).  While the MFMAs of chunk c
//   run, the activations of chunk c+1 are loaded and its A fragments decoded.
// * The input axis is split over KSPLIT workgroups so that every product fills
//   the 256 CUs; partial tiles (fp32) go to a workspace and a second kernel adds
//   the splits in order.  With KSPLIT = 1 the tile is written to y directly.
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

template <int MS, int NT> struct Tile {
    static constexpr int KB = 64 / MS;               // k-blocks (8 inputs) per MFMA
    static constexpr int SS = KB * 4;                // groups per super-step (4 k-steps)
    static constexpr int BN = MS * NT;               // tokens per workgroup
    static constexpr int CHG = MS == 16 ? 32 : 16;   // groups per staged chunk
    static constexpr int SPC = CHG / SS;             // super-steps per chunk
    static constexpr int XROW = CHG * 8 + 8;         // halves per staged token row (+16 B pad)
    static constexpr int XBUF = BN * XROW;           // halves per chunk buffer
    static constexpr int XLOADS = BN * CHG / (kMfmaWaves * kWave);   // 16-B loads per thread
};

template <int K, int BITS, int MS, int NT>
__global__ void __launch_bounds__(kMfmaWaves * kWave)
mfma_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ cb,
            const uint16_t *__restrict__ x, uint16_t *__restrict__ y, float *__restrict__ partial,
            int out, int in, int batch, int groups_per_split) {
    typedef Tile<MS, NT> T;
    typedef typename Acc<MS>::type acc_t;
    typedef typename CodeBlock<K, BITS>::type cblock_t;
    constexpr int CBE = BITS == 8 ? K * 256 : 0;
    constexpr int NACC = Acc<MS>::n;
    constexpr int STEPS = T::SPC * 4;                // MFMA k-steps per chunk
    __shared__ uint4 cbs[CBE > 0 ? CBE : 1];
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][T::XBUF];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = in / kGroup;
    const int row0 = blockIdx.x * (kMfmaWaves * MS) + wave * MS;
    const int tok0 = blockIdx.y * T::BN;
    const int split = blockIdx.z;
    const int g_begin = split * groups_per_split;
    const int g_end = min(G, g_begin + groups_per_split);
    const int nchunks = (g_end - g_begin + T::CHG - 1) / T::CHG;

    const int m = lane % MS;
    const int kb = lane / MS;
    const int o = min(row0 + m, out - 1);            // rows past the end are computed, not stored
    const cblock_t *crow = reinterpret_cast<const cblock_t *>(
        codes + size_t(o) * size_t(G) * (K * BITS / 8));
    const uint4 *cbg = reinterpret_cast<const uint4 *>(cb);

    for (int i = threadIdx.x; i < CBE; i += blockDim.x)
        cbs[i] = reinterpret_cast<const uint4 *>(cb)[i];

    // activations of chunk c: token n, group g_begin + c*CHG + jj -> xs[buf][n*XROW + jj*8]
    auto load_x = [&](int c, uint4 (&r)[T::XLOADS]) {
#pragma unroll
        for (int i = 0; i < T::XLOADS; ++i) {
            const int e = threadIdx.x + i * (kMfmaWaves * kWave);
            const int n = e / T::CHG, jj = e % T::CHG;
            const int j = g_begin + c * T::CHG + jj;
            const int tn = tok0 + n;
            r[i] = make_uint4(0, 0, 0, 0);
            if (tn < batch && j < g_end)
                r[i] = *reinterpret_cast<const uint4 *>(x + size_t(tn) * in + size_t(j) * kGroup);
        }
    };
    auto store_x = [&](int buf, const uint4 (&r)[T::XLOADS]) {
#pragma unroll
        for (int i = 0; i < T::XLOADS; ++i) {
            const int e = threadIdx.x + i * (kMfmaWaves * kWave);
            const int n = e / T::CHG, jj = e % T::CHG;
            *reinterpret_cast<uint4 *>(&xs[buf][n * T::XROW + jj * 8]) = r[i];
        }
    };
    // A fragments of chunk c: super-step q, k-step s -> group g_begin + c*CHG + q*SS + 4*kb + s.
    // gather() only issues the codebook reads (raw vectors); fold() adds the K
    // vectors and masks groups past the split, after the current chunk's MFMAs,
    // so L2 latency of the 16-bit codebook overlaps with them.
    auto gather = [&](int c, uint4 (&v0)[STEPS], uint4 (&v1)[STEPS], bool (&ok)[T::SPC]) {
#pragma unroll
        for (int q = 0; q < T::SPC; ++q) {
            const int jb = g_begin + c * T::CHG + q * T::SS + 4 * kb;
            ok[q] = jb < g_end;                      // g_end - g_begin is a multiple of 4
            const cblock_t cw = __builtin_nontemporal_load(crow + min(jb, G - 4) / 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t c0 = block_code<K, BITS>(cw, s * K);
                v0[q * 4 + s] = BITS == 8 ? cbs[c0] : cbg[c0];
                if constexpr (K == 2) {
                    const uint32_t c1 = block_code<K, BITS>(cw, s * K + 1);
                    v1[q * 4 + s] = BITS == 8 ? cbs[256 + c1] : cbg[(1u << 16) + c1];
                }
            }
        }
    };
    auto fold = [&](const uint4 (&v0)[STEPS], const uint4 (&v1)[STEPS], const bool (&ok)[T::SPC],
                    half8 (&a)[STEPS]) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            half8 f = __builtin_bit_cast(half8, v0[st]);
            if constexpr (K == 2) f = f + __builtin_bit_cast(half8, v1[st]);
            a[st] = ok[st / 4] ? f : half8{};
        }
    };

    acc_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = acc_t{};

    uint4 xr[T::XLOADS];
    half8 acur[STEPS];
    uint4 g0[STEPS], g1[STEPS];                  // g1 only used when K = 2
    bool gok[T::SPC];
    if (nchunks > 0) {
        load_x(0, xr);
        if constexpr (BITS == 16) gather(0, g0, g1, gok);
    }
    if (CBE) __syncthreads();                        // codebooks staged
    if (nchunks > 0) {
        if constexpr (BITS == 8) gather(0, g0, g1, gok);   // LDS codebooks are ready only now
        store_x(0, xr);
        fold(g0, g1, gok, acur);
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        const bool more = c + 1 < nchunks;
        if (more) {
            load_x(c + 1, xr);
            gather(c + 1, g0, g1, gok);
        }
        const uint16_t *xb = xs[buf];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int q = st / 4, s = st % 4;
            const int jj = q * T::SS + 4 * kb + s;   // group inside the chunk (same as A)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const half8 b = *reinterpret_cast<const half8 *>(
                    &xb[(t * MS + m) * T::XROW + jj * 8]);
                acc[t] = mfma<MS>(acur[st], b, acc[t]);
            }
        }
        if (more) {
            store_x(buf ^ 1, xr);
            fold(g0, g1, gok, acur);
        }
        __syncthreads();
    }

    // epilogue: partial tile (KSPLIT > 1) or y
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < NACC; ++r) {
            const int row = row0 + out_row<MS>(lane, r);
            const int n = tok0 + t * MS + (lane % MS);
            if (row < out && n < batch) {
                if (partial)
                    partial[(size_t(split) * batch + n) * out + row] = acc[t][r];
                else
                    y[size_t(n) * out + row] = f2h_bits(acc[t][r]);
            }
        }
    }
}

struct MfmaCfg {
    int ms, nt, ksplit, groups_per_split, grid_x, grid_y;
};

MfmaCfg mfma_cfg(const Problem &p) {
    MfmaCfg c{};
    if (p.batch <= 16) { c.ms = 16; c.nt = 1; }
    else if (p.batch <= 32) { c.ms = 32; c.nt = 1; }
    else if (p.batch <= 64) { c.ms = 32; c.nt = 2; }
    else { c.ms = 32; c.nt = 4; }
    const int64_t G = p.in / kGroup;
    const int chg = c.ms == 16 ? 32 : 16;
    c.grid_x = int((p.out + kMfmaWaves * c.ms - 1) / (kMfmaWaves * c.ms));
    c.grid_y = (p.batch + c.ms * c.nt - 1) / (c.ms * c.nt);
    const int64_t tiles = int64_t(c.grid_x) * c.grid_y;
    const int64_t nchunks = (G + chg - 1) / chg;
    int64_t ks = (512 + tiles - 1) / tiles;          // about two workgroups per CU
    // each split writes and re-reads batch*out fp32: keep that within twice the codes
    const int64_t code_bytes_per_row = p.in / 4;     // 2 bits per weight
    const int64_t cap = (2 * code_bytes_per_row) / (int64_t(p.batch) * 8);
    if (ks > cap) ks = cap;
    if (ks > nchunks) ks = nchunks;
    if (ks < 1) ks = 1;
    // whole chunks per split (multiples of 4 groups keep code blocks whole)
    int64_t gps = (nchunks + ks - 1) / ks * chg;
    c.ksplit = int((G + gps - 1) / gps);
    c.groups_per_split = int(gps);
    return c;
}

template <int K, int BITS, int MS, int NT>
hipError_t launch_t(const Problem &p, const MfmaCfg &c, float *partial) {
    hipLaunchKernelGGL((mfma_kernel<K, BITS, MS, NT>), dim3(c.grid_x, c.grid_y, c.ksplit),
                       dim3(kMfmaWaves * kWave), 0, p.stream,
                       static_cast<const uint8_t *>(p.codes),
                       static_cast<const uint16_t *>(p.codebooks),
                       static_cast<const uint16_t *>(p.x), static_cast<uint16_t *>(p.y), partial,
                       int(p.out), int(p.in), p.batch, c.groups_per_split);
    return hipGetLastError();
}

template <int K, int BITS>
hipError_t launch_kb(const Problem &p, const MfmaCfg &c, float *partial) {
    if (c.ms == 16) return launch_t<K, BITS, 16, 1>(p, c, partial);
    if (c.nt == 1) return launch_t<K, BITS, 32, 1>(p, c, partial);
    if (c.nt == 2) return launch_t<K, BITS, 32, 2>(p, c, partial);
    return launch_t<K, BITS, 32, 4>(p, c, partial);
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

size_t mfma_workspace_bytes(const Problem &p) {
    const MfmaCfg c = mfma_cfg(p);
    return c.ksplit > 1 ? size_t(c.ksplit) * size_t(p.batch) * size_t(p.out) * sizeof(float) : 0;
}

// workspace: KSPLIT x batch x out fp32 partial tiles (unused when KSPLIT = 1)
hipError_t launch_mfma(const Problem &p, void *workspace) {
    const MfmaCfg c = mfma_cfg(p);
    float *partial = c.ksplit > 1 ? static_cast<float *>(workspace) : nullptr;
    hipError_t e;
    if (p.B == 8) e = p.K == 1 ? launch_kb<1, 8>(p, c, partial) : launch_kb<2, 8>(p, c, partial);
    else e = p.K == 1 ? launch_kb<1, 16>(p, c, partial) : launch_kb<2, 16>(p, c, partial);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_partial_sum(partial, p.y, p.batch * p.out, c.ksplit, p.stream);
}

}  // namespace aqlm
