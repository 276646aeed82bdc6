// Batched additive-quantized GEMM on the gfx950 matrix cores.
//
// With several tokens the product is a dense contraction, so W is decoded to fp16
// and fed to v_mfma_f32_{16x16x32,32x32x16}_f16 (fp32 accumulation).  Even at 2
// tokens (a 16-token tile mostly padding) this beats the gather kernels on MI355X:
// a group is decoded once for all tokens and the matrix cores are otherwise idle.
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
// * Workgroup = 8 waves on 4*MS consecutive rows x (MS*NT) tokens.  Wave pairs own
//   different rows (each wave of a pair one half of every chunk's input groups,
//   their tiles added in LDS at the end: two waves per SIMD) and share the
//   activations: chunks of CHG groups x all tokens
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
//
// Batch <= 32 uses a second kernel (mfma_kw_kernel): there a 16-row tile is too
// little work to fill the chip with row tiles alone, so the 16 waves of a
// workgroup take the same 16 rows and different 32-group units of the input
// axis.  Each lane's A fragments are 8 consecutive groups of its row (one code
// load), its B fragments the matching activations straight from global memory
// (L2-resident), and the 16 partial tiles are added in LDS, in wave order, at
// the end: no partial sums leave the workgroup.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kMfmaWaves = 4;                  // row groups of a tiled workgroup
constexpr int kTiledThreads = 2 * kMfmaWaves * kWave;   // two waves per row group

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
template <> struct CodeBlock<4, 8> { typedef u32x4 type; };
template <> struct CodeBlock<8, 8> { typedef u32x8 type; };

// Decode of one group from K > 2 codebook vectors: the fp32 left fold in codebook order,
// rounded once to fp16 (the fp16 value aqlm_dequantize writes).  K <= 2 adds in fp16
// directly, which rounds the exact sum once and is the same value.
template <int K>
__device__ __forceinline__ half8 fold_fp32(const uint4 (&v)[K]) {
    float f[8];
    const half8 h0 = __builtin_bit_cast(half8, v[0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = float(h0[e]);
#pragma unroll
    for (int k = 1; k < K; ++k) {
        const half8 h = __builtin_bit_cast(half8, v[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] += float(h[e]);
    }
    half8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = _Float16(f[e]);
    return r;
}

template <int K, int BITS>
__device__ __forceinline__ uint32_t block_code(const typename CodeBlock<K, BITS>::type &cw, int n) {
    // n-th code inside the block (compile-time n after unrolling)
    if constexpr (K * BITS == 8) {
        return (cw >> (8 * n)) & 0xFFu;
    } else if constexpr (K * BITS == 16) {
        const uint32_t w = (n >> (BITS == 8 ? 2 : 1)) ? cw.y : cw.x;
        return BITS == 8 ? (w >> (8 * (n & 3))) & 0xFFu : (w >> (16 * (n & 1))) & 0xFFFFu;
    } else if constexpr (BITS == 8) {
        return (cw[n >> 2] >> (8 * (n & 3))) & 0xFFu;
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
    static constexpr int XLOADS = BN * CHG / kTiledThreads;   // 16-B loads per thread
    static_assert(SPC == 2, "one super-step per wave of a row group");
    static_assert(BN * CHG % kTiledThreads == 0, "whole activation loads per thread");
};

template <int K, int BITS, int MS, int NT, int NS>
__global__ void __launch_bounds__(kTiledThreads)
mfma_kernel(const uint16_t *__restrict__ x, float *__restrict__ partial, int in,
            int batch, int groups_per_split, const Segs segs) {
    typedef Tile<MS, NT> T;
    typedef typename Acc<MS>::type acc_t;
    typedef typename CodeBlock<K, BITS>::type cblock_t;
    constexpr int CBE = BITS == 8 ? K * 256 : 0;
    constexpr int NACC = Acc<MS>::n;
    constexpr int STEPS = 4;                         // MFMA k-steps per chunk and wave
    __shared__ uint4 cbs[CBE > 0 ? CBE : 1];
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][T::XBUF];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // Waves w and w+4 own row group w & 3 (MS rows) and take super-steps 0 and 1 of
    // every chunk (h = w >> 2): two waves per SIMD, whose partial tiles are added in
    // LDS at the end.
    const int rg = wave & (kMfmaWaves - 1), h = wave >> 2;
    const int G = in / kGroup;
    // row tiles of each matrix are numbered consecutively (segs.aux0)
    const int mi = seg_of<NS>(segs.n, segs.aux0, blockIdx.x);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const int rows_all = seg_total<NS>(segs.n, segs.row0);
    const uint8_t *__restrict__ codes = static_cast<const uint8_t *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ cb = static_cast<const uint16_t *>(pick(segs.cb, mi));
    uint16_t *__restrict__ y = static_cast<uint16_t *>(pick(segs.y, mi));
    const int row0 = (blockIdx.x - pick(segs.aux0, mi)) * (kMfmaWaves * MS) + rg * MS;
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

    // Software pipeline over chunks of CHG groups.  While the MFMAs of chunk c run,
    // chunk c+1's A fragments are gathered (its codes arrived during chunk c-1) and its
    // activations staged in LDS (loaded during chunk c-1); chunk c+2's codes and
    // activations are loaded.  Every global load thus has a whole chunk of MFMAs to
    // arrive.  Loads past the split are clamped into the matrix (always in bounds) and
    // masked where used, so none is conditional.
    //
    // activations of chunk c: token n, group g_begin + c*CHG + jj -> xs[buf][n*XROW + jj*8]
    auto load_x = [&](int c, uint4 (&r)[T::XLOADS]) {
#pragma unroll
        for (int i = 0; i < T::XLOADS; ++i) {
            const int e = threadIdx.x + i * kTiledThreads;
            const int n = e / T::CHG, jj = e % T::CHG;
            const int j = min(g_begin + c * T::CHG + jj, g_end - 1);
            const int tn = min(tok0 + n, batch - 1);
            r[i] = *reinterpret_cast<const uint4 *>(x + size_t(tn) * in + size_t(j) * kGroup);
        }
    };
    // Groups past the split are zeroed (their A fragments are zero too; zeroing B as
    // well keeps an inf or NaN of a clamped duplicate out of the sum).  Tokens past the
    // batch are clamped duplicates whose outputs are never stored.  The mask is an AND
    // with an opaque value: a select on the loaded vector would be turned into a branch
    // that sinks the load to this point.
    auto store_x = [&](int buf, int c, const uint4 (&r)[T::XLOADS]) {
#pragma unroll
        for (int i = 0; i < T::XLOADS; ++i) {
            const int e = threadIdx.x + i * kTiledThreads;
            const int n = e / T::CHG, jj = e % T::CHG;
            uint32_t msk = g_begin + c * T::CHG + jj < g_end ? 0xFFFFFFFFu : 0u;
            asm volatile("" : "+v"(msk));
            *reinterpret_cast<uint4 *>(&xs[buf][n * T::XROW + jj * 8]) =
                make_uint4(r[i].x & msk, r[i].y & msk, r[i].z & msk, r[i].w & msk);
        }
    };
    // codes of chunk c, this wave's super-step h: groups g_begin + c*CHG + h*SS + 4*kb + (0..3)
    auto load_codes = [&](int c, cblock_t &cw) {
        const int jb = g_begin + c * T::CHG + h * T::SS + 4 * kb;
        cw = __builtin_nontemporal_load(crow + min(jb, G - 4) / 4);
    };
    // A fragments: gather() only issues the codebook reads (raw vectors); fold() adds
    // the K vectors and masks groups past the split after the current chunk's MFMAs,
    // so the read latency (LDS, or L2 for the 16-bit codebook) overlaps with them.
    auto gather = [&](const cblock_t &cw, uint4 (&v0)[STEPS], uint4 (&v1)[STEPS]) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            if constexpr (K > 2) {
                // (8-bit codes only) folded here in fp32; v0 holds the fp16 result
                uint4 v[K];
#pragma unroll
                for (int k = 0; k < K; ++k) v[k] = cbs[k * 256 + block_code<K, BITS>(cw, s * K + k)];
                v0[s] = __builtin_bit_cast(uint4, fold_fp32<K>(v));
                continue;
            }
            const uint32_t c0 = block_code<K, BITS>(cw, s * K);
            v0[s] = BITS == 8 ? cbs[c0] : cbg[c0];
            if constexpr (K == 2) {
                const uint32_t c1 = block_code<K, BITS>(cw, s * K + 1);
                v1[s] = BITS == 8 ? cbs[256 + c1] : cbg[(1u << 16) + c1];
            }
        }
    };
    auto fold = [&](int c, const uint4 (&v0)[STEPS], const uint4 (&v1)[STEPS], half8 (&a)[STEPS]) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            // g_end - g_begin is a multiple of 4: a 4-group block is all in or all out
            const bool ok = g_begin + c * T::CHG + h * T::SS + 4 * kb < g_end;
            half8 f = __builtin_bit_cast(half8, v0[st]);
            if constexpr (K == 2) f = f + __builtin_bit_cast(half8, v1[st]);
            a[st] = ok ? f : half8{};
        }
    };

    acc_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = acc_t{};

    // Register slots: at chunk c (parity S = c & 1), cw[S] holds chunk c+1's codes
    // and xr[S] its activations (both loaded two chunks earlier); slot S^1 holds chunk
    // c+2's, still in flight.  After use, slot S is refilled with chunk c+3's.  The
    // chunk loop is unrolled by two so that every slot index is a constant.
    uint4 xr[2][T::XLOADS];
    cblock_t cw[2];
    half8 acur[STEPS];
    uint4 g0[STEPS], g1[STEPS];                  // g1 only used when K = 2
    (void)g1;
    {
        // prologue: chunk 0 decoded and staged; chunks 1 and 2 in flight.
        // (Every split has at least one chunk.)  The codebook loads go first and
        // every chunk load is issued before their LDS stores wait for them.
        constexpr int CBPT = (CBE + kTiledThreads - 1) / kTiledThreads;
        uint4 cbv[CBPT > 0 ? CBPT : 1];
#pragma unroll
        for (int i = 0; i < CBPT; ++i)
            cbv[i] = cbg[min(int(threadIdx.x) + i * kTiledThreads, CBE - 1)];
        cblock_t cw0;
        uint4 x0[T::XLOADS];
        load_codes(0, cw0);
        load_x(0, x0);
        load_codes(1, cw[0]);
        load_x(1, xr[0]);
        load_codes(2, cw[1]);
        load_x(2, xr[1]);
        if constexpr (BITS == 16) gather(cw0, g0, g1);
        // unconditional stores (clamped threads rewrite the last vector with its own
        // value), so that the codebook loads are not sunk behind the others
#pragma unroll
        for (int i = 0; i < CBPT; ++i)
            cbs[min(int(threadIdx.x) + i * kTiledThreads, CBE - 1)] = cbv[i];
        if (CBE) __syncthreads();                    // codebooks staged
        if constexpr (BITS == 8) gather(cw0, g0, g1);
        store_x(0, 0, x0);
        fold(0, g0, g1, acur);
        __syncthreads();
    }

    // Nothing in a chunk is conditional: past the last chunk the loads are clamped
    // duplicates and the staged values go unused (a conditional load would make the
    // compiler wait for every load in flight where the paths join).
    auto chunk = [&](int c, auto slot) {
        constexpr int S = decltype(slot)::value;
        gather(cw[S], g0, g1);                   // chunk c+1's codebook vectors
        // B fragments of k-step st: token t*MS + m, group h*SS + 4*kb + st of the chunk
        // (the same group as the A fragment).  Those of step st+1 are read while the
        // MFMAs of step st run, so no MFMA waits for an LDS read of its own.
        const uint16_t *xb = xs[S];
        auto load_b = [&](int st, half8 (&b)[NT]) {
            const int jj = h * T::SS + 4 * kb + st;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                b[t] = *reinterpret_cast<const half8 *>(&xb[(t * MS + m) * T::XROW + jj * 8]);
        };
        half8 bq[2][NT];
        load_b(0, bq[0]);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (st + 1 < STEPS) load_b(st + 1, bq[(st + 1) & 1]);
            // pinned order: left to itself the scheduler sinks each read to its MFMA
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = mfma<MS>(acur[st], bq[st & 1][t], acc[t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_x(S ^ 1, c + 1, xr[S]);
        fold(c + 1, g0, g1, acur);
        load_x(c + 3, xr[S]);
        load_codes(c + 3, cw[S]);
        __syncthreads();
    };
    // Chunks go in pairs.  With an odd count the last one is past the split: its A and
    // B fragments are all zero and it adds nothing (mfma_cfg makes the counts even where
    // it can).  The first pair is unconditional (do-while), so that the prologue's loads
    // stay above the barriers.
    int c = 0;
    do {
        chunk(c, std::integral_constant<int, 0>{});
        chunk(c + 1, std::integral_constant<int, 1>{});
        c += 2;
    } while (c < nchunks);

    // Epilogue: the workgroup's tile goes through LDS (the activation buffers are free
    // now) as [token][row], so that the stores to global memory are row-contiguous:
    // one 4-byte (partial) or 2-byte (y) store per lane, consecutive lanes on
    // consecutive rows.  The super-step-1 waves write their tiles, then the
    // super-step-0 waves add theirs (sum = h0 + h1, in that order).
    constexpr int ROWS = kMfmaWaves * MS;            // rows per workgroup
    constexpr int TROW = ROWS + 4;                   // floats per token row (+16 B pad)
    static_assert(sizeof(float) * T::BN * TROW <= sizeof(xs), "output tile fits the LDS buffers");
    float *tile = reinterpret_cast<float *>(&xs[0][0]);
    auto tile_pass = [&](bool add) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r4 = 0; r4 < NACC / 4; ++r4) {
                // registers 4*r4 .. 4*r4+3 hold 4 consecutive rows of one token
                const int rl = rg * MS + out_row<MS>(lane, 4 * r4);
                const int tl = t * MS + (lane % MS);
                float4 *q = reinterpret_cast<float4 *>(&tile[tl * TROW + rl]);
                float4 v = make_float4(acc[t][4 * r4], acc[t][4 * r4 + 1], acc[t][4 * r4 + 2],
                                       acc[t][4 * r4 + 3]);
                if (add) {
                    const float4 u = *q;
                    v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
                }
                *q = v;
            }
        }
    };
    if (h == 1) tile_pass(false);
    __syncthreads();
    if (h == 0) tile_pass(true);
    __syncthreads();
    const int wg_row0 = (blockIdx.x - pick(segs.aux0, mi)) * ROWS;
    const size_t prow0 = size_t(pick(segs.row0, mi)) + wg_row0;
    for (int e = threadIdx.x; e < T::BN * ROWS; e += kTiledThreads) {
        const int tl = e / ROWS, rl = e % ROWS;
        const int n = tok0 + tl, row = wg_row0 + rl;
        if (row < out && n < batch) {
            const float v = tile[tl * TROW + rl];
            if (partial)
                partial[(size_t(split) * batch + n) * rows_all + prow0 + rl] = v;
            else
                y[size_t(n) * out + row] = f2h_bits(v);
        }
    }
}

struct MfmaCfg {
    int ms, nt, ksplit, groups_per_split, grid_x, grid_y;
};

// split = false: the whole input axis in one workgroup per tile (no workspace needed).
MfmaCfg mfma_cfg(const Problem &p, Segs *segs = nullptr, bool split = true) {
    MfmaCfg c{};
    if (p.batch <= 16) { c.ms = 16; c.nt = 1; }
    else if (p.batch <= 32) { c.ms = 32; c.nt = 1; }
    else if (p.batch <= 64) { c.ms = 32; c.nt = 2; }
    else { c.ms = 32; c.nt = 4; }
    const int64_t G = p.in / kGroup;
    const int chg = c.ms == 16 ? 32 : 16;
    const int rows_per_tile = kMfmaWaves * c.ms;
    int gx = 0;                                      // row tiles, whole ones per matrix
    for (int m = 0; m < p.segs.n; ++m) {
        if (segs) segs->aux0[m] = gx;
        gx += (p.segs.row0[m + 1] - p.segs.row0[m] + rows_per_tile - 1) / rows_per_tile;
    }
    if (segs) segs->aux0[p.segs.n] = gx;
    c.grid_x = gx;
    c.grid_y = (p.batch + c.ms * c.nt - 1) / (c.ms * c.nt);
    const int64_t tiles = int64_t(c.grid_x) * c.grid_y;
    const int64_t nchunks = (G + chg - 1) / chg;
    // At most one workgroup per CU (one workgroup fills a CU's registers: a 257th
    // would run in a second round), and at least 2*NT chunks per split.  Measured on
    // MI355X at batches 64 and 128 (splits 1..8): fewer splits leave CUs idle, more
    // cost more in the batch*out fp32 partial sums each split writes and the reduction
    // re-reads, and a split of few chunks does not amortise its start-up (4096 x 4096
    // at batch 128: 4 splits of 8 chunks beat 8 of 4; 11008 x 4096: 2 splits (172
    // workgroups) beat 3 (258); 4096 x 11008: 8 splits of 12 chunks beat fewer).
    int64_t ks = 256 / tiles;
    if (ks > nchunks / (2 * c.nt)) ks = nchunks / (2 * c.nt);
    if (ks < 1 || !split) ks = 1;
    // whole chunks per split (multiples of 4 groups keep code blocks whole), an even
    // number of them (the kernel runs chunks in pairs)
    int64_t cps = (nchunks + ks - 1) / ks;
    cps += cps & 1;
    int64_t gps = cps * chg;
    c.ksplit = int((G + gps - 1) / gps);
    c.groups_per_split = int(gps);
    return c;
}

template <int K, int BITS, int MS, int NT>
hipError_t launch_t(const Problem &p, const MfmaCfg &c, const Segs &segs, float *partial) {
    const dim3 g(c.grid_x, c.grid_y, c.ksplit), b(kTiledThreads);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    if (segs.n == 1)
        hipLaunchKernelGGL((mfma_kernel<K, BITS, MS, NT, 1>), g, b, 0, p.stream, x, partial,
                           int(p.in), p.batch, c.groups_per_split, segs);
    else
        hipLaunchKernelGGL((mfma_kernel<K, BITS, MS, NT, kMaxSegs>), g, b, 0, p.stream, x,
                           partial, int(p.in), p.batch, c.groups_per_split, segs);
    return hipGetLastError();
}

template <int K, int BITS>
hipError_t launch_kb(const Problem &p, const MfmaCfg &c, const Segs &segs, float *partial) {
    if (c.ms == 16) return launch_t<K, BITS, 16, 1>(p, c, segs, partial);
    if (c.nt == 1) return launch_t<K, BITS, 32, 1>(p, c, segs, partial);
    if (c.nt == 2) return launch_t<K, BITS, 32, 2>(p, c, segs, partial);
    return launch_t<K, BITS, 32, 4>(p, c, segs, partial);
}


// ---------------------------------------------------------------- batch <= 32
constexpr int kKw = 16;                     // waves per workgroup, one share of the input each

// the codes of 8 consecutive groups of one row: 8*K*BITS/32 dwords
template <int K, int BITS> struct Seg {
    static constexpr int NW = 8 * K * BITS / 32;
};

template <int K, int BITS>
__device__ __forceinline__ void load_seg(const uint8_t *p, uint32_t (&w)[Seg<K, BITS>::NW]) {
    constexpr int NW = Seg<K, BITS>::NW;
    if constexpr (NW == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
        for (int h = 0; h < NW / 4; ++h) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + h);
            w[4 * h] = v.x; w[4 * h + 1] = v.y; w[4 * h + 2] = v.z; w[4 * h + 3] = v.w;
        }
    }
}

// code n of a segment (n = group * K + codebook, compile-time after unrolling)
template <int BITS, int NW>
__device__ __forceinline__ uint32_t seg_code(const uint32_t (&w)[NW], int n) {
    if constexpr (BITS == 8) return (w[n >> 2] >> (8 * (n & 3))) & 0xFFu;
    else return (w[n >> 1] >> (16 * (n & 1))) & 0xFFFFu;
}

// Persistent: one workgroup per CU walks 16-row tiles (tile, tile + grid, ...), with
// the next tile's codes loaded while the current one is multiplied.  A wave owns
// units wave, wave + 16, ... (at most MAXU); with a single unit its activations
// are loaded once and kept in registers for every tile.
template <int K, int BITS, int NT, int MAXU, int NSEGS>
__global__ void __launch_bounds__(kKw * kWave)
mfma_kw_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ cb,
               const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int out, int in,
               int batch, int ntiles, const Segs segs) {
    // codes / cb / y / out describe the one matrix when NSEGS == 1; with NSEGS > 1 the
    // matrices come from segs (tiles of each matrix numbered consecutively, segs.aux0)
    constexpr int CBE = BITS == 8 ? K * 256 : 0;
    constexpr int NW = Seg<K, BITS>::NW;
    constexpr int CB = K * BITS / 8;                 // code bytes per group
    __shared__ uint4 cbs[CBE > 0 ? NSEGS * CBE : 1];
    __shared__ float red[2][kKw][NT * 4][kWave];     // double-buffered: one barrier per tile

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = in / kGroup;
    const int U = (G + 31) / 32;                     // units of 32 groups
    const int m = lane & 15, kb = lane >> 4;
    const uint4 *cbg = reinterpret_cast<const uint4 *>(cb);

    // lane (m, kb), unit u: groups g0 .. g0+7 of row m, g0 = 32u + 8kb; MFMA step s uses
    // group g0 + s, so the 32 k of one step are groups {32u + 8kb + s : kb < 4}, in A
    // and B alike.  Units past the last one are clamped for loading and masked in use.
    auto seg_start = [&](int u) { return min(u * 32 + 8 * kb, G - 8); };
    auto unit_of = [&](int i) { return wave + kKw * i; };
    // this lane's code row in global tile `tile` (rows past the matrix end: computed,
    // not stored)
    auto code_row = [&](int tile) -> const uint8_t * {
        if constexpr (NSEGS == 1) {
            return codes + size_t(min(tile * 16 + m, out - 1)) * size_t(G) * CB;
        } else {
            const int mi = range_of(segs.n, segs.aux0, tile);
            const int out_m = segs.row0[mi + 1] - segs.row0[mi];
            const int o = min((tile - segs.aux0[mi]) * 16 + m, out_m - 1);
            return static_cast<const uint8_t *>(segs.codes[mi]) + size_t(o) * size_t(G) * CB;
        }
    };
    auto load_codes = [&](int tile, uint32_t (&cw)[MAXU][NW]) {
        const uint8_t *crow = code_row(tile);
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
            load_seg<K, BITS>(crow + size_t(seg_start(min(unit_of(i), U - 1))) * CB, cw[i]);
    };
    auto load_x = [&](int u, half8 (&bx)[NT][8]) {
        const bool ok = u * 32 + 8 * kb < G;
        const int gc = seg_start(min(u, U - 1));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tok = t * 16 + m;
            const bool okt = ok && tok < batch;
            const uint16_t *xp = x + size_t(min(tok, batch - 1)) * in + size_t(gc) * kGroup;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint4 v = *reinterpret_cast<const uint4 *>(xp + s * kGroup);
                bx[t][s] = okt ? __builtin_bit_cast(half8, v) : half8{};
            }
        }
    };

    // Every first load is issued before anything waits: the codebooks (one 16-byte
    // vector per thread and matrix: K*256 <= 1024 threads), the first tile's codes and,
    // with one unit per wave, the activations; the staging store then waits for the
    // codebooks.
    constexpr int CBPT = (CBE + kKw * kWave - 1) / (kKw * kWave);   // vectors per thread
    uint4 cbv[NSEGS][CBPT > 0 ? CBPT : 1];
    if constexpr (CBE > 0) {
#pragma unroll
        for (int q = 0; q < NSEGS; ++q) {
            const uint4 *src = NSEGS == 1 ? cbg : static_cast<const uint4 *>(segs.cb[min(q, segs.n - 1)]);
#pragma unroll
            for (int i = 0; i < CBPT; ++i)
                cbv[q][i] = src[min(int(threadIdx.x) + i * kKw * kWave, CBE - 1)];
        }
    }
    int tile = blockIdx.x;
    uint32_t cw[MAXU][NW];
    load_codes(tile, cw);
    half8 bx[NT][8];
    if constexpr (MAXU == 1) load_x(wave, bx);
    if constexpr (CBE > 0) {
        // unconditional (threads past the end rewrite the last vector with its own
        // value), so the codebook load is not sunk behind the others
#pragma unroll
        for (int q = 0; q < NSEGS; ++q)
#pragma unroll
            for (int i = 0; i < CBPT; ++i)
                cbs[q * CBE + min(int(threadIdx.x) + i * kKw * kWave, CBE - 1)] = cbv[q][i];
        __syncthreads();
    }

    int buf = 0;
    do {
        // the next tile's codes replace each unit's codes as soon as they are decoded
        // Past the last tile the reload is skipped (16-bit codes, whose codebook gathers
        // share L2 with it) or repeats this tile's cached lines (8-bit codes: there the
        // branch-free form measured faster).
        const bool has_next = tile + int(gridDim.x) < ntiles;     // workgroup-uniform
        const int next = has_next ? tile + int(gridDim.x) : tile;
        const uint8_t *nrow = code_row(next);
        // this tile's matrix: codebooks, output
        const int mi = NSEGS == 1 ? 0 : range_of(segs.n, segs.aux0, tile);
        const uint4 *cbm;
        if constexpr (NSEGS == 1) cbm = BITS == 8 ? cbs : cbg;
        else cbm = BITS == 8 ? cbs + mi * CBE : static_cast<const uint4 *>(segs.cb[mi]);
        float4v acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = float4v{};
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            const int u = unit_of(i);
            if (i > 0 && u >= U) break;              // wave-uniform; unit 0 always runs
            if constexpr (MAXU > 1) load_x(u, bx);
            const bool ok = u * 32 + 8 * kb < G;     // G is a multiple of 8
            half8 a[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                half8 f;
                if constexpr (K > 2) {
                    uint4 v[K];
#pragma unroll
                    for (int k = 0; k < K; ++k) v[k] = cbm[k * (1u << BITS) + seg_code<BITS, NW>(cw[i], s * K + k)];
                    f = fold_fp32<K>(v);
                } else {
                    const uint32_t c0 = seg_code<BITS, NW>(cw[i], s * K);
                    f = __builtin_bit_cast(half8, cbm[c0]);
                    if constexpr (K == 2) {
                        const uint32_t c1 = seg_code<BITS, NW>(cw[i], s * K + 1);
                        f = f + __builtin_bit_cast(half8, cbm[(1u << BITS) + c1]);
                    }
                }
                a[s] = ok ? f : half8{};
            }
            if (BITS == 8 || has_next)
                load_seg<K, BITS>(nrow + size_t(seg_start(min(u, U - 1))) * CB, cw[i]);
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], bx[t][s], acc[t], 0, 0, 0);
        }

        // the 16 waves' tiles, added in wave order
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[buf][wave][t * 4 + r][lane] = acc[t][r];
        __syncthreads();
        int out_m = out, row0 = tile * 16;
        uint16_t *ym = y;
        if constexpr (NSEGS > 1) {
            out_m = segs.row0[mi + 1] - segs.row0[mi];
            row0 = (tile - segs.aux0[mi]) * 16;
            ym = static_cast<uint16_t *>(segs.y[mi]);
        }
        for (int e = threadIdx.x; e < NT * 4 * kWave; e += blockDim.x) {
            const int tr = e / kWave, l = e % kWave;
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < kKw; ++w) sum += red[buf][w][tr][l];
            const int t = tr >> 2, r = tr & 3;
            const int row = row0 + 4 * (l >> 4) + r; // 16x16 result layout
            const int tok = t * 16 + (l & 15);
            if (row < out_m && tok < batch) ym[size_t(tok) * out_m + row] = f2h_bits(sum);
        }
        buf ^= 1;
        tile += gridDim.x;
    } while (tile < ntiles);
}

// units per wave that fit the 128 registers of a 16-wave workgroup without spilling
template <int K, int BITS>
constexpr int kw_max_units(int nt) {
    if (K * BITS > 16) return nt > 1 ? 0 : 1;        // 32-bit code words: one unit, one token tile
    return nt > 1 ? 1 : 3;
}

template <int K, int BITS>
hipError_t launch_kw(const Problem &p) {
    const int G = int(p.in / kGroup);
    const int U = (G + 31) / 32;
    const int maxu = (U + kKw - 1) / kKw;
    Segs segs = p.segs;
    int ntiles = 0;
    for (int m = 0; m < segs.n; ++m) {
        segs.aux0[m] = ntiles;
        ntiles += (segs.row0[m + 1] - segs.row0[m] + 15) / 16;
    }
    segs.aux0[segs.n] = ntiles;
    const dim3 g(ntiles < 256 ? ntiles : 256), b(kKw * kWave);   // one workgroup per CU
    const uint8_t *codes = static_cast<const uint8_t *>(p.codes);
    const uint16_t *cb = static_cast<const uint16_t *>(p.codebooks);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    uint16_t *y = static_cast<uint16_t *>(p.y);
#define AQLM_KW(NT, MU)                                                                        \
    do {                                                                                       \
        if (segs.n == 1)                                                                       \
            hipLaunchKernelGGL((mfma_kw_kernel<K, BITS, NT, MU, 1>), g, b, 0, p.stream, codes, \
                               cb, x, y, int(p.out), int(p.in), p.batch, ntiles, segs);        \
        else                                                                                   \
            hipLaunchKernelGGL((mfma_kw_kernel<K, BITS, NT, MU, kMaxSegs>), g, b, 0, p.stream, \
                               codes, cb, x, y, int(p.out), int(p.in), p.batch, ntiles, segs); \
    } while (0)
    if (p.batch > 16) {
        if constexpr (kw_max_units<K, BITS>(2) >= 1) AQLM_KW(2, 1);
    } else if (maxu <= 1) {
        AQLM_KW(1, 1);
    } else if constexpr (kw_max_units<K, BITS>(1) >= 3) {
        if (maxu <= 2) AQLM_KW(1, 2);
        else AQLM_KW(1, 3);
    }
#undef AQLM_KW
    return hipGetLastError();
}

bool kw_fits(const Problem &p) {
    const int64_t G = p.in / kGroup;
    if (p.batch > 32 || G % 8) return false;
    // 8 codebooks of 8-bit codes: 32 KiB of LDS per matrix, one matrix only
    if (p.K == 8 && p.segs.n > 1) return false;
    const int nt = p.batch > 16 ? 2 : 1;
    const int64_t maxu = ((G + 31) / 32 + kKw - 1) / kKw;
    int lim = 0;
    if (p.B == 8)
        lim = p.K == 1 ? kw_max_units<1, 8>(nt) : p.K == 2 ? kw_max_units<2, 8>(nt)
            : p.K == 4 ? kw_max_units<4, 8>(nt) : kw_max_units<8, 8>(nt);
    else
        lim = p.K == 1 ? kw_max_units<1, 16>(nt) : kw_max_units<2, 16>(nt);
    return maxu <= lim;
}

// ------------------------------------ batch > 64, 8-bit codes, K <= 2, in % 64 == 0
//
// The same product with every global load moved to the load units' LDS path.  A
// workgroup of NW waves owns 32*NW rows x 32*TN tokens; wave w owns rows 32w .. 32w+31
// and all the tokens, so each of its weight fragments is decoded once (lane l: row
// l % 32, one group of 8 inputs) and used for TN MFMAs.  Per k-tile of 64 inputs
// (8 groups):
// * the activations (TN*32 rows of 128 bytes, chunks permuted by the row's place in
//   the bank period) and the codes (32*NW rows of 8*K bytes) arrive by
//   global_load_lds_dwordx4 / global_load_lds_dword in rings three k-tiles deep,
//   issued two (activations) and three (codes) k-tiles ahead;
// * the codebook gathers of k-tile kt+1 (from the LDS-resident codebooks) are issued
//   between the MFMAs of k-tile kt, two per k-step, and folded after them;
// * one barrier per k-tile; no register holds staged data.
// Lane l of a wave takes groups 4(l/32) .. 4(l/32)+3 of its row in the four k-steps
// of a k-tile (one 8-byte code read), and the activation fragment of the same group,
// so both MFMA operands hold the same 8 inputs in a lane.
//
// No one unit bounds it.  Per k-tile and CU (NW = 8, TN = 4) the MFMAs take 1024
// cycles, the activation-fragment reads ~1024 LDS cycles (8 per conflict-free 64-lane
// 16-byte read) and the gathers ~850 (~13 per random one); measured on MI355X a k-tile
// takes ~0.85 us (~2040 cycles), with the LDS active ~45% of the time.  Timing variants
// that each drop one phase (their results wrong, timing only) at batch 2048: without
// the staging loads -27%, without the gathers -12%, without the fragment reads -10%,
// without the barrier -5%, without the MFMAs -4%: the phases add up more than they
// overlap at two waves per SIMD.  Measured slower: 64-row wave tiles at one wave per
// SIMD (~1.1 us per k-tile), 8 copies of the codebooks over the bank period (9.8
// instead of 13.2 cycles per gather in isolation, no gain in the kernel), and staging
// through registers (global loads, then ds_write one k-tile later) instead of the LDS
// DMA (3-4% slower).
constexpr int kDqXcds = 8;

template <int NW, int TN, int K>
struct DqTile {
    static constexpr int THREADS = NW * kWave;
    static constexpr int BM = 32 * NW;           // rows per workgroup
    static constexpr int BN = 32 * TN;           // tokens per workgroup
    static constexpr int XB = BN * 128;          // activation stage: BN rows of 64 fp16
    static constexpr int CR = 8 * K;             // code bytes per row and k-tile
    static constexpr int CS = BM * CR;           // code stage
    static constexpr int XR = BN / (8 * NW);     // activation rounds per wave (8 rows of 128 B)
    static constexpr int CRW = CS / (256 * NW);  // code rounds per wave (64 dwords)
    static constexpr int LOADS = XR + CRW;       // loads per wave and k-tile
    static_assert(XR >= 1 && BN % (8 * NW) == 0, "whole activation rounds per wave");
    static_assert(CRW >= 1 && CS % (256 * NW) == 0, "whole code rounds per wave");
    static_assert(NW % 2 == 0, "8*NW rows per activation round, a multiple of 16");
    // chunk c of staged activation row r
    static __device__ __forceinline__ uint32_t off(int r, int c) {
        return uint32_t(r) * 128u + (uint32_t(c ^ ((r >> 1) & 7)) << 4);
    }
};

template <int K, int NW, int TN, int NS>
__global__ void __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_dq_kernel(const uint16_t *__restrict__ x, float *__restrict__ partial, int in, int batch,
               int kt_per_split, int tiles_m, int tiles_n, int ntiles, int per_xcd,
               int splits_fastest, const Segs segs) {
    typedef DqTile<NW, TN, K> T;
    __shared__ __attribute__((aligned(1024))) char xs0[T::XB];
    __shared__ __attribute__((aligned(1024))) char xs1[T::XB];
    __shared__ __attribute__((aligned(1024))) char xs2[T::XB];
    __shared__ __attribute__((aligned(256))) char cs0[T::CS];
    __shared__ __attribute__((aligned(256))) char cs1[T::CS];
    __shared__ __attribute__((aligned(256))) char cs2[T::CS];
    __shared__ uint4 cbs[K * 256];

    // workgroup b runs on XCD b % 8; each XCD takes a contiguous run of tiles, row tiles
    // fastest.  splits_fastest = 0: the splits outermost, so the workgroups of one XCD
    // share one split's activations in its L2; 1: the splits of a tile fastest (whole
    // tiles per XCD), so a tile's partial sums stay in one XCD's L2 for the partial-sum
    // kernel (dq_partial_sum_kernel)
    const int b = blockIdx.x;
    const int L = (b % kDqXcds) * per_xcd + b / kDqXcds;
    if (L >= ntiles) return;                     // the whole workgroup: no barrier skipped
    const int per_split = tiles_m * tiles_n;
    const int ksplit = ntiles / per_split;
    const int split = splits_fastest ? L % ksplit : L / per_split;
    const int rem = splits_fastest ? L / ksplit : L - split * per_split;
    const int tn = rem / tiles_m, tm = rem - tn * tiles_m;

    // this row tile's matrix (row tiles of each matrix numbered consecutively, segs.aux0)
    const int mi = seg_of<NS>(segs.n, segs.aux0, tm);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const int rows_all = seg_total<NS>(segs.n, segs.row0);
    const uint8_t *__restrict__ codes = static_cast<const uint8_t *>(pick(segs.codes, mi));
    const uint4 *__restrict__ cbg = static_cast<const uint4 *>(pick(segs.cb, mi));
    uint16_t *__restrict__ y = static_cast<uint16_t *>(pick(segs.y, mi));
    const int row0 = (tm - pick(segs.aux0, mi)) * T::BM;
    const int tok0 = tn * T::BN;
    const int G = in / kGroup;
    const int kt0 = split * kt_per_split;
    const int nk = min(kt_per_split, G / 8 - kt0);   // >= 1

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 31, h = lane >> 5;

    // Codebooks: K*256 vectors, loaded first (clamped duplicates past the end), stored
    // once the rings are in flight.
    constexpr int CBE = K * 256;
    constexpr int CBPT = (CBE + T::THREADS - 1) / T::THREADS;
    uint4 cbv[CBPT];
#pragma unroll
    for (int i = 0; i < CBPT; ++i) cbv[i] = cbg[min(int(threadIdx.x) + i * T::THREADS, CBE - 1)];

    // Activation round i of wave w fills staged rows 8(w + NW*i) .. +7 (1 KiB); lane l
    // fills row 8(w + NW*i) + l/8, slot l%8, i.e. logical chunk (l%8) ^ ((row >> 1) & 7),
    // the same chunk in every round (8*NW is a multiple of 16).  Rows past the batch are
    // clamped duplicates whose outputs are never stored.
    const int xrow = 8 * wave + (lane >> 3);
    const int xcl = (lane & 7) ^ ((xrow >> 1) & 7);
    const uint16_t *xsrc[T::XR];
#pragma unroll
    for (int i = 0; i < T::XR; ++i)
        xsrc[i] = x + size_t(min(tok0 + xrow + 8 * NW * i, batch - 1)) * size_t(in) +
                  size_t(kt0) * 64 + 8 * xcl;
    // Code round j of wave w fills code-stage bytes 256 (w*CRW + j) .. +255: lane l the
    // dword q = 64 (w*CRW + j) + l, byte 4q % CR of row 4q / CR.  Rows past the matrix are
    // clamped duplicates.
    const uint8_t *csrc[T::CRW];
#pragma unroll
    for (int j = 0; j < T::CRW; ++j) {
        const int q = 64 * (wave * T::CRW + j) + lane;
        const int r = 4 * q / T::CR;
        csrc[j] = codes + size_t(min(row0 + r, out - 1)) * size_t(G) * K + size_t(kt0) * T::CR +
                  (4 * q) % T::CR;
    }
    auto lds_addr = [&](char *p, uint32_t wave_off) {
        return __builtin_amdgcn_readfirstlane(
            uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)p)) + wave_off);
    };
    const uint32_t xa0 = lds_addr(xs0, 1024u * wave), xa1 = lds_addr(xs1, 1024u * wave),
                   xa2 = lds_addr(xs2, 1024u * wave);
    const uint32_t ca0 = lds_addr(cs0, 256u * T::CRW * wave), ca1 = lds_addr(cs1, 256u * T::CRW * wave),
                   ca2 = lds_addr(cs2, 256u * T::CRW * wave);
    // The loads are asm so that the compiler does not track them (its wait insertion
    // would make LDS reads wait for every load into LDS in flight); the waits they need
    // are the explicit vmcnt ones.  No output register; m0 holds the wave's LDS
    // destination, and no other code of this kernel uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    auto dma_x = [&](uint32_t stage, int kt) {
#pragma unroll
        for (int i = 0; i < T::XR; ++i) {
            const uint16_t *g = xsrc[i] + size_t(kt) * 64;
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(g), "s"(stage + uint32_t(1024 * NW * i))
                         : "memory", "m0");
        }
    };
    auto dma_c = [&](uint32_t stage, int kt) {
#pragma unroll
        for (int j = 0; j < T::CRW; ++j) {
            const uint8_t *g = csrc[j] + size_t(kt) * T::CR;
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                         :
                         : "v"(g), "s"(stage + uint32_t(256 * j))
                         : "memory", "m0");
        }
    };
#pragma clang diagnostic pop
    // s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for)
    auto wait_vm = [](auto n) {
        constexpr int N = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    };

    // this lane's codes of a k-tile: groups 4h .. 4h+3 of row 32w + m
    const int coff = (32 * wave + m) * T::CR + 4 * K * h;
    auto read_codes = [&](const char *cst) -> u32x2 {
        if constexpr (K == 2) return *reinterpret_cast<const u32x2 *>(cst + coff);
        else return u32x2{*reinterpret_cast<const uint32_t *>(cst + coff), 0u};
    };
    // codebook vectors of group 4h + s
    auto gather = [&](const u32x2 &cw, int s, uint4 &v0, uint4 &v1) {
        if constexpr (K == 2) {
            const uint32_t w = s < 2 ? cw.x : cw.y;
            v0 = cbs[(w >> (16 * (s & 1))) & 0xFFu];
            v1 = cbs[256 + ((w >> (16 * (s & 1) + 8)) & 0xFFu)];
        } else {
            v0 = cbs[(cw.x >> (8 * s)) & 0xFFu];
        }
    };
    // K = 2: the fp16 sum rounds the exact sum once, the value aqlm_dequantize writes
    auto fold = [&](const uint4 &v0, const uint4 &v1) -> half8 {
        if constexpr (K == 2) return __builtin_bit_cast(half8, v0) + __builtin_bit_cast(half8, v1);
        else return __builtin_bit_cast(half8, v0);
    };

    float16v acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = float16v{};

    // Prologue: codes of k-tiles 0..2 and activations of 0..1 in flight; the codebook
    // store waits for everything; then k-tile 0 is decoded, and a barrier frees code
    // stage 0 for k-tile 3.  Past the last k-tile the loads are clamped duplicates into
    // stages nobody reads (no conditional load).
    dma_c(ca0, 0);
    dma_x(xa0, 0);
    dma_c(ca1, min(1, nk - 1));
    dma_x(xa1, min(1, nk - 1));
    dma_c(ca2, min(2, nk - 1));
#pragma unroll
    for (int i = 0; i < CBPT; ++i) cbs[min(int(threadIdx.x) + i * T::THREADS, CBE - 1)] = cbv[i];
    wait_vm(std::integral_constant<int, 0>{});
    __syncthreads();
    half8 acur[4];
    {
        const u32x2 cw = read_codes(cs0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 v0, v1{};
            gather(cw, s, v0, v1);
            acur[s] = fold(v0, v1);
        }
    }
    __syncthreads();

    // k-tile kt: activations in stage kt % 3, codes of kt+1 in code stage (kt+1) % 3;
    // the step refills activation stage (kt+2) % 3 and code stage kt % 3.
    int kt = 0;
    auto step = [&](const char *xcur, const char *cnext, uint32_t xdma, uint32_t cdma) {
        dma_x(xdma, min(kt + 2, nk - 1));
        dma_c(cdma, min(kt + 3, nk - 1));
        auto frags = [&](int s, half8 (&xb)[TN]) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
                xb[j] = *reinterpret_cast<const half8 *>(xcur + T::off(32 * j + m, 4 * h + s));
        };
        half8 xb[2][TN];
        uint4 g0[4], g1[4];
        frags(0, xb[0]);
        const u32x2 cw = read_codes(cnext);
        // Order pinned per k-step: the next step's fragment reads, then this step's two
        // gathers, then its MFMAs, so that an MFMA waits for its own fragments only.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s + 1 < 4) frags(s + 1, xb[(s + 1) & 1]);
            gather(cw, s, g0[s], g1[s]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xb[s & 1][j], acur[s], acc[j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acur[s] = fold(g0[s], g1[s]);
        // this wave's loads of k-tile kt+1 (activations) and kt+2 (codes) have landed;
        // its LDS reads of this k-tile were consumed above
        wait_vm(std::integral_constant<int, T::LOADS>{});
        __builtin_amdgcn_s_barrier();
        return ++kt < nk;
    };
    while (step(xs0, cs1, xa2, ca0) && step(xs1, cs2, xa0, ca1) && step(xs2, cs0, xa1, ca2)) {
    }
    wait_vm(std::integral_constant<int, 0>{});   // no load may land after the workgroup ends

    // result register r of lane l: token 32j + 8(r/4) + 4h + r%4, row 32w + m; 32 lanes
    // store 32 consecutive rows of one token
    const int lrow = row0 + 32 * wave + m;
    const size_t prow = size_t(pick(segs.row0, mi)) + lrow;
    const bool full = row0 + T::BM <= out && tok0 + T::BN <= batch;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = tok0 + 32 * j + 8 * (r >> 2) + 4 * h + (r & 3);
            if (full || (lrow < out && tok < batch)) {
                if (partial)
                    partial[(size_t(split) * batch + tok) * rows_all + prow] = acc[j][r];
                else
                    y[size_t(tok) * out + lrow] = f2h_bits(acc[j][r]);
            }
        }
    }
}

struct DqCfg {
    int tn, ksplit, kt_per_split, tiles_m, tiles_n, ntiles, per_xcd, splits_fastest;
};

constexpr int kDqWaves = 8;

// From batch 65: at 33..64 tokens the tiled kernel above measured faster on the 7B layer.
bool dq_fits(const Problem &p) {
    return p.B == 8 && (p.K == 1 || p.K == 2) && p.batch > 64 && p.in % 64 == 0;
}

// split = false: the whole input axis in one workgroup per tile (no workspace needed).
DqCfg dq_cfg(const Problem &p, Segs *segs = nullptr, bool split = true) {
    DqCfg c{};
    // 64-token tiles up to batch 128 (more tiles, fewer input-axis splits: measured faster
    // on the 7B shapes at batch 128), 128-token tiles above
    c.tn = p.batch > 128 ? 4 : 2;
    const int bm = 32 * kDqWaves, bn = 32 * c.tn;
    int tm = 0;
    for (int m = 0; m < p.segs.n; ++m) {
        if (segs) segs->aux0[m] = tm;
        tm += (p.segs.row0[m + 1] - p.segs.row0[m] + bm - 1) / bm;
    }
    if (segs) segs->aux0[p.segs.n] = tm;
    c.tiles_m = tm;
    c.tiles_n = (p.batch + bn - 1) / bn;
    const int64_t tiles = int64_t(c.tiles_m) * c.tiles_n;
    const int64_t nkt = p.in / 64;
    // One workgroup per CU (a workgroup of 8 waves fills its registers).  Each split adds
    // a batch x out fp32 partial sum written and read back, so splits keep at least 16
    // k-tiles unless that leaves fewer than 64 workgroups (then at least 4).  Measured on
    // MI355X, 7B shapes: 4096 x 4096 at batch 256 takes 32.9 us in 4 splits against 34.6
    // in 8, 4096 x 11008 41.7 in 8 against 47.5 in 4.
    const int64_t fill = 256 / tiles;
    int64_t ks = std::min(fill, nkt / 16);
    if (tiles * std::max<int64_t>(ks, 1) < 64) ks = std::min(fill, nkt / 4);
    if (ks < 1 || !split) ks = 1;
    const int64_t kps = (nkt + ks - 1) / ks;
    c.kt_per_split = int(kps);
    c.ksplit = int((nkt + kps - 1) / kps);
    const int64_t n = tiles * c.ksplit;
    c.ntiles = int(n);
    c.per_xcd = int((n + kDqXcds - 1) / kDqXcds);
    // Up to batch 256 the splits of a tile run on one XCD (whole tiles per XCD: a multiple
    // of the split count) and their partial sums are added there.  Measured on MI355X, 2x8,
    // per call: batch 128 4096x4096 17.8 against 20.8 us, 11008x4096 27.9 against 29.8,
    // 4096x11008 27.4 against 29.5; batch 256 4096x4096 25.2 against 32.6; at batch 512 the
    // XCD's share of a long input's activations no longer stays in its L2 (4096x11008 64.4
    // against 60.1), so the splits stay outermost there.
    c.splits_fastest = c.ksplit > 1 && p.batch <= 256 ? 1 : 0;
    if (c.splits_fastest) c.per_xcd = (c.per_xcd + c.ksplit - 1) / c.ksplit * c.ksplit;
    return c;
}

template <int K, int TN>
hipError_t launch_dq_t(const Problem &p, const DqCfg &c, const Segs &segs, float *partial) {
    const dim3 g(c.per_xcd * kDqXcds), b(kDqWaves * kWave);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    if (segs.n == 1)
        hipLaunchKernelGGL((mfma_dq_kernel<K, kDqWaves, TN, 1>), g, b, 0, p.stream, x, partial,
                           int(p.in), p.batch, c.kt_per_split, c.tiles_m, c.tiles_n, c.ntiles,
                           c.per_xcd, c.splits_fastest, segs);
    else
        hipLaunchKernelGGL((mfma_dq_kernel<K, kDqWaves, TN, kMaxSegs>), g, b, 0, p.stream, x,
                           partial, int(p.in), p.batch, c.kt_per_split, c.tiles_m, c.tiles_n,
                           c.ntiles, c.per_xcd, c.splits_fastest, segs);
    return hipGetLastError();
}

template <int K>
hipError_t launch_dq_k(const Problem &p, const DqCfg &c, const Segs &segs, float *partial) {
    if (c.tn == 4) return launch_dq_t<K, 4>(p, c, segs, partial);
    return launch_dq_t<K, 2>(p, c, segs, partial);
}

// The split partial sums of mfma_dq_kernel with splits_fastest, each on the XCD that ran its
// tile (whole tiles per XCD), so that it reads them from that XCD's L2: one wave per (tile,
// token), lane l rows 4l .. 4l+3 of the tile's 256, 16-byte loads, the splits added in
// order.  Needs every matrix's first row and row count, and each y_m, 4-element aligned
// (launch_dq checks; otherwise the generic partial-sum kernel runs).
template <int NS, int PMAX>
__global__ void __launch_bounds__(64)
dq_partial_sum_kernel(const float *__restrict__ partial, int batch, int ksplit, int tiles_m, int tiles_n,
                      int tiles_per_xcd, int bn, const Segs segs) {
    const int b = blockIdx.x;
    const int j = b / kDqXcds;
    const int ti = j / bn, tin = j - ti * bn;
    const int t = (b % kDqXcds) * tiles_per_xcd + ti;
    if (t >= tiles_m * tiles_n) return;
    const int tn = t / tiles_m, tm = t - tn * tiles_m;
    const int tok = tn * bn + tin;
    if (tok >= batch) return;
    const int mi = seg_of<NS>(segs.n, segs.aux0, tm);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const int rows_all = seg_total<NS>(segs.n, segs.row0);
    const int lrow = (tm - pick(segs.aux0, mi)) * (32 * kDqWaves) + int(threadIdx.x) * 4;
    if (lrow >= out) return;                      // out is a multiple of 4
    const size_t prow = size_t(pick(segs.row0, mi)) + lrow;
    float4 v[PMAX];
#pragma unroll
    for (int q = 0; q < PMAX; ++q)
        v[q] = *reinterpret_cast<const float4 *>(partial + (size_t(min(q, ksplit - 1)) * batch + tok) * rows_all + prow);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
        const bool in = q < ksplit;
        s0 += in ? v[q].x : 0.0f;
        s1 += in ? v[q].y : 0.0f;
        s2 += in ? v[q].z : 0.0f;
        s3 += in ? v[q].w : 0.0f;
    }
    uint16_t *y = static_cast<uint16_t *>(pick(segs.y, mi)) + size_t(tok) * out + lrow;
    *reinterpret_cast<uint2 *>(y) = uint2{f2h_bits(s0) | (uint32_t(f2h_bits(s1)) << 16),
                                          f2h_bits(s2) | (uint32_t(f2h_bits(s3)) << 16)};
}

template <int NS>
void launch_dq_partial_sum_ns(const DqCfg &c, const Segs &segs, const float *partial, int batch,
                              hipStream_t s) {
    const int tpx = c.per_xcd / c.ksplit, bn = 32 * c.tn;
    const dim3 g(unsigned(kDqXcds * tpx * bn)), b(kWave);
    if (c.ksplit <= 4)
        hipLaunchKernelGGL((dq_partial_sum_kernel<NS, 4>), g, b, 0, s, partial, batch, c.ksplit, c.tiles_m,
                           c.tiles_n, tpx, bn, segs);
    else if (c.ksplit <= 8)
        hipLaunchKernelGGL((dq_partial_sum_kernel<NS, 8>), g, b, 0, s, partial, batch, c.ksplit, c.tiles_m,
                           c.tiles_n, tpx, bn, segs);
    else
        hipLaunchKernelGGL((dq_partial_sum_kernel<NS, 16>), g, b, 0, s, partial, batch, c.ksplit, c.tiles_m,
                           c.tiles_n, tpx, bn, segs);
}

hipError_t launch_dq_partial_sum(const Problem &p, const DqCfg &c, const Segs &segs, const float *partial) {
    bool aligned = c.splits_fastest && (reinterpret_cast<uintptr_t>(partial) & 15u) == 0 && c.ksplit <= 16;
    for (int m = 0; m <= segs.n; ++m) aligned = aligned && segs.row0[m] % 4 == 0;
    for (int m = 0; m < segs.n; ++m) aligned = aligned && (reinterpret_cast<uintptr_t>(segs.y[m]) & 7u) == 0;
    if (!aligned) return launch_partial_sum_segs(partial, segs, p.batch, c.ksplit, p.stream);
    if (segs.n == 1) launch_dq_partial_sum_ns<1>(c, segs, partial, p.batch, p.stream);
    else launch_dq_partial_sum_ns<kMaxSegs>(c, segs, partial, p.batch, p.stream);
    return hipGetLastError();
}

hipError_t launch_dq(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const DqCfg c = dq_cfg(p, &segs, workspace != nullptr);
    float *partial = c.ksplit > 1 ? static_cast<float *>(workspace) : nullptr;
    const hipError_t e = p.K == 1 ? launch_dq_k<1>(p, c, segs, partial) : launch_dq_k<2>(p, c, segs, partial);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_dq_partial_sum(p, c, segs, partial);
}

}  // namespace

bool mfma_supported(const Problem &p) {
    // K in {1, 2} for either code width; 4 and 8 codebooks of 8-bit codes
    const bool kb = ((p.K == 1 || p.K == 2) && (p.B == 8 || p.B == 16)) ||
                    ((p.K == 4 || p.K == 8) && p.B == 8);
    if (!kb) return false;
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
    if (kw_fits(p)) return 0;
    if (dq_fits(p)) {
        const DqCfg c = dq_cfg(p);
        return c.ksplit > 1 ? size_t(c.ksplit) * size_t(p.batch) * size_t(p.out) * sizeof(float) : 0;
    }
    const MfmaCfg c = mfma_cfg(p);
    return c.ksplit > 1 ? size_t(c.ksplit) * size_t(p.batch) * size_t(p.out) * sizeof(float) : 0;
}

// workspace: KSPLIT x batch x T fp32 partial tiles; null: one split (KSPLIT = 1)
hipError_t launch_mfma(const Problem &p, void *workspace) {
    if (kw_fits(p)) {
        if (p.B == 8)
            return p.K == 1 ? launch_kw<1, 8>(p) : p.K == 2 ? launch_kw<2, 8>(p)
                 : p.K == 4 ? launch_kw<4, 8>(p) : launch_kw<8, 8>(p);
        return p.K == 1 ? launch_kw<1, 16>(p) : launch_kw<2, 16>(p);
    }
    if (dq_fits(p)) return launch_dq(p, workspace);
    Segs segs = p.segs;
    const MfmaCfg c = mfma_cfg(p, &segs, workspace != nullptr);
    float *partial = c.ksplit > 1 ? static_cast<float *>(workspace) : nullptr;
    hipError_t e;
    if (p.B == 8)
        e = p.K == 1 ? launch_kb<1, 8>(p, c, segs, partial)
          : p.K == 2 ? launch_kb<2, 8>(p, c, segs, partial)
          : p.K == 4 ? launch_kb<4, 8>(p, c, segs, partial) : launch_kb<8, 8>(p, c, segs, partial);
    else
        e = p.K == 1 ? launch_kb<1, 16>(p, c, segs, partial) : launch_kb<2, 16>(p, c, segs, partial);
    if (e != hipSuccess || c.ksplit == 1) return e;
    return launch_partial_sum_segs(partial, segs, p.batch, c.ksplit, p.stream);
}

}  // namespace aqlm
