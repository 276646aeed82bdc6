// Prefill-size batches: W decoded once per call, then a dense fp16 GEMM on the
// gfx950 matrix cores.
//
// At a few hundred tokens and more the product is compute-bound, and re-decoding W
// for every token tile (what the smaller-batch matrix-core kernels do) costs more than
// decoding it once: launch_dequant16 writes the dense fp16 W (the bits aqlm_dequantize
// writes, the fold of page "AQLM (Additive Quantization for LLMs)", section "Niveau
// intermediaire", rounded once) into the workspace, and prefill_gemm_kernel multiplies
// it with x: Y[n][o] = sum_i W[o][i] x[n][i], fp16 x fp16 with fp32 accumulation
// (v_mfma_f32_32x32x16_f16), y rounded once to fp16.
//
// * Workgroup = 4 waves (2 x 2) on BM = 64*TM rows x BN = 64*TN tokens (256 x 128 or
//   128 x 128); a wave owns 32*TM rows x 32*TN tokens (TM*TN accumulator tiles of
//   32 x 32).
// * Both operands are contiguous along the input axis.  Each k-tile of BK = 32 or 64
//   inputs is staged in LDS (double-buffered, one barrier per k-tile): BK*2 bytes per
//   tile row, the 16-byte chunks of a row permuted by its place in the 256-byte bank
//   period, so that a fragment read (16 lanes: 16 rows, one chunk) and a staging
//   store (16 lanes: all chunks of 16 / (BK/8) rows) each touch all 64 banks once.
//   The next k-tile's global loads are issued before the current tile's MFMAs; the
//   fragments of k-step s+1 are read from LDS while the MFMAs of step s run.
// * MFMA operands: A = activations (lane l: token l % 32, inputs 8(l/32) .. +7 of the
//   k-step), B = weights (lane l: row l % 32, the same inputs).  Result register r of
//   lane l is token 8(r/4) + 4(l/32) + r%4, row l % 32: 32 lanes store 32 consecutive
//   outputs of one token row (64 bytes).
// * Tiles are numbered row-panel-major and cut into 8 contiguous runs, one per XCD
//   (workgroup b runs on XCD b % 8), so that the token tiles of one row panel share
//   that XCD's L2.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kPfThreads = 256;            // 4 waves
constexpr int kXcds = 8;

// BK inputs per k-tile (32 or 64): CPR = BK/8 chunks of 16 bytes per staged row.  WM
// waves along the rows (2 or 4), two along the tokens.
template <int TM, int TN, int BK, int WM = 2>
struct PfTile {
    static constexpr int THREADS = 2 * WM * kWave;
    static constexpr int BM = WM * 32 * TM;                  // rows per workgroup
    static constexpr int BN = 64 * TN;                       // tokens per workgroup
    static constexpr int CPR = BK / 8;                       // chunks per staged row
    static constexpr int ROWB = BK * 2;                      // LDS bytes per staged row
    static constexpr int RPL = THREADS / CPR;                // staged rows per load round
    static constexpr int LOADS = (BM + BN) / RPL;            // 16-B loads per thread
    static constexpr int BUF = (BM + BN) * ROWB;             // LDS bytes per buffer
    static constexpr int STEPS = BK / 16;                    // MFMA k-steps per k-tile
    static_assert(BN % RPL == 0 && BM % RPL == 0, "a load round is all tokens or all weights");
    // chunk c of staged row r: the rows that share a bank period (16 / CPR of them)
    // get distinct chunk permutations
    static __device__ __forceinline__ uint32_t off(int r, int c) {
        return uint32_t(r) * ROWB + (uint32_t(c ^ ((r / (16 / CPR)) & (CPR - 1))) << 4);
    }
};

template <int TM, int TN, int BK>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_gemm_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ x,
                    uint16_t *__restrict__ y, int out, int in, int batch, int tiles_n, int ntiles,
                    int per_xcd) {
    typedef PfTile<TM, TN, BK> T;
    __shared__ __attribute__((aligned(16))) char lds[2 * T::BUF];

    const int b = blockIdx.x;
    const int L = (b % kXcds) * per_xcd + b / kXcds;
    if (L >= ntiles) return;                     // the whole workgroup: no barrier skipped
    const int row0 = (L / tiles_n) * T::BM;
    const int tok0 = (L % tiles_n) * T::BN;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wm = wave & 1, wn = wave >> 1;
    const int nk = (in + BK - 1) / BK;

    // Staging: thread t, load i covers staged row t / CPR + i * RPL, chunk t % CPR;
    // rows 0 .. BN-1 are token rows, BN .. BN+BM-1 weight rows (a load round never
    // straddles the two).  Rows past the matrix are clamped duplicates (never stored);
    // chunks past the input axis are zeroed.
    const int sc = threadIdx.x % T::CPR;
    const int sr = threadIdx.x / T::CPR;
    auto gload = [&](int kt, uint4 (&v)[T::LOADS]) {
        const int k = min(kt * BK + 8 * sc, in - 8);
#pragma unroll
        for (int i = 0; i < T::LOADS; ++i) {
            const int r = sr + i * T::RPL;
            const uint16_t *src;
            if (i * T::RPL < T::BN)
                src = x + size_t(min(tok0 + r, batch - 1)) * size_t(in) + k;
            else
                src = W + size_t(min(row0 + r - T::BN, out - 1)) * size_t(in) + k;
            v[i] = *reinterpret_cast<const uint4 *>(src);
        }
    };
    auto sstore = [&](int buf, int kt, const uint4 (&v)[T::LOADS]) {
        // an AND with an opaque mask: a select would become a branch around the load
        uint32_t msk = kt * BK + 8 * sc < in ? 0xFFFFFFFFu : 0u;
        asm volatile("" : "+v"(msk));
        char *base = lds + buf * T::BUF;
#pragma unroll
        for (int i = 0; i < T::LOADS; ++i) {
            const int r = sr + i * T::RPL;
            *reinterpret_cast<uint4 *>(base + T::off(r, sc)) =
                make_uint4(v[i].x & msk, v[i].y & msk, v[i].z & msk, v[i].w & msk);
        }
    };
    // fragments of k-step s (inputs 16s .. 16s+15 of the k-tile): chunk 2s + lane/32
    auto frags = [&](const char *base, int s, half8 (&xa)[TN], half8 (&wb)[TM]) {
        const int c = 2 * s + (lane >> 5);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            xa[j] = *reinterpret_cast<const half8 *>(
                base + T::off(wn * 32 * TN + 32 * j + (lane & 31), c));
#pragma unroll
        for (int i = 0; i < TM; ++i)
            wb[i] = *reinterpret_cast<const half8 *>(
                base + T::off(T::BN + wm * 32 * TM + 32 * i + (lane & 31), c));
    };

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = float16v{};

    uint4 v[T::LOADS];
    gload(0, v);
    sstore(0, 0, v);
    __syncthreads();

    int kt = 0;
    do {
        const int buf = kt & 1;
        gload(min(kt + 1, nk - 1), v);           // in flight during this tile's MFMAs
        const char *base = lds + buf * T::BUF;
        half8 xa[2][TN], wb[2][TM];
        frags(base, 0, xa[0], wb[0]);
#pragma unroll
        for (int s = 0; s < T::STEPS; ++s) {
            if (s + 1 < T::STEPS) frags(base, s + 1, xa[(s + 1) & 1], wb[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[s & 1][j], wb[s & 1][i],
                                                                       acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        sstore(buf ^ 1, kt + 1, v);
        __syncthreads();
    } while (++kt < nk);

    // full tiles store unconditionally; edge tiles check every output
    const bool full = row0 + T::BM <= out && tok0 + T::BN <= batch;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = row0 + wm * 32 * TM + 32 * i + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = tok0 + wn * 32 * TN + 32 * j + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (full || (row < out && tok < batch))
                    y[size_t(tok) * out + row] = f2h_bits(acc[i][j][r]);
            }
        }
    }
}

// The same product with the k-tiles staged by the load units straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's LDS base + 16 l), in
// three stages: the loads of k-tile kt+2 are issued before the MFMAs of k-tile kt, so
// two k-tiles of MFMAs cover their latency, and no register holds staged data.  The
// bank permutation is applied on the global side: lane l of a wave's load round
// fetches the chunk that belongs at its LDS slot.  For in % 64 == 0 (no chunk past
// the input axis); the stages are separate arrays so that LDS reads of one are not
// ordered behind the loads into another.
template <int TM, int TN, int WM>
__global__ void __launch_bounds__(2 * WM * kWave) __attribute__((amdgpu_waves_per_eu(WM / 2, WM / 2)))
prefill_gemm_dma_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ x,
                        uint16_t *__restrict__ y, int out, int in, int batch, int tiles_n,
                        int ntiles, int per_xcd) {
    typedef PfTile<TM, TN, 64, WM> T;
    static_assert(T::CPR == 8 && T::RPL % 16 == 0, "8 rows of 8 chunks per wave and round");
    __shared__ __attribute__((aligned(1024))) char st0[T::BUF];
    __shared__ __attribute__((aligned(1024))) char st1[T::BUF];
    __shared__ __attribute__((aligned(1024))) char st2[T::BUF];

    const int b = blockIdx.x;
    const int L = (b % kXcds) * per_xcd + b / kXcds;
    if (L >= ntiles) return;                     // the whole workgroup: no barrier skipped
    const int row0 = (L / tiles_n) * T::BM;
    const int tok0 = (L % tiles_n) * T::BN;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave % WM, wn = wave / WM;
    const int nk = in / 64;

    // Round i of wave w fills staged rows 8w + RPL*i .. +7 (1 KB); lane l fills row
    // 8w + RPL*i + l/8, slot l%8, i.e. logical chunk (l%8) ^ ((row >> 1) & 7), the same
    // chunk in every round (RPL, a multiple of 16, does not change (row >> 1) & 7).
    const int lrow = 8 * wave + (lane >> 3);
    const int cl = (lane & 7) ^ ((lrow >> 1) & 7);
    const uint16_t *src[T::LOADS];
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
        const int r = lrow + T::RPL * i;
        src[i] = T::RPL * i < T::BN ? x + size_t(min(tok0 + r, batch - 1)) * size_t(in) + 8 * cl
                                : W + size_t(min(row0 + r - T::BN, out - 1)) * size_t(in) + 8 * cl;
    }
    // The loads are written in asm so that the compiler does not track them: its wait
    // insertion would otherwise, where the loop's paths join, make the first LDS read of
    // a step wait for every load into LDS in flight (including the one just issued for
    // k-tile kt+2).  The waits they need are the explicit ones below.  The asm has no
    // output register; it reads its address registers when it issues, and m0 holds the
    // wave's LDS destination.
    // LDS byte address of each stage's first row of this wave
    auto lds_addr = [&](char *stage) {
        return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(
                   (__attribute__((address_space(3))) char *)stage)) + uint32_t(8 * wave * T::ROWB));
    };
    const uint32_t a0 = lds_addr(st0), a1 = lds_addr(st1), a2 = lds_addr(st2);
    // m0 is a reserved register: clang warns that the clobber may not be honoured, but
    // no other code of this kernel uses m0 (checked in the generated assembly).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    auto dma = [&](uint32_t stage, int kt) {
#pragma unroll
        for (int i = 0; i < T::LOADS; ++i) {
            const uint16_t *g = src[i] + size_t(kt) * 64;
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(g), "s"(stage + uint32_t(T::RPL * i * T::ROWB))
                         : "memory", "m0");
        }
    };
#pragma clang diagnostic pop
    // s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for)
    auto wait_vm = [](auto n) {
        constexpr int N = decltype(n)::value;
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    };

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = float16v{};

    auto compute = [&](const char *base) {
        auto frags = [&](int s, half8 (&xa)[TN], half8 (&wb)[TM]) {
            const int c = 2 * s + (lane >> 5);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                xa[j] = *reinterpret_cast<const half8 *>(
                    base + T::off(wn * 32 * TN + 32 * j + (lane & 31), c));
#pragma unroll
            for (int i = 0; i < TM; ++i)
                wb[i] = *reinterpret_cast<const half8 *>(
                    base + T::off(T::BN + wm * 32 * TM + 32 * i + (lane & 31), c));
        };
        half8 xa[2][TN], wb[2][TM];
        frags(0, xa[0], wb[0]);
#pragma unroll
        for (int s = 0; s < T::STEPS; ++s) {
            if (s + 1 < T::STEPS) frags(s + 1, xa[(s + 1) & 1], wb[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[s & 1][j], wb[s & 1][i],
                                                                       acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: k-tiles 0 and 1 in flight, wait for 0.  Past the last k-tile the loads
    // are clamped duplicates into a stage nobody reads (no conditional load).
    //
    // The barriers are bare s_barrier: __syncthreads' release fence would wait for every
    // load into LDS in flight (vmcnt(0)), i.e. also for k-tile kt+2.  Each wave waits for
    // its own loads of the next k-tile instead (loads complete in issue order), and its
    // LDS reads of a stage complete before its MFMAs, hence before the barrier after
    // which that stage is refilled.
    dma(a0, 0);
    dma(a1, min(1, nk - 1));
    wait_vm(std::integral_constant<int, T::LOADS>{});
    __builtin_amdgcn_s_barrier();
    // Stage of k-tile kt = kt % 3; step S computes stage S and refills stage (S+2) % 3.
    int kt = 0;
    auto step = [&](const char *cur, uint32_t nxt) {
        dma(nxt, min(kt + 2, nk - 1));
        compute(cur);
        wait_vm(std::integral_constant<int, T::LOADS>{});   // k-tile kt+1 has landed
        __builtin_amdgcn_s_barrier();
        return ++kt < nk;
    };
    while (step(st0, a2) && step(st1, a0) && step(st2, a1)) {
    }
    wait_vm(std::integral_constant<int, 0>{});   // no load may land after the workgroup ends

    const bool full = row0 + T::BM <= out && tok0 + T::BN <= batch;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = row0 + wm * 32 * TM + 32 * i + (lane & 31);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = tok0 + wn * 32 * TN + 32 * j + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (full || (row < out && tok < batch))
                    y[size_t(tok) * out + row] = f2h_bits(acc[i][j][r]);
            }
        }
    }
}

struct PfCfg {
    int tm, tn, tiles_m, tiles_n, per_xcd;
};

// Tile shape: the fewest rounds of workgroups weighted by a tile's MFMA efficiency (a
// 128-row-by-64-token wave tile reads LDS for three quarters of its MFMA time, a
// 64 x 64 one for all of it).  A 128 x 128 wave tile (256 accumulators) does not fit
// the registers beside the staging and fragment registers without spilling.
PfCfg pf_cfg(const Problem &p) {
    struct Opt { int tm, tn; double eff; };
    const Opt opts[2] = {{4, 2, 1.0}, {2, 2, 0.7}};
    PfCfg best{};
    double best_t = 0;
    for (const Opt &o : opts) {
        const int64_t tm = (p.out + 64 * o.tm - 1) / (64 * o.tm);
        const int64_t tn = (p.batch + 64 * o.tn - 1) / (64 * o.tn);
        const int64_t tiles = tm * tn;
        const int64_t rounds = (tiles + 255) / 256;
        const double t = double(rounds) * (64.0 * o.tm) * (64.0 * o.tn) / o.eff;
        if (best_t == 0 || t < best_t) {
            best_t = t;
            best = PfCfg{o.tm, o.tn, int(tm), int(tn), int((tiles + kXcds - 1) / kXcds)};
        }
    }
    return best;
}

size_t w_bytes(const Problem &p) { return (size_t(p.out) * size_t(p.in) * 2 + 255) / 256 * 256; }

template <int TM, int TN, int WM = 2>
hipError_t launch_pf(const Problem &p, const PfCfg &c, const uint16_t *W) {
    constexpr int BK = 64;
    if (p.in % 64 == 0) {
        hipLaunchKernelGGL((prefill_gemm_dma_kernel<TM, TN, WM>), dim3(unsigned(c.per_xcd * kXcds)),
                           dim3(2 * WM * kWave), 0, p.stream, W, static_cast<const uint16_t *>(p.x),
                           static_cast<uint16_t *>(p.y), int(p.out), int(p.in), p.batch,
                           c.tiles_n, c.tiles_m * c.tiles_n, c.per_xcd);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((prefill_gemm_kernel<TM, TN, BK>), dim3(unsigned(c.per_xcd * kXcds)),
                       dim3(kPfThreads), 0, p.stream, W, static_cast<const uint16_t *>(p.x),
                       static_cast<uint16_t *>(p.y), int(p.out), int(p.in), p.batch, c.tiles_n,
                       c.tiles_m * c.tiles_n, c.per_xcd);
    return hipGetLastError();
}

}  // namespace

// Any K and B (the decode is the generic fold) and any in % 8 == 0; x and the codebooks
// are read in 16-byte pieces.
bool prefill_supported(const Problem &p) {
    if (p.out > (int64_t(1) << 30) || p.in > (int64_t(1) << 30) || p.batch < 1) return false;
    if (p.out * p.in > (int64_t(1) << 40)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codebooks) | reinterpret_cast<uintptr_t>(p.x);
    return (a & 15u) == 0;
}

size_t prefill_workspace_bytes(const Problem &p) { return w_bytes(p); }

hipError_t launch_prefill(const Problem &p, void *workspace) {
    uint16_t *W = static_cast<uint16_t *>(workspace);
    hipError_t e = launch_dequant16(p, W);
    if (e != hipSuccess) return e;
    const PfCfg c = pf_cfg(p);
    if (c.tm == 4) return launch_pf<2, 2, 4>(p, c, W);     // 256 x 128: 8 waves of 64 x 64
    return launch_pf<2, 2>(p, c, W);
}

}  // namespace aqlm
