// 16-bit-code GEMV with the codebook split by vector position (gfx950).
//
// The 8-wide dot product of the additive decode (page "AQLM (Additive
// Quantization for LLMs)", section "Niveau intermediaire") splits over its 8
// positions t:
//     y[b][o] = sum_t sum_k sum_j C_k[i_k(o,j)][t] * x[b][8j + t].
// One position of one codebook is a plane of 65536 fp16 values = 128 KiB, which
// fits the LDS of a CU, while the whole 1 MiB codebook does not.  So a workgroup
// owns one plane (k, t) and one range of rows: it streams every code of its rows
// and turns each into a 2-byte LDS read, instead of a 16-byte gather through L2,
// whose request rate caps the plain 16-bit kernel.
//
// * Codebooks are taken pre-packed plane-major, [K][8][65536] fp16
//   (aqlm_pack_codebooks: a one-time layout change of the weights).
// * The K*8 workgroups of one row range get block ids that are equal modulo 8,
//   so the dispatcher puts them on the same XCD: the codes come from HBM once and
//   from that XCD's L2 for the other planes.
// * Each wave walks its rows' 16-byte code chunks with several chunks in flight
//   (a ring of 5..8 loads, issued branch-free); plane values for two codes are
//   packed into one register and multiplied with v_dot2_f32_f16 against the
//   matching activations, which sit in LDS as a plane x[b][8j + t] too.  Rows are
//   summed across lanes several at a time by a transposing butterfly.
// * Per-plane row sums go to a workspace; a second kernel adds the K*8 planes in
//   order and writes fp16 y.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kDsWaves = 16;
constexpr int kEntries = 65536;
constexpr int kXPlaneHalves = 14336;   // batch * in/8 activations of one position
// tokens of the matrix-core form: one 16-token tile (measured on MI355X against unpacking
// and the canonical kernels: 1.3-6x faster at batches 5..8, even at 16, slower from 32)
constexpr int kDsmMaxBatch = 16;

typedef _Float16 hf;

template <int NSEG>
struct DsShape {
    // rows reduced together, and code chunks in flight per lane (a multiple of NSEG)
    static constexpr int RB = NSEG <= 1 ? 8 : NSEG <= 2 ? 4 : NSEG <= 4 ? 2 : 1;
    static constexpr int D = NSEG * RB;
};

template <int K, int NB, int NSEG, int NS>
__global__ void __launch_bounds__(kDsWaves * kWave)
ds_kernel(const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ planes1,
          const uint16_t *__restrict__ x, float *__restrict__ partial, int out1, int in,
          int batch, int nranges, int rows_per_range, const Segs segs) {
    constexpr int P = K * 8;                 // planes
    constexpr int GPC = 8 / K;               // groups per 16-byte chunk
    constexpr int RB = DsShape<NSEG>::RB;
    constexpr int D = DsShape<NSEG>::D;
    __shared__ __attribute__((aligned(16))) hf tab[kEntries];
    __shared__ __attribute__((aligned(16))) hf xs[kXPlaneHalves];

    // block -> (plane, row range); the planes of a range share id % 8, i.e. an XCD
    const int id = blockIdx.x;
    const int grp = id / (P * 8), rem = id - grp * (P * 8);
    const int p = rem >> 3;
    const int rr = grp * 8 + (rem & 7);
    if (rr >= nranges) return;
    const int k = p >> 3, t = p & 7;
    // this range's matrix: the arguments for one matrix (NS == 1), else from segs
    // (ranges of each matrix numbered consecutively, segs.aux0)
    const int mi = seg_of<NS>(segs.n, segs.aux0, rr);
    const int lrr = NS == 1 ? rr : rr - pick(segs.aux0, mi);
    const int out = NS == 1 ? out1 : pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const int T = NS == 1 ? out1 : segs.row0[segs.n];
    const int orow0 = NS == 1 ? 0 : pick(segs.row0, mi);
    const uint8_t *__restrict__ codes =
        NS == 1 ? codes1 : static_cast<const uint8_t *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ planes =
        NS == 1 ? planes1 : static_cast<const uint16_t *>(pick(segs.cb, mi));

    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform values live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = in / kGroup;
    const int NC = G / GPC;                  // chunks per row
    const int r_begin = lrr * rows_per_range;
    const int r_end = min(out, r_begin + rows_per_range);
    const int rpw = (rows_per_range + kDsWaves - 1) / kDsWaves;
    const int w_begin = r_begin + wave * rpw;
    const int w_end = min(r_end, w_begin + rpw);
    const int nitems = max(0, w_end - w_begin) * NSEG;

    // Branch-free loads: the row pointer is wave-uniform (scalar) and each lane adds
    // its chunk offset, clamped into the row; a conditional load would make the
    // compiler wait for it at once.  Clamped lanes and items are masked where the
    // chunk is used.
    const size_t row_bytes = size_t(NC) * 16u;
    const int nrows = max(1, w_end - w_begin);
    uint32_t lane_off[NSEG];
    bool lane_ok[NSEG];
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
        lane_off[sg] = uint32_t(min(lane + kWave * sg, NC - 1)) * 16u;
        lane_ok[sg] = lane + kWave * sg < NC;
    }
    auto load_item = [&](int item, int sg) -> u32x4 {
        const int rowi = min(item / NSEG, nrows - 1);
        const uint8_t *rp = codes + size_t(min(w_begin + rowi, out - 1)) * row_bytes;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rp + lane_off[sg]));
    };

    {
        // 128 KiB plane: every load of a thread issued before its LDS writes.  The
        // plane gates all work, so it goes first; code loads issued with it would
        // compete for the same bandwidth and delay it (about 2.5 us measured).
        const uint4 *src = reinterpret_cast<const uint4 *>(planes + size_t(p) * kEntries);
        uint4 *dst = reinterpret_cast<uint4 *>(tab);
        constexpr int PER = kEntries / 8 / (kDsWaves * kWave);
        uint4 tmp[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) tmp[i] = src[threadIdx.x + i * kDsWaves * kWave];
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[threadIdx.x + i * kDsWaves * kWave] = tmp[i];
        for (int b = 0; b < batch; ++b)
            for (int j = threadIdx.x; j < G; j += blockDim.x)
                xs[b * G + j] = __builtin_bit_cast(hf, x[size_t(b) * in + size_t(j) * kGroup + t]);
    }
    __syncthreads();
    if (nitems == 0) return;

    u32x4 ring[D];
#pragma unroll
    for (int q = 0; q < D; ++q) ring[q] = load_item(q, q % NSEG);

    // at batch 1 each lane's activations (GPC per chunk position) stay in registers
    constexpr bool XREG = NB == 1;
    hf xr[XREG ? NSEG : 1][GPC];
    if constexpr (XREG) {
#pragma unroll
        for (int sg = 0; sg < NSEG; ++sg) {
            const int c = min(lane + kWave * sg, NC - 1);
#pragma unroll
            for (int g = 0; g < GPC; ++g) xr[sg][g] = xs[c * GPC + g];
        }
    }

    for (int base = 0; base < nitems; base += D) {
        float acc[RB][NB];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;
#pragma unroll
        for (int q = 0; q < D; ++q) {
            const int item = base + q;
            const u32x4 cw = ring[q];
            const int r = q / NSEG;                        // compile-time
            const int seg = q % NSEG;
            ring[q] = load_item(item + D, seg);
            const bool ok = item < nitems && lane_ok[seg];
            const int c = min(lane + kWave * seg, NC - 1);
            // plane values of this chunk's codes (codebook k of each group)
            hf v[GPC];
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                // code n = g*K + k of the chunk: word n/2 is g/2 (K = 1) or g (K = 2),
                // known at compile time; only K = 2 selects the half at run time
                uint32_t code;
                if constexpr (K == 1) {
                    const uint32_t w = cw[g >> 1];
                    code = (g & 1) ? (w >> 16) : (w & 0xFFFFu);
                } else {
                    code = (cw[g] >> (16 * k)) & 0xFFFFu;
                }
                v[g] = tab[code];
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (NB == 1 || b < batch) {
                    const hf *xp = xs + b * G + c * GPC;
                    float d = 0.0f;
#pragma unroll
                    for (int g = 0; g < GPC; g += 2) {
                        const half2v a = {v[g], v[g + 1]};
                        half2v xv;
                        if constexpr (XREG) xv = half2v{xr[seg][g], xr[seg][g + 1]};
                        else xv = half2v{xp[g], xp[g + 1]};
                        d = __builtin_amdgcn_fdot2(a, xv, d, false);
                    }
                    acc[r][b] += ok ? d : 0.0f;
                }
            }
        }
        // rows base/NSEG .. +RB-1 of this wave, reduced together
        const int row0 = w_begin + base / NSEG;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (NB == 1 || b < batch) {
                float v[RB];
#pragma unroll
                for (int r = 0; r < RB; ++r) v[r] = acc[r][b];
                const float s = transpose_reduce<RB>(v, lane);
                const int row = row0 + lane / (kWave / RB);
                if ((lane & (kWave / RB - 1)) == 0 && row < w_end)
                    partial[(size_t(p) * batch + b) * T + orow0 + row] = s;
            }
        }
    }
}

// ------------------------------------------------------------------ batch 5 .. 128
// The same position split on the matrix cores.  Workgroups are laid out as for
// ds_kernel (one plane (k, t) x one row range, the planes of a range on one XCD);
// a wave takes 16-row tiles of the range and runs each over the whole input axis
// with v_mfma_f32_16x16x32_f16, 16 tokens per token tile:
// * weight operand (B): lane (row j, k-block kb) holds the plane values of groups
//   32s + 8kb .. +7 of its row: one 16-byte code load (K = 1; two for K = 2) and 8
//   LDS lookups;
// * activation operand (A): the position-t activations of the same 8 groups, one
//   16-byte load from xT[t][token][group], a transposed copy that xt_kernel writes
//   first (the activations are the A operand so that a result register holds 16
//   consecutive weight rows of one token: row-contiguous partial-sum stores);
// * D steps of codes and activations are in flight per lane (a ring, as in
//   ds_kernel);
// * up to 16 tokens (one token tile).  Measured on MI355X the kernel is bound by the
//   L2 request rate of its loads, not by the lookups: the MFMA operand layout puts 16
//   rows in every load instruction, 64 bytes each, for the codes and likewise for the
//   activations.
// Per-plane partial sums go to the workspace and partial_sum adds the K*8 planes.

// xT[t][b][j] = x[b][8j + t]
__global__ void __launch_bounds__(256)
xt_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ xT, int batch, int G) {
    const int64_t n = int64_t(batch) * G;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * 256) {
        // x[b][8j .. 8j+7] with i = b*G + j (in = 8G)
        const uint4 v = *reinterpret_cast<const uint4 *>(x + i * kGroup);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
            xT[int64_t(t) * n + i] = uint16_t(w[t >> 1] >> (16 * (t & 1)));
    }
}

// k-steps of codes and activations in flight per lane (4K + 4NT registers each)
template <int K, int NT> constexpr int dsm_ring() { return K * NT >= 4 ? 3 : 4; }

template <int K, int NT, int NS>
__global__ void __launch_bounds__(kDsWaves * kWave)
dsm_kernel(const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ planes1,
           const uint16_t *__restrict__ xT, float *__restrict__ partial, int out1, int in,
           int batch, int tb, int nranges, int rows_per_range, const Segs segs) {
    // tokens tb .. tb + 16*NT - 1 (a token block; larger batches launch once per block)
    constexpr int P = K * 8;
    constexpr int D = dsm_ring<K, NT>();
    __shared__ __attribute__((aligned(16))) hf tab[kEntries];

    // block -> (plane, row range), as in ds_kernel
    const int id = blockIdx.x;
    const int grp = id / (P * 8), rem = id - grp * (P * 8);
    const int p = rem >> 3;
    const int rr = grp * 8 + (rem & 7);
    if (rr >= nranges) return;
    const int k = p >> 3, t = p & 7;
    const int mi = seg_of<NS>(segs.n, segs.aux0, rr);
    const int lrr = NS == 1 ? rr : rr - pick(segs.aux0, mi);
    const int out = NS == 1 ? out1 : pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const int T = NS == 1 ? out1 : segs.row0[segs.n];
    const int orow0 = NS == 1 ? 0 : pick(segs.row0, mi);
    const uint8_t *__restrict__ codes =
        NS == 1 ? codes1 : static_cast<const uint8_t *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ planes =
        NS == 1 ? planes1 : static_cast<const uint16_t *>(pick(segs.cb, mi));

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = in / kGroup;
    const int r_begin = lrr * rows_per_range;
    const int r_end = min(out, r_begin + rows_per_range);

    {
        // 128 KiB plane: every load of a thread issued before its LDS writes
        const uint4 *src = reinterpret_cast<const uint4 *>(planes + size_t(p) * kEntries);
        uint4 *dst = reinterpret_cast<uint4 *>(tab);
        constexpr int PER = kEntries / 8 / (kDsWaves * kWave);
        uint4 tmp[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) tmp[i] = src[threadIdx.x + i * kDsWaves * kWave];
#pragma unroll
        for (int i = 0; i < PER; ++i) dst[threadIdx.x + i * kDsWaves * kWave] = tmp[i];
    }
    __syncthreads();

    const int ntiles = (r_end - r_begin + 15) / 16;   // <= 0: nothing to do
    const int nsteps = (G + 31) / 32;
    const int i16 = lane & 15, kb = lane >> 4;
    const uint16_t *xp = xT + size_t(t) * batch * G;  // plane t: [batch][G]
    const size_t row_bytes = size_t(G) * K * 2;

    // (one token block per launch: a loop over blocks here would let the compiler hoist
    // the loads that do not depend on it, and change the ring's load order, see below)
    for (int tile = wave; tile < ntiles; tile += kDsWaves) {
        const int row = min(r_begin + tile * 16 + i16, r_end - 1);  // past the end: not stored
        const uint8_t *crow = codes + size_t(row) * row_bytes;
        // the activation loads do not depend on the tile: an opaque zero in their
        // address keeps them in this loop, in the ring's order (hoisted out of it,
        // every wait in the k-step loop would become a wait for most of the ring)
        int tz = tile;
        asm volatile("" : "+s"(tz));
        const uint16_t *xq = xp + (tz - tile);
        {
            // codes and activations of k-step s (clamped into the row: always in bounds)
            auto load = [&](int s, u32x4 (&cw)[K], half8 (&xa)[NT]) {
                const int jb = min(s * 32 + 8 * kb, G - 8);
#pragma unroll
                for (int kk = 0; kk < K; ++kk)
                    cw[kk] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(crow + size_t(jb) * K * 2) + kk);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int tok = min(tb + nt * 16 + i16, batch - 1);
                    xa[nt] = *reinterpret_cast<const half8 *>(xq + size_t(tok) * G + jb);
                }
            };
            u32x4 rc[D][K];
            half8 rx[D][NT];
            // issued slot by slot in the loop's own order (codes, then activations):
            // the waits in the loop are counted against this order too, so a reordered
            // prologue would make every wait there a wait for the whole ring
#pragma unroll
            for (int q = 0; q < D; ++q) {
                load(q, rc[q], rx[q]);
                __builtin_amdgcn_sched_barrier(0);
            }
            float4v acc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = float4v{};
            for (int base = 0; base < nsteps; base += D) {
#pragma unroll
                for (int q = 0; q < D; ++q) {
                    const int s = base + q;
                    const u32x4 (&cw)[K] = rc[q];
                    const half8 (&xa)[NT] = rx[q];
                    // groups past the row (a clamped block, or a step past the last) add
                    // nothing: both operands are zeroed (an AND with an opaque mask, so
                    // that the loads are not turned into branches)
                    uint32_t msk = s * 32 + 8 * kb < G ? 0xFFFFFFFFu : 0u;
                    asm volatile("" : "+v"(msk));
                    half8 w;
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        uint32_t code;
                        if constexpr (K == 1) {
                            const uint32_t v = cw[0][g >> 1];
                            code = (g & 1) ? (v >> 16) : (v & 0xFFFFu);
                        } else {
                            // 32 bytes: group g's two codes are word g (codebook k in half k)
                            code = (cw[g >> 2][g & 3] >> (16 * k)) & 0xFFFFu;
                        }
                        w[g] = tab[code];
                    }
                    u32x4 wb = __builtin_bit_cast(u32x4, w);
                    wb &= msk;
                    w = __builtin_bit_cast(half8, wb);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        u32x4 xb = __builtin_bit_cast(u32x4, xa[nt]);
                        xb &= msk;
                        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(half8, xb), w, acc[nt], 0, 0, 0);
                    }
                    // the slot is consumed: refill it D steps ahead (loaded in place,
                    // so the ring needs no register copies)
                    __builtin_amdgcn_sched_barrier(0);
                    load(s + D, rc[q], rx[q]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // result lane l, register r: token 4(l/16) + r of the token tile, row l % 16
            const int rowo = r_begin + tile * 16 + i16;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = tb + nt * 16 + 4 * kb + r;
                    if (tok < batch && rowo < r_end)
                        partial[(size_t(p) * batch + tok) * T + orow0 + rowo] = acc[nt][r];
                }
        }
    }
}

// planes[k][t][c] = codebooks[k][c][t]
__global__ void __launch_bounds__(256)
pack_kernel(const uint16_t *__restrict__ cb, uint16_t *__restrict__ planes, int K, int entries) {
    const int64_t n = int64_t(K) * entries;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t kk = i / entries, c = i - kk * entries;
#pragma unroll
        for (int t = 0; t < 8; ++t) planes[(kk * 8 + t) * entries + c] = cb[i * 8 + t];
    }
}

// codebooks[k][c][t] = planes[k][t][c]
__global__ void __launch_bounds__(256)
unpack_kernel(const uint16_t *__restrict__ planes, uint16_t *__restrict__ cb, int K, int entries) {
    const int64_t n = int64_t(K) * entries;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t kk = i / entries, c = i - kk * entries;
#pragma unroll
        for (int t = 0; t < 8; ++t) cb[i * 8 + t] = planes[(kk * 8 + t) * entries + c];
    }
}

struct DsCfg {
    int nseg, nranges, nranges_padded, rows_per_range, grid;
};

// Row ranges of rows_per_range rows, about max(8, 256 / planes) of them over all matrices
// (one workgroup per CU); each matrix gets whole ranges of its own (segs.aux0).
DsCfg ds_cfg(const Problem &p, Segs *segs = nullptr) {
    DsCfg c{};
    const int P = p.K * 8;
    const int64_t G = p.in / kGroup;
    const int64_t NC = G / (8 / p.K);
    c.nseg = int((NC + kWave - 1) / kWave);
    int nr = 256 / P;                           // one workgroup per CU
    if (nr < 8) nr = 8;
    if (nr > p.out) nr = int(p.out);
    // each matrix of a grouped call gets whole ranges of its own; they may not outnumber
    // nr (one workgroup fills a CU's LDS), so the range grows until they fit
    int64_t rpr = (p.out + nr - 1) / nr;
    auto ranges = [&](int64_t r) {
        int64_t t = 0;
        for (int m = 0; m < p.segs.n; ++m) t += (p.segs.row0[m + 1] - p.segs.row0[m] + r - 1) / r;
        return t;
    };
    while (ranges(rpr) > nr) ++rpr;
    c.rows_per_range = int(rpr);
    int total = 0;
    for (int m = 0; m < p.segs.n; ++m) {
        if (segs) segs->aux0[m] = total;
        total += (p.segs.row0[m + 1] - p.segs.row0[m] + c.rows_per_range - 1) / c.rows_per_range;
    }
    if (segs) segs->aux0[p.segs.n] = total;
    c.nranges = total;
    c.nranges_padded = (c.nranges + 7) / 8 * 8;
    c.grid = P * c.nranges_padded;
    return c;
}

template <int K, int NB, int NSEG>
hipError_t launch3(const Problem &p, const DsCfg &c, const Segs &segs, float *partial) {
    const dim3 g(c.grid), b(kDsWaves * kWave);
    const uint16_t *x = static_cast<const uint16_t *>(p.x);
    const uint8_t *codes = static_cast<const uint8_t *>(segs.codes[0]);
    const uint16_t *planes = static_cast<const uint16_t *>(segs.cb[0]);
    const int out = segs.row0[1];
    if (segs.n == 1)
        hipLaunchKernelGGL((ds_kernel<K, NB, NSEG, 1>), g, b, 0, p.stream, codes, planes, x,
                           partial, out, int(p.in), p.batch, c.nranges, c.rows_per_range, segs);
    else
        hipLaunchKernelGGL((ds_kernel<K, NB, NSEG, kMaxSegs>), g, b, 0, p.stream, codes, planes,
                           x, partial, out, int(p.in), p.batch, c.nranges, c.rows_per_range,
                           segs);
    return hipGetLastError();
}

template <int K, int NB>
hipError_t launch2(const Problem &p, const DsCfg &c, const Segs &segs, float *partial) {
    switch (c.nseg) {
        case 1: return launch3<K, NB, 1>(p, c, segs, partial);
        case 2: return launch3<K, NB, 2>(p, c, segs, partial);
        case 3: return launch3<K, NB, 3>(p, c, segs, partial);
        case 4: return launch3<K, NB, 4>(p, c, segs, partial);
        case 5: return launch3<K, NB, 5>(p, c, segs, partial);
        case 6: return launch3<K, NB, 6>(p, c, segs, partial);
        case 7: return launch3<K, NB, 7>(p, c, segs, partial);
        default: return launch3<K, NB, 8>(p, c, segs, partial);
    }
}

template <int K>
hipError_t launch1(const Problem &p, const DsCfg &c, const Segs &segs, float *partial) {
    if (p.batch <= 1) return launch2<K, 1>(p, c, segs, partial);
    if (p.batch <= 2) return launch2<K, 2>(p, c, segs, partial);
    return launch2<K, 4>(p, c, segs, partial);
}

template <int K, int NT>
hipError_t launch_m2(const Problem &p, const DsCfg &c, const Segs &segs, const uint16_t *xT,
                     float *partial) {
    const dim3 g(c.grid), b(kDsWaves * kWave);
    const uint8_t *codes = static_cast<const uint8_t *>(segs.codes[0]);
    const uint16_t *planes = static_cast<const uint16_t *>(segs.cb[0]);
    const int out = segs.row0[1];
    for (int tb = 0; tb < p.batch; tb += 16 * NT) {
        if (segs.n == 1)
            hipLaunchKernelGGL((dsm_kernel<K, NT, 1>), g, b, 0, p.stream, codes, planes, xT,
                               partial, out, int(p.in), p.batch, tb, c.nranges, c.rows_per_range,
                               segs);
        else
            hipLaunchKernelGGL((dsm_kernel<K, NT, kMaxSegs>), g, b, 0, p.stream, codes, planes,
                               xT, partial, out, int(p.in), p.batch, tb, c.nranges,
                               c.rows_per_range, segs);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int K>
hipError_t launch_m1(const Problem &p, const DsCfg &c, const Segs &segs, const uint16_t *xT,
                     float *partial) {
    return launch_m2<K, 1>(p, c, segs, xT, partial);
}

}  // namespace

bool dsm_supported(const Problem &p) {
    if (p.B != 16 || (p.K != 1 && p.K != 2)) return false;
    // two codebooks double the lookups per weight: past batch 8 the canonical kernels win
    if (p.batch < 1 || p.batch > (p.K == 1 ? kDsmMaxBatch : 8)) return false;
    const int64_t G = p.in / kGroup;
    if (G % 8) return false;
    if (p.out > (1 << 28) || int64_t(p.batch) * p.in > (int64_t(1) << 31)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks) |
                        reinterpret_cast<uintptr_t>(p.x);
    return (a & 15u) == 0;
}

// workspace: [K*8][batch][T] fp32 partial sums, then xT [8][batch][G] fp16 (256-byte aligned)
static size_t dsm_partial_bytes(const Problem &p) {
    return (size_t(p.K) * 8 * size_t(p.batch) * size_t(p.out) * sizeof(float) + 255) / 256 * 256;
}

size_t dsm_workspace_bytes(const Problem &p) {
    return dsm_partial_bytes(p) + size_t(p.batch) * size_t(p.in) * 2;
}

hipError_t launch_dsm(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const DsCfg c = ds_cfg(p, &segs);
    float *partial = static_cast<float *>(workspace);
    uint16_t *xT = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) + dsm_partial_bytes(p));
    const int G = int(p.in / kGroup);
    const int64_t n = int64_t(p.batch) * G;
    const int blocks = int((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(xt_kernel, dim3(blocks), dim3(256), 0, p.stream,
                       static_cast<const uint16_t *>(p.x), xT, p.batch, G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = p.K == 1 ? launch_m1<1>(p, c, segs, xT, partial) : launch_m1<2>(p, c, segs, xT, partial);
    if (e != hipSuccess) return e;
    return launch_partial_sum_segs(partial, segs, p.batch, p.K * 8, p.stream);
}

bool ds_supported(const Problem &p) {
    if (p.B != 16 || (p.K != 1 && p.K != 2)) return false;
    if (p.batch < 1 || p.batch > 4) return false;
    const int64_t G = p.in / kGroup;
    if (G % (8 / p.K)) return false;
    if (int64_t(p.batch) * G > kXPlaneHalves) return false;
    const int64_t NC = G / (8 / p.K);
    if ((NC + kWave - 1) / kWave > 8) return false;
    if (p.out > (1 << 28)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks);
    return (a & 15u) == 0;
}

size_t ds_workspace_bytes(const Problem &p) {
    return size_t(p.K) * 8 * size_t(p.batch) * size_t(p.out) * sizeof(float);
}

// segs.cb holds the packed planes [K][8][65536]; workspace: K*8 x batch x T fp32
hipError_t launch_ds(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const DsCfg c = ds_cfg(p, &segs);
    float *partial = static_cast<float *>(workspace);
    hipError_t e = p.K == 1 ? launch1<1>(p, c, segs, partial) : launch1<2>(p, c, segs, partial);
    if (e != hipSuccess) return e;
    return launch_partial_sum_segs(partial, segs, p.batch, p.K * 8, p.stream);
}

hipError_t launch_pack_codebooks(const void *cb, void *planes, int K, int B, hipStream_t s) {
    const int entries = 1 << B;
    const int64_t n = int64_t(K) * entries;
    const int blocks = int((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t *>(cb), static_cast<uint16_t *>(planes), K,
                       entries);
    return hipGetLastError();
}

hipError_t launch_unpack_codebooks(const void *planes, void *cb, int K, int B, hipStream_t s) {
    const int entries = 1 << B;
    const int64_t n = int64_t(K) * entries;
    const int blocks = int((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t *>(planes), static_cast<uint16_t *>(cb), K,
                       entries);
    return hipGetLastError();
}

}  // namespace aqlm
