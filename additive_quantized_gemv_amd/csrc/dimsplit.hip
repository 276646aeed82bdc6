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

}  // namespace

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
