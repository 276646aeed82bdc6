// 2x8 GEMV at batch 1 through per-group lookup tables (gfx950).
//
// By distributivity of the additive decode (page "AQLM (Additive Quantization
// for LLMs)", section "Niveau intermediaire"),
//     y[o] = sum_j ( L_0[j][i_0(o,j)] + L_1[j][i_1(o,j)] ),   L_k[j][c] = C_k[c] . x[8j .. 8j+7],
// so after building the tables each group-row costs two 4-byte LDS reads and
// two adds instead of two 16-byte gathers and eight dot2s.
//
// * The input axis is cut into slices of 64 groups (512 inputs).  A workgroup
//   owns one slice and a range of rows.  Its tables, 2 x 256 x 64 fp32 =
//   128 KiB, fill the LDS; they are built with v_mfma_f32_32x32x8_f16 as the
//   product [512 codebook entries x 8] . [8 x 64 groups].
// * LDS layout: entry (k, c, group jl) at byte (k*256 + c)*256 + jl*4.  Lane jl
//   of a wave always looks up group jl, so the 64 lanes of one ds_read_b32 hit
//   64 distinct banks whatever the codes are (no bank conflicts).  The byte
//   address is assembled from the code bytes with one v_perm_b32.
// * Each wave takes 16 rows at a time (one 2-byte code load per lane per row),
//   then reduces the 16 row partials across the 64 lanes with a transposing
//   butterfly (permlane32/permlane16 swaps, then DPP), ~2 ops per row.
// * Slice partials go to a workspace; a second small kernel sums them in slice
//   order and writes fp16 y (deterministic).  The kernel boundary is what makes
//   partials written on one XCD visible to another.  An in-kernel handoff (last
//   workgroup of a row range sums the slices) needs an agent-scope release fence
//   per workgroup, i.e. an L2 write-back; measured on MI355X that single-kernel
//   form took 24 us per 11008x4096 product against 7 + 4 us for the two kernels.
//   A form without the fence (partials written with write-through agent-scope
//   atomic stores, an arrival counter per row block, the last workgroup summing
//   with coherent loads) is correct but slower too: 10.0 against 8.6 us per call
//   for 4096x11008, the store round trip plus the re-read costing more than the
//   second launch from a graph.
// * Every code load of a wave (up to 32 rows) is issued before the tables are
//   built, so each wave waits for HBM once.
// * Packed variant (aqlm_pack_codes): the codes of a slice are stored as tiles
//   of 8 rows x 64 groups, lane jl's 16 bytes holding the 8 rows' code pairs of
//   group jl.  A wave then reads 1 KiB contiguous per load (instead of one
//   128-byte row segment per load, half of which straddle two cache lines when
//   rows are not 128-byte multiples), with one load and address per 8 rows.
//   The group padding of the last slice holds code 0 and meets zero
//   activations, so it adds nothing.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kSlice = 64;              // groups per slice (= lanes)
constexpr int kLutWaves = 16;           // 1024 threads
constexpr int kReduceRows = 16;         // rows reduced together by the butterfly
constexpr int kRowsPerWave = 32;        // rows of one wave (all loaded up front)
constexpr int kLutBytes = 2 * 256 * kSlice * 4;

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lds_f32(const char *base, uint32_t byte_addr) {
    return *reinterpret_cast<const float *>(base + byte_addr);
}

// Operands of the table build.  Wave w computes entries 32w .. 32w+31 for both
// 32-group halves of the slice with v_mfma_f32_32x32x8_f16: lane l supplies
// positions 4(l/32) .. 4(l/32)+3 of entry 32w + l%32 (A) and of the activations
// of group j0 + 32h + l%32 (B, h = 0, 1), zero past the last group.
// PLANAR: codebooks in the plane-major layout [K][8][256] of aqlm_pack_codebooks.
template <bool PLANAR>
__device__ __forceinline__ void load_build_operands(const uint16_t *__restrict__ cb,
                                                    const uint16_t *__restrict__ x, int j0, int G,
                                                    int wave, int lane, half4 &a, half4 (&bx)[2]) {
    const int e = wave * 32 + (lane & 31);
    const int kq = (lane >> 5) * 4;
    if constexpr (PLANAR) {
        const int k = e >> 8, c = e & 255;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = __builtin_bit_cast(_Float16, cb[(k * 8 + kq + i) * 256 + c]);
    } else {
        a = *reinterpret_cast<const half4 *>(cb + size_t(e) * kGroup + kq);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int j = min(j0 + nb * 32 + (lane & 31), G - 1);
        bx[nb] = *reinterpret_cast<const half4 *>(x + size_t(j) * kGroup + kq);
        if (j0 + nb * 32 + (lane & 31) >= G) bx[nb] = half4{0, 0, 0, 0};
    }
}

// L[e][jl] -> LDS byte (e * 64 + jl) * 4; result lane l, register r holds entry
// 32w + 8(r/4) + 4(l/32) + r%4 of group 32h + l%32.
__device__ __forceinline__ void store_tables(char *lut, const half4 &a, const half4 (&bx)[2],
                                             int wave, int lane) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        float16v d = {};
        d = __builtin_amdgcn_mfma_f32_32x32x8f16(a, bx[nb], d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int n = nb * 32 + (lane & 31);
            *reinterpret_cast<float *>(lut + (wave * 32 + m) * 256 + n * 4) = d[r];
        }
    }
}

// Row blocks of each matrix are numbered consecutively (segs.aux0); a workgroup works
// on one matrix, whose rows it indexes locally; partial sums go to global row
// segs.row0[m] + local row of a [slice][T] workspace.
template <int NS>
__global__ void __launch_bounds__(kLutWaves * kWave)
lut_kernel(const uint16_t *__restrict__ x, float *__restrict__ partial, int G,
           int rows_per_block, int nslices, const Segs segs) {
    __shared__ __attribute__((aligned(16))) char lut[kLutBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slice = blockIdx.x % nslices;
    const int rb = blockIdx.x / nslices;
    const int mi = seg_of<NS>(segs.n, segs.aux0, rb);
    const int rblock = rb - pick(segs.aux0, mi);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const uint16_t *__restrict__ codes = static_cast<const uint16_t *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ cb = static_cast<const uint16_t *>(pick(segs.cb, mi));
    float *__restrict__ part = partial + size_t(slice) * seg_total<NS>(segs.n, segs.row0) + pick(segs.row0, mi);
    const int j0 = slice * kSlice;
    const int jl = lane;
    const int r_begin = rblock * rows_per_block;
    const int r_end = min(out, r_begin + rows_per_block);
    // this wave's rows: a contiguous run of rows_per_block / kLutWaves (<= kRowsPerWave)
    const int rpw = rows_per_block / kLutWaves;
    const int w_begin = r_begin + wave * rpw;
    const int w_rows = max(0, min(rpw, r_end - w_begin));

    // ---- build L[e][jl] = C[e] . x_{j0+jl} for the 512 entries e = k*256 + c.
    // Its (L2-resident) operands are loaded before the code stream: loads complete
    // in issue order, so the tables are built while the codes are still in flight.
    half4 a, bx[2];
    load_build_operands<false>(cb, x, j0, G, wave, lane, a, bx);

    // then every code load of this wave (up to 32 rows): the wave waits for HBM once
    uint32_t code[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int row = min(w_begin + min(r, max(w_rows - 1, 0)), out - 1);
        code[r] = uint32_t(__builtin_nontemporal_load(codes + size_t(row) * G + min(j0 + jl, G - 1)));
    }

    store_tables(lut, a, bx, wave, lane);
    __syncthreads();

    // byte-address template: byte0 = 4*jl, byte2 = 1 selects the second table half
    const uint32_t lanebase = (uint32_t(jl) << 2) | (1u << 16);
#pragma unroll
    for (int h = 0; h < kRowsPerWave / kReduceRows; ++h) {
        if (h * kReduceRows >= w_rows) break;
        float v[kReduceRows];
#pragma unroll
        for (int r = 0; r < kReduceRows; ++r) {
            // addr0 = [4jl, i0, 0, 0], addr1 = [4jl, i1, 1, 0]
            const uint32_t c = code[h * kReduceRows + r];
            const uint32_t a0 = __builtin_amdgcn_perm(lanebase, c, 0x0C0C0004u);
            const uint32_t a1 = __builtin_amdgcn_perm(lanebase, c, 0x0C060104u);
            v[r] = lds_f32(lut, a0) + lds_f32(lut, a1);
        }
        const float s = transpose_reduce<kReduceRows>(v, lane);
        const int r = h * kReduceRows + (lane >> 2);
        if ((lane & 3) == 0 && r < w_rows) part[w_begin + r] = s;
    }
}

// Same product from packed codes: tile (slice s, row octet q) is 64 lanes x 16 B at
// byte ((s * NQ + q) * 64 + jl) * 16, NQ = ceil(out / 8); bytes 2r, 2r+1 of lane
// jl's 16 B are the two codes of row 8q + r, group 64s + jl.  Codebooks are the
// plane-major packed ones.  A workgroup's row range starts on an octet; wave w
// takes the range's octets w, w + 16, w + 32, w + 48.
constexpr int kOctetsPerWave = kRowsPerWave / 8;
constexpr int kOctetsPerPass = kOctetsPerWave * kLutWaves;   // 64 octets = 512 rows
constexpr int kMaxPasses = 8;

template <int NS>
__global__ void __launch_bounds__(kLutWaves * kWave)
lut_packed_kernel(const uint16_t *__restrict__ x, float *__restrict__ partial,
                  int G, int rows_per_block, int nslices, const Segs segs) {
    __shared__ __attribute__((aligned(16))) char lut[kLutBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = blockIdx.x % nslices;
    const int rb = blockIdx.x / nslices;
    const int mi = seg_of<NS>(segs.n, segs.aux0, rb);
    const int rblock = rb - pick(segs.aux0, mi);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const u32x4 *__restrict__ pcodes = static_cast<const u32x4 *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ planes = static_cast<const uint16_t *>(pick(segs.cb, mi));
    float *__restrict__ part = partial + size_t(slice) * seg_total<NS>(segs.n, segs.row0) + pick(segs.row0, mi);
    const int j0 = slice * kSlice;
    const int NQ = (out + 7) / 8;
    const int r_begin = rblock * rows_per_block;             // a multiple of 8
    const int r_end = min(out, r_begin + rows_per_block);
    const int nq = (r_end - r_begin + 7) / 8;                 // >= 1

    half4 a, bx[2];
    load_build_operands<true>(planes, x, j0, G, wave, lane, a, bx);

    // all code tiles of this wave (clamped into the range: always in bounds)
    const u32x4 *tile = pcodes + (size_t(slice) * NQ + r_begin / 8) * kWave + lane;
    u32x4 code[kOctetsPerWave];
#pragma unroll
    for (int i = 0; i < kOctetsPerWave; ++i)
        code[i] = __builtin_nontemporal_load(tile + size_t(min(wave + kLutWaves * i, nq - 1)) * kWave);

    store_tables(lut, a, bx, wave, lane);
    __syncthreads();

    const uint32_t lanebase = (uint32_t(lane) << 2) | (1u << 16);
#pragma unroll
    for (int i = 0; i < kOctetsPerWave; i += 2) {
        if (wave + kLutWaves * i >= nq) break;               // wave-uniform
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // row r % 8 of octet i + r / 8: halfword r % 8 of the tile
            const uint32_t w = code[i + r / 8][(r & 7) >> 1];
            const bool hi = r & 1;
            const uint32_t a0 = __builtin_amdgcn_perm(lanebase, w, hi ? 0x0C0C0204u : 0x0C0C0004u);
            const uint32_t a1 = __builtin_amdgcn_perm(lanebase, w, hi ? 0x0C060304u : 0x0C060104u);
            v[r] = lds_f32(lut, a0) + lds_f32(lut, a1);
        }
        const float sum = transpose_reduce<16>(v, lane);
        const int vi = lane >> 2;                            // value index: octet i + vi/8, row vi%8
        const int q = wave + kLutWaves * (i + (vi >> 3));
        const int row = r_begin + 8 * q + (vi & 7);
        if ((lane & 3) == 0 && q < nq && row < r_end) part[row] = sum;
    }
}

// The same for row blocks of more than 512 rows: the block is walked in passes of 64
// octets (wave w takes octets 64p + w + 16i), the tables built once and the next
// pass's code tiles loaded while a pass is looked up (two register buffers, loads
// from clamped octets, so none is conditional).  With 512-row blocks a large product
// needs several rounds of workgroups, each building its tables again.
template <int NS>
__global__ void __launch_bounds__(kLutWaves * kWave)
lut_packed_mp_kernel(const uint16_t *__restrict__ x, float *__restrict__ partial,
                     int G, int rows_per_block, int nslices, const Segs segs) {
    __shared__ __attribute__((aligned(16))) char lut[kLutBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int slice = blockIdx.x % nslices;
    const int rb = blockIdx.x / nslices;
    const int mi = seg_of<NS>(segs.n, segs.aux0, rb);
    const int rblock = rb - pick(segs.aux0, mi);
    const int out = pick(segs.row0, mi + 1) - pick(segs.row0, mi);
    const u32x4 *__restrict__ pcodes = static_cast<const u32x4 *>(pick(segs.codes, mi));
    const uint16_t *__restrict__ planes = static_cast<const uint16_t *>(pick(segs.cb, mi));
    float *__restrict__ part = partial + size_t(slice) * seg_total<NS>(segs.n, segs.row0) + pick(segs.row0, mi);
    const int j0 = slice * kSlice;
    const int NQ = (out + 7) / 8;
    const int r_begin = rblock * rows_per_block;             // a multiple of 8
    const int r_end = min(out, r_begin + rows_per_block);
    const int nq = (r_end - r_begin + 7) / 8;                 // >= 1
    const int npass = (nq + kOctetsPerPass - 1) / kOctetsPerPass;

    half4 a, bx[2];
    load_build_operands<true>(planes, x, j0, G, wave, lane, a, bx);

    const u32x4 *tile = pcodes + (size_t(slice) * NQ + r_begin / 8) * kWave + lane;
    auto load_pass = [&](u32x4 (&code)[kOctetsPerWave], int pass) {
#pragma unroll
        for (int i = 0; i < kOctetsPerWave; ++i)
            code[i] = __builtin_nontemporal_load(
                tile + size_t(min(pass * kOctetsPerPass + wave + kLutWaves * i, nq - 1)) * kWave);
    };
    const uint32_t lanebase = (uint32_t(lane) << 2) | (1u << 16);
    auto look_up = [&](const u32x4 (&code)[kOctetsPerWave], int pass) {
#pragma unroll
        for (int i = 0; i < kOctetsPerWave; i += 2) {
            const int q0 = pass * kOctetsPerPass + wave + kLutWaves * i;
            if (q0 >= nq) break;                                 // wave-uniform
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t w = code[i + r / 8][(r & 7) >> 1];
                const bool hi = r & 1;
                const uint32_t a0 = __builtin_amdgcn_perm(lanebase, w, hi ? 0x0C0C0204u : 0x0C0C0004u);
                const uint32_t a1 = __builtin_amdgcn_perm(lanebase, w, hi ? 0x0C060304u : 0x0C060104u);
                v[r] = lds_f32(lut, a0) + lds_f32(lut, a1);
            }
            const float sum = transpose_reduce<16>(v, lane);
            const int vi = lane >> 2;
            const int q = q0 + kLutWaves * (vi >> 3);
            const int row = r_begin + 8 * q + (vi & 7);
            if ((lane & 3) == 0 && q < nq && row < r_end) part[row] = sum;
        }
    };

    u32x4 code[kOctetsPerWave], code2[kOctetsPerWave];
    load_pass(code, 0);
    store_tables(lut, a, bx, wave, lane);
    __syncthreads();
    for (int pass = 0; pass < npass; pass += 2) {
        load_pass(code2, pass + 1);
        look_up(code, pass);
        load_pass(code, pass + 2);
        if (pass + 1 < npass) look_up(code2, pass + 1);       // wave-uniform
    }
}

// codes [out][G] (two 8-bit codes per 16-bit word) -> packed tiles; padding is code 0
__global__ void __launch_bounds__(256)
pack_codes_kernel(const uint16_t *__restrict__ codes, uint16_t *__restrict__ packed, int out,
                  int G, int nslices) {
    const int NQ = (out + 7) / 8;
    const int64_t lanes = int64_t(nslices) * NQ * kWave;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < lanes;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int jl = int(i % kWave);
        const int64_t t = i / kWave;
        const int q = int(t % NQ), s = int(t / NQ);
        const int j = s * kSlice + jl;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = 8 * q + r;
            packed[i * 8 + r] = (row < out && j < G) ? codes[size_t(row) * G + j] : uint16_t(0);
        }
    }
}

// packed tiles -> codes [out][G]: thread i reads tile lane i (16 bytes: the code pairs of
// 8 rows for one group) and writes them to the 8 rows; consecutive threads hold
// consecutive groups, so every read is contiguous and each row's writes coalesce
__global__ void __launch_bounds__(256)
unpack_codes_kernel(const uint16_t *__restrict__ packed, uint16_t *__restrict__ codes, int out,
                    int G, int nslices) {
    const int NQ = (out + 7) / 8;
    const int64_t lanes = int64_t(nslices) * NQ * kWave;
    const uint4 *__restrict__ tiles = reinterpret_cast<const uint4 *>(packed);
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < lanes;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int jl = int(i % kWave);
        const int64_t t = i / kWave;
        const int q = int(t % NQ), s = int(t / NQ);
        const int j = s * kSlice + jl;
        if (j >= G) continue;                    // padding groups of the last slice
        const uint4 v = tiles[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int row = 8 * q + r;
            if (row < out) codes[size_t(row) * G + j] = uint16_t(w[r >> 1] >> (16 * (r & 1)));
        }
    }
}

struct LutCfg {
    int nslices, nrblocks, rows_per_block;
};

// Row blocks of at most kLutWaves * kRowsPerWave rows (a wave's rows are all loaded at
// once), about 256 / nslices of them over all matrices (one workgroup per CU); each
// matrix gets whole blocks of its own (segs.aux0 is filled here).
LutCfg lut_cfg(const Problem &p, bool packed, Segs *segs = nullptr) {
    LutCfg c{};
    const int64_t G = p.in / kGroup;
    c.nslices = int((G + kSlice - 1) / kSlice);
    const int64_t max_rows = int64_t(kLutWaves) * kRowsPerWave;
    int64_t nrb = c.nslices >= 256 ? 1 : 256 / c.nslices;
    const int64_t most = max_rows * (packed ? kMaxPasses : 1);   // rows per block at most
    const int64_t need = (p.out + most - 1) / most;
    if (nrb < need) nrb = need;
    int64_t rpb = (p.out + nrb - 1) / nrb;
    if (packed) rpb = (rpb + 7) / 8 * 8;                      // ranges start on an octet
    else rpb = (rpb + kLutWaves - 1) / kLutWaves * kLutWaves; // whole rows per wave
    if (rpb < kLutWaves) rpb = kLutWaves;
    // packed codes: up to kMaxPasses passes of 512 rows per block (one round of workgroups)
    const int64_t cap = packed ? max_rows * kMaxPasses : max_rows;
    if (rpb > cap) rpb = cap;
    // Each matrix of a grouped call gets whole blocks of its own; the blocks may not
    // outnumber nrb (a workgroup fills a CU's LDS: one more block column would run in
    // a second round), so the block grows until they fit.
    const int64_t unit = packed ? 8 : kLutWaves;
    auto blocks = [&](int64_t r) {
        int64_t t = 0;
        for (int m = 0; m < p.segs.n; ++m) t += (p.segs.row0[m + 1] - p.segs.row0[m] + r - 1) / r;
        return t;
    };
    while (blocks(rpb) > nrb && rpb + unit <= cap) rpb += unit;
    c.rows_per_block = int(rpb);
    int64_t total = 0;
    for (int m = 0; m < p.segs.n; ++m) {
        if (segs) segs->aux0[m] = int(total);
        total += (p.segs.row0[m + 1] - p.segs.row0[m] + rpb - 1) / rpb;
    }
    if (segs) segs->aux0[p.segs.n] = int(total);
    c.nrblocks = int(total);
    return c;
}

}  // namespace

bool lut_supported(const Problem &p) {
    if (p.K != 2 || p.B != 8 || p.batch != 1) return false;
    if (p.out > (1 << 30) || p.in > (1 << 30)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks) |
                        reinterpret_cast<uintptr_t>(p.x);
    return (a & 7u) == 0;
}

size_t lut_workspace_bytes(const Problem &p) {
    const LutCfg c = lut_cfg(p, false);
    return size_t(c.nslices) * size_t(p.out) * sizeof(float);
}

// workspace: partial sums, nslices x T fp32 (no initial contents needed)
hipError_t launch_lut(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const LutCfg c = lut_cfg(p, false, &segs);
    float *partial = static_cast<float *>(workspace);
    if (segs.n == 1)
        hipLaunchKernelGGL(lut_kernel<1>, dim3(c.nslices * c.nrblocks), dim3(kLutWaves * kWave), 0,
                           p.stream, static_cast<const uint16_t *>(p.x), partial,
                           int(p.in / kGroup), c.rows_per_block, c.nslices, segs);
    else
        hipLaunchKernelGGL(lut_kernel<kMaxSegs>, dim3(c.nslices * c.nrblocks),
                           dim3(kLutWaves * kWave), 0, p.stream,
                           static_cast<const uint16_t *>(p.x), partial, int(p.in / kGroup),
                           c.rows_per_block, c.nslices, segs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_partial_sum_segs(partial, segs, 1, c.nslices, p.stream);
}

int64_t lut_packed_codes_bytes(int64_t out, int64_t in) {
    const int64_t G = in / kGroup;
    return (G + kSlice - 1) / kSlice * ((out + 7) / 8) * kWave * 16;
}

bool lut_packed_supported(const Problem &p) {
    if (p.K != 2 || p.B != 8 || p.batch != 1) return false;
    if (p.out > (1 << 30) || p.in > (1 << 30)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks) |
                        reinterpret_cast<uintptr_t>(p.x);
    return (a & 15u) == 0;
}

size_t lut_packed_workspace_bytes(const Problem &p) {
    const LutCfg c = lut_cfg(p, true);
    return size_t(c.nslices) * size_t(p.out) * sizeof(float);
}

// segs.codes: packed tiles; segs.cb: plane-major; workspace: nslices x T fp32
hipError_t launch_lut_packed(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const LutCfg c = lut_cfg(p, true, &segs);
    float *partial = static_cast<float *>(workspace);
    if (c.rows_per_block > kLutWaves * kRowsPerWave) {
        if (segs.n == 1)
            hipLaunchKernelGGL(lut_packed_mp_kernel<1>, dim3(c.nslices * c.nrblocks),
                               dim3(kLutWaves * kWave), 0, p.stream,
                               static_cast<const uint16_t *>(p.x), partial, int(p.in / kGroup),
                               c.rows_per_block, c.nslices, segs);
        else
            hipLaunchKernelGGL(lut_packed_mp_kernel<kMaxSegs>, dim3(c.nslices * c.nrblocks),
                               dim3(kLutWaves * kWave), 0, p.stream,
                               static_cast<const uint16_t *>(p.x), partial, int(p.in / kGroup),
                               c.rows_per_block, c.nslices, segs);
    } else if (segs.n == 1)
        hipLaunchKernelGGL(lut_packed_kernel<1>, dim3(c.nslices * c.nrblocks),
                           dim3(kLutWaves * kWave), 0, p.stream,
                           static_cast<const uint16_t *>(p.x), partial, int(p.in / kGroup),
                           c.rows_per_block, c.nslices, segs);
    else
        hipLaunchKernelGGL(lut_packed_kernel<kMaxSegs>, dim3(c.nslices * c.nrblocks),
                           dim3(kLutWaves * kWave), 0, p.stream,
                           static_cast<const uint16_t *>(p.x), partial, int(p.in / kGroup),
                           c.rows_per_block, c.nslices, segs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_partial_sum_segs(partial, segs, 1, c.nslices, p.stream);
}

// pack: src = codes [out][G] 16-bit words, dst = tiles; unpack: the reverse
hipError_t launch_pack_codes_lut(const void *src, void *dst, int64_t out, int64_t in, bool pack,
                                 hipStream_t s) {
    const int G = int(in / kGroup);
    const int nslices = (G + kSlice - 1) / kSlice;
    const int64_t work = int64_t(nslices) * ((out + 7) / 8) * kWave;   // tile lanes
    const int blocks = int((work + 255) / 256 < 4096 ? (work + 255) / 256 : 4096);
    if (pack)
        hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst),
                           int(out), G, nslices);
    else
        hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst),
                           int(out), G, nslices);
    return hipGetLastError();
}

}  // namespace aqlm
