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
// * Every code load of a wave (up to 32 rows) is issued before the tables are
//   built, so each wave waits for HBM once.
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

__global__ void __launch_bounds__(kLutWaves * kWave)
lut_kernel(const uint16_t *__restrict__ codes, const uint16_t *__restrict__ cb,
           const uint16_t *__restrict__ x, float *__restrict__ partial, int out, int G,
           int rows_per_block, int nslices) {
    __shared__ __attribute__((aligned(16))) char lut[kLutBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slice = blockIdx.x % nslices;
    const int rblock = blockIdx.x / nslices;
    const int j0 = slice * kSlice;
    const int jl = lane;
    const int r_begin = rblock * rows_per_block;
    const int r_end = min(out, r_begin + rows_per_block);
    // this wave's rows: a contiguous run of rows_per_block / kLutWaves (<= kRowsPerWave)
    const int rpw = rows_per_block / kLutWaves;
    const int w_begin = r_begin + wave * rpw;
    const int w_rows = max(0, min(rpw, r_end - w_begin));

    // ---- build L[e][jl] = C[e] . x_{j0+jl} for the 512 entries e = k*256 + c
    // wave w computes entries 32w .. 32w+31 for both 32-group halves of the slice.
    // Its (L2-resident) operands are loaded before the code stream: loads complete
    // in issue order, so the tables are built while the codes are still in flight.
    const int e = wave * 32 + (lane & 31);
    const int kq = (lane >> 5) * 4;              // this lane's 4 of the 8 vector positions
    const half4 a = *reinterpret_cast<const half4 *>(cb + size_t(e) * kGroup + kq);
    half4 bx[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int j = min(j0 + nb * 32 + (lane & 31), G - 1);
        bx[nb] = *reinterpret_cast<const half4 *>(x + size_t(j) * kGroup + kq);
        if (j0 + nb * 32 + (lane & 31) >= G) bx[nb] = half4{0, 0, 0, 0};
    }

    // then every code load of this wave (up to 32 rows): the wave waits for HBM once
    uint32_t code[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int row = min(w_begin + min(r, max(w_rows - 1, 0)), out - 1);
        code[r] = uint32_t(__builtin_nontemporal_load(codes + size_t(row) * G + min(j0 + jl, G - 1)));
    }

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
        if ((lane & 3) == 0 && r < w_rows) partial[size_t(slice) * out + w_begin + r] = s;
    }
}

// y[row] = sum over slices (in slice order) of the partial sums, rounded to fp16.
// Loads are issued eight at a time so that a row waits for memory ceil(n/8) times.
__global__ void __launch_bounds__(256)
lut_reduce_kernel(const float *__restrict__ partial, uint16_t *__restrict__ y, int out,
                  int nslices) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= out) return;
    float s = 0.0f;
    for (int s0 = 0; s0 < nslices; s0 += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = (s0 + i < nslices) ? partial[size_t(s0 + i) * out + row] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += t[i];
    }
    y[row] = f2h_bits(s);
}

struct LutCfg {
    int nslices, nrblocks, rows_per_block;
};

LutCfg lut_cfg(const Problem &p) {
    LutCfg c{};
    const int64_t G = p.in / kGroup;
    c.nslices = int((G + kSlice - 1) / kSlice);
    // one workgroup per CU: about 256 / nslices row ranges, each at most
    // kLutWaves * kRowsPerWave rows (a wave's rows are all loaded at once)
    const int64_t max_rows = int64_t(kLutWaves) * kRowsPerWave;
    int64_t nrb = c.nslices >= 256 ? 1 : 256 / c.nslices;
    const int64_t need = (p.out + max_rows - 1) / max_rows;
    if (nrb < need) nrb = need;
    int64_t rpb = (p.out + nrb - 1) / nrb;
    rpb = (rpb + kLutWaves - 1) / kLutWaves * kLutWaves;   // whole rows per wave
    if (rpb < kLutWaves) rpb = kLutWaves;
    c.rows_per_block = int(rpb);
    c.nrblocks = int((p.out + rpb - 1) / rpb);
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
    const LutCfg c = lut_cfg(p);
    return size_t(c.nslices) * size_t(p.out) * sizeof(float);
}

// workspace: partial sums, nslices x out fp32 (no initial contents needed)
hipError_t launch_lut(const Problem &p, void *workspace) {
    const LutCfg c = lut_cfg(p);
    float *partial = static_cast<float *>(workspace);
    const int grid = c.nslices * c.nrblocks;
    hipLaunchKernelGGL(lut_kernel, dim3(grid), dim3(kLutWaves * kWave), 0, p.stream,
                       static_cast<const uint16_t *>(p.codes),
                       static_cast<const uint16_t *>(p.codebooks),
                       static_cast<const uint16_t *>(p.x), partial, int(p.out),
                       int(p.in / kGroup), c.rows_per_block, c.nslices);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lut_reduce_kernel, dim3(unsigned((p.out + 255) / 256)), dim3(256), 0,
                       p.stream, partial, static_cast<uint16_t *>(p.y), int(p.out), c.nslices);
    return hipGetLastError();
}

}  // namespace aqlm
