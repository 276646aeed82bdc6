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
// * Slice partials go to a workspace; the last workgroup to finish a row range
//   (atomic counter) sums the slices in slice order and writes fp16 y, then
//   resets its counter.  Results are deterministic.
#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kSlice = 64;              // groups per slice (= lanes)
constexpr int kLutWaves = 16;           // 1024 threads
constexpr int kRowsPerIter = 16;        // rows a wave handles at once
constexpr int kLutBytes = 2 * 256 * kSlice * 4;
constexpr size_t kCounterBytes = 4096;  // room for 1024 row-range counters (at most 256 used)

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lds_f32(const char *base, uint32_t byte_addr) {
    return *reinterpret_cast<const float *>(base + byte_addr);
}

// Sum of the two halves returned by a permlane swap.  The halves are taken as
// plain scalars first: bit-casting an element of the builtin's two-element result
// directly reads element 0 twice with this compiler.
__device__ __forceinline__ float swap_sum(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// sum over the 64 lanes of 16 values v[0..15]; afterwards lane l holds the total of
// value (l >> 2).
__device__ __forceinline__ float transpose_reduce16(float v[16], int lane) {
    // lanes 0-31 keep rows 0..7, lanes 32-63 keep rows 8..15
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[i]),
                                                        __builtin_bit_cast(uint32_t, v[i + 8]),
                                                        false, false);
        v[i] = swap_sum(s[0], s[1]);
    }
    // bit 4 of the lane selects rows i or i+4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v[i]),
                                                        __builtin_bit_cast(uint32_t, v[i + 4]),
                                                        false, false);
        v[i] = swap_sum(s[0], s[1]);
    }
    // bit 3: pair with the mirrored lane of the 16-lane row
    const bool b3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b3 ? v[i] : v[i + 2];
        const float keep = b3 ? v[i + 2] : v[i];
        v[i] = keep + dpp_f<0x140>(send);       // row_mirror
    }
    // bit 2: pair with the mirrored lane of the 8-lane half row
    const bool b2 = lane & 4;
    {
        const float send = b2 ? v[0] : v[1];
        const float keep = b2 ? v[1] : v[0];
        v[0] = keep + dpp_f<0x141>(send);       // row_half_mirror
    }
    float t = v[0];
    t += dpp_f<0xB1>(t);                         // xor 1
    t += dpp_f<0x4E>(t);                         // xor 2
    return t;
}

__global__ void __launch_bounds__(kLutWaves * kWave)
lut_kernel(const uint16_t *__restrict__ codes, const uint16_t *__restrict__ cb,
           const uint16_t *__restrict__ x, uint16_t *__restrict__ y, float *__restrict__ partial,
           unsigned *__restrict__ counters, int out, int G, int rows_per_block, int nslices) {
    __shared__ __attribute__((aligned(16))) char lut[kLutBytes];
    __shared__ int last_flag;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slice = blockIdx.x % nslices;
    const int rblock = blockIdx.x / nslices;
    const int j0 = slice * kSlice;
    const int jl = lane;
    const bool jvalid = j0 + jl < G;
    const int r_begin = rblock * rows_per_block;
    const int r_end = min(out, r_begin + rows_per_block);

    // issue the first row group's code loads before building the tables
    int rg = r_begin + wave * kRowsPerIter;
    uint32_t code[kRowsPerIter];
#pragma unroll
    for (int r = 0; r < kRowsPerIter; ++r) {
        const int o = min(rg + r, out - 1);
        code[r] = jvalid ? uint32_t(__builtin_nontemporal_load(codes + size_t(o) * G + j0 + jl))
                         : 0u;
    }

    // ---- build L[e][jl] = C[e] . x_{j0+jl} for the 512 entries e = k*256 + c
    // wave w computes entries 32w .. 32w+31 for both 32-group halves of the slice
    {
        const int e = wave * 32 + (lane & 31);
        const int kq = (lane >> 5) * 4;          // this lane's 4 of the 8 vector positions
        const half4 a = *reinterpret_cast<const half4 *>(cb + size_t(e) * kGroup + kq);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int j = j0 + nb * 32 + (lane & 31);
            half4 bx = {0, 0, 0, 0};
            if (j < G) bx = *reinterpret_cast<const half4 *>(x + size_t(j) * kGroup + kq);
            float16v d = {};
            d = __builtin_amdgcn_mfma_f32_32x32x8f16(a, bx, d, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int n = nb * 32 + (lane & 31);
                *reinterpret_cast<float *>(lut + (wave * 32 + m) * 256 + n * 4) = d[r];
            }
        }
    }
    __syncthreads();

    // byte-address template: byte0 = 4*jl, byte2 = 1 selects the second table half
    const uint32_t lanebase = (uint32_t(jl) << 2) | (1u << 16);
    for (; rg < r_end; rg += kLutWaves * kRowsPerIter) {
        float v[kRowsPerIter];
#pragma unroll
        for (int r = 0; r < kRowsPerIter; ++r) {
            // addr0 = [4jl, i0, 0, 0], addr1 = [4jl, i1, 1, 0]
            const uint32_t a0 = __builtin_amdgcn_perm(lanebase, code[r], 0x0C0C0004u);
            const uint32_t a1 = __builtin_amdgcn_perm(lanebase, code[r], 0x0C060104u);
            v[r] = lds_f32(lut, a0) + lds_f32(lut, a1);
        }
        // prefetch the next row group of this wave
        const int rn = rg + kLutWaves * kRowsPerIter;
        if (rn < r_end) {
#pragma unroll
            for (int r = 0; r < kRowsPerIter; ++r) {
                const int o = min(rn + r, out - 1);
                code[r] = jvalid ? uint32_t(__builtin_nontemporal_load(codes + size_t(o) * G +
                                                                       j0 + jl))
                                 : 0u;
            }
        }
        const float s = transpose_reduce16(v, lane);
        const int row = rg + (lane >> 2);
        if ((lane & 3) == 0 && row < r_end) partial[size_t(slice) * out + row] = s;
    }

    // ---- last workgroup of this row range sums the slices
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&counters[rblock], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == unsigned(nslices - 1));
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    for (int row = r_begin + threadIdx.x; row < r_end; row += blockDim.x) {
        float s = 0.0f;
        for (int sl = 0; sl < nslices; ++sl)
            s += __builtin_nontemporal_load(partial + size_t(sl) * out + row);
        y[row] = f2h_bits(s);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[rblock], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct LutCfg {
    int nslices, nrblocks, rows_per_block;
};

LutCfg lut_cfg(const Problem &p) {
    LutCfg c{};
    const int64_t G = p.in / kGroup;
    c.nslices = int((G + kSlice - 1) / kSlice);
    int nrb = c.nslices >= 256 ? 1 : 256 / c.nslices;
    const int64_t max_rb = (p.out + kRowsPerIter - 1) / kRowsPerIter;
    if (nrb > max_rb) nrb = int(max_rb);
    if (nrb < 1) nrb = 1;
    int64_t rpb = (p.out + nrb - 1) / nrb;
    rpb = (rpb + kRowsPerIter - 1) / kRowsPerIter * kRowsPerIter;
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
    return kCounterBytes + size_t(c.nslices) * size_t(p.out) * sizeof(float);
}

// workspace: [kCounterBytes of counters, all zero between calls][partials: nslices x out fp32].
// The counters sit at a fixed offset so that calls with different shapes reuse
// them: every counter a call uses is back at zero when the call ends.
hipError_t launch_lut(const Problem &p, void *workspace) {
    const LutCfg c = lut_cfg(p);
    unsigned *counters = static_cast<unsigned *>(workspace);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes);
    const int grid = c.nslices * c.nrblocks;
    hipLaunchKernelGGL(lut_kernel, dim3(grid), dim3(kLutWaves * kWave), 0, p.stream,
                       static_cast<const uint16_t *>(p.codes),
                       static_cast<const uint16_t *>(p.codebooks),
                       static_cast<const uint16_t *>(p.x), static_cast<uint16_t *>(p.y), partial,
                       counters, int(p.out), int(p.in / kGroup), c.rows_per_block, c.nslices);
    return hipGetLastError();
}

}  // namespace aqlm
