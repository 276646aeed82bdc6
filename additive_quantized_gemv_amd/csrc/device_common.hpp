// Device-side helpers shared by the gfx950 kernels of libaqlm_mi355x.
#pragma once
#define AQLM_DEVICE_COMMON

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace aqlm {

constexpr int kGroup = 8;   // weights per code group (8 consecutive input columns)
constexpr int kWave = 64;   // CDNA wavefront width

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ bit helpers

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float h2f(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint16_t f2h_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// a.x*b.x + a.y*b.y + c with fp32 accumulation (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// 8-wide fp16 dot product accumulated into c (four v_dot2_f32_f16).
__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b, float c) {
    c = dot2(a.x, b.x, c);
    c = dot2(a.y, b.y, c);
    c = dot2(a.z, b.z, c);
    c = dot2(a.w, b.w, c);
    return c;
}

// ------------------------------------------------------- DPP wave reductions

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, BANK_MASK, true));
}

// Sum over the 64 lanes of a wave; the total is valid in lane 63.
// quad_perm xor-1 / xor-2, half-row and row mirrors, then row_bcast:15 / :31.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += dpp_f<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);         // row_half_mirror
    v += dpp_f<0x140>(v);         // row_mirror
    v += dpp_f<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(
        __builtin_bit_cast(int, wave_sum_to_lane63(v)), 63));
}

// Sum of the two halves returned by a permlane swap.  The halves are taken as
// plain scalars: bit-casting an element of the builtin's two-element result
// directly reads element 0 twice with this compiler.
__device__ __forceinline__ float swap_sum(uint32_t lo, uint32_t hi) {
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Exchange step over lane bit BIT: pairs (a, b) -> one value per lane, the sum over
// the two lanes of `a` where the bit is clear and of `b` where it is set.
template <int BIT>
__device__ __forceinline__ float butterfly_step(float a, float b, int lane) {
    if constexpr (BIT == 5) {
        const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                        __builtin_bit_cast(uint32_t, b), false,
                                                        false);
        return swap_sum(s[0], s[1]);
    } else if constexpr (BIT == 4) {
        const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a),
                                                        __builtin_bit_cast(uint32_t, b), false,
                                                        false);
        return swap_sum(s[0], s[1]);
    } else {
        const bool hi = (lane >> BIT) & 1;
        const float send = hi ? a : b;
        const float keep = hi ? b : a;
        // partners: row_mirror flips bits 0-3, row_half_mirror bits 0-2, quad perms bit 1 / 0
        if constexpr (BIT == 3) return keep + dpp_f<0x140>(send);
        else if constexpr (BIT == 2) return keep + dpp_f<0x141>(send);
        else if constexpr (BIT == 1) return keep + dpp_f<0x4E>(send);
        else return keep + dpp_f<0xB1>(send);
    }
}

// All-lane sum over lane bit BIT (the value of the partner lane is added).
template <int BIT>
__device__ __forceinline__ float allreduce_step(float v) {
    if constexpr (BIT == 5) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return swap_sum(s[0], s[1]);
    } else if constexpr (BIT == 4) {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return swap_sum(s[0], s[1]);
    } else if constexpr (BIT == 3) {
        return v + dpp_f<0x140>(v);
    } else if constexpr (BIT == 2) {
        return v + dpp_f<0x141>(v);
    } else if constexpr (BIT == 1) {
        return v + dpp_f<0x4E>(v);
    } else {
        return v + dpp_f<0xB1>(v);
    }
}

template <int R, int LEVEL>
__device__ __forceinline__ void butterfly_levels(float *v, int lane) {
    if constexpr (R > 1) {
        constexpr int BIT = 5 - LEVEL;
#pragma unroll
        for (int i = 0; i < R / 2; ++i) v[i] = butterfly_step<BIT>(v[i], v[i + R / 2], lane);
        butterfly_levels<R / 2, LEVEL + 1>(v, lane);
    }
}

template <int LEVEL>
__device__ __forceinline__ float allreduce_levels(float v) {
    if constexpr (LEVEL < 6) return allreduce_levels<LEVEL + 1>(allreduce_step<5 - LEVEL>(v));
    else return v;
}

// Sums v[0..R-1] over the 64 lanes of the wave at once (R a power of two <= 64,
// about 2 instructions per value): afterwards lane l holds the total of value
// l >> (6 - log2 R).
template <int R>
__device__ __forceinline__ float transpose_reduce(float *v, int lane) {
    constexpr int LOG = R <= 1 ? 0 : R <= 2 ? 1 : R <= 4 ? 2 : R <= 8 ? 3 : R <= 16 ? 4 : R <= 32 ? 5 : 6;
    static_assert((1 << LOG) == R, "R must be a power of two");
    butterfly_levels<R, 0>(v, lane);
    return allreduce_levels<LOG>(v[0]);
}

// The index m (< n <= 4) with bounds[m] <= v < bounds[m + 1]; bounds ascending.
__device__ __forceinline__ int range_of(int n, const int *bounds, int v) {
    int m = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i) m += (i < n && v >= bounds[i]) ? 1 : 0;
    return m;
}

// a[m] for a uniform m (a matrix-table lookup).
template <class T, int N>
__device__ __forceinline__ T pick(const T (&a)[N], int m) {
    T r = a[0];
#pragma unroll
    for (int i = 1; i < N; ++i) r = (m == i) ? a[i] : r;
    return r;
}


// Makes the (wave-uniform) kernel arguments given live in scalar registers at this point,
// so their loads are issued together and waited for once, before what follows.
// Matrix-table lookups of a kernel compiled for NS matrices: with NS = 1 the index is the
// constant 0 and the table's other entries are never read.
template <int NS, int N>
__device__ __forceinline__ int seg_of(int n, const int (&bounds)[N], int v) {
    return NS == 1 ? 0 : range_of(n, bounds, v);
}
template <int NS, int N>
__device__ __forceinline__ int seg_total(int n, const int (&row0)[N]) {
    return NS == 1 ? row0[1] : pick(row0, n);
}

template <class T>
__device__ __forceinline__ void scalar_ready(const T &v) {
    asm volatile("" ::"s"(v));
}
template <class... A>
__device__ __forceinline__ void scalars_ready(const A &...a) {
    (scalar_ready(a), ...);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Streaming 16-byte load that should not stay in the caches (codes are read once).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace aqlm
