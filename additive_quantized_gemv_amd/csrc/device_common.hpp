// Device-side helpers shared by the gfx950 kernels of libaqlm_mi355x.
#pragma once

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

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Streaming 16-byte load that should not stay in the caches (codes are read once).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace aqlm
