// Ceiling microbenchmarks (libaqlm_ceilings.so, used by bench.py only; not part of the
// product library): the rates the product kernels are bounded by on this GPU, measured
// with the same access patterns and no arithmetic of the method.
//
// * stream_read: one pass over n bytes with 16-byte non-temporal loads (the code
//   stream), grid-stride over a launch of one round of workgroups.  Timed per launch,
//   it gives the streaming read rate a single kernel of that size reaches.
// * l2_gather: random 16-byte reads from a table that stays in L2 (the 1 MiB codebook
//   of 16-bit codes): the L2 request rate that bounds an L2-gather decode.
// * lds_read: random LDS reads from a 128 KiB table per CU, in four patterns: 16-byte
//   reads (a gather of codebook vectors from LDS), 4-byte reads, 4-byte reads with half
//   of the lanes on one shared word (the position-pair lookups of the codebook-split
//   kernel, where codes of the other half of the code space read a zero word), and
//   16-byte reads with one lane in eight active (a workgroup holding one eighth of the
//   code space as whole vectors, looking up only the codes that fall in it).
//
// Every kernel folds what it read into one word per thread, stored to `sink`, so that
// no load is removed; indices come from a counter-based integer hash.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint32_t mix(uint32_t x) {
    // integer finaliser of MurmurHash3 (fmix32)
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// four 16-byte loads in flight per thread per round
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(256) l2_gather_kernel(const uint4 *__restrict__ table,
                                                        uint32_t entries_mask, int per_thread,
                                                        uint32_t *__restrict__ sink) {
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    // 8 gathers in flight per thread, as the L2-gather decode keeps them
    for (int i = 0; i < per_thread; i += 8) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = table[mix(t * 0x9e3779b9u + uint32_t(i + j)) & entries_mask];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    sink[t] = acc;
}

constexpr int kLdsBytes = 128 * 1024;

// MODE 0: 16-byte random reads; 1: 4-byte random reads; 2: 4-byte reads, odd lanes on
// one shared word; 3: 16-byte random reads issued with one lane in eight active (the
// active lanes drawn at random once per read slot, the others masked off).  1024
// threads per workgroup (16 waves), one workgroup per CU.  Each thread draws 8 random
// byte addresses once; iteration i reads them XORed with a wave-uniform offset (one
// VALU operation per read, so the LDS, not the index arithmetic, sets the rate; odd
// lanes in mode 2 keep the shared word).
template <int MODE>
__global__ void __launch_bounds__(1024) lds_read_kernel(int iters, uint32_t *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint32_t tab[kLdsBytes / 4];
    for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x) tab[i] = mix(uint32_t(i));
    __syncthreads();
    const uint32_t t = threadIdx.x;
    constexpr uint32_t align = (MODE == 0 || MODE == 3) ? 16u : 4u;
    uint32_t addr[8];
    bool act[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t r = mix(t * 0x9e3779b9u + uint32_t(j));
        addr[j] = (r % uint32_t(kLdsBytes)) & ~(align - 1);
        if (MODE == 2 && (t & 1)) addr[j] = kLdsBytes - 4;
        act[j] = MODE != 3 || (r >> 29) == 0;
    }
    const uint32_t keep = (MODE == 2 && (t & 1)) ? 0u : ~0u;
    const char *base = reinterpret_cast<const char *>(tab);
    uint32_t acc = 0;
    for (int i = 0; i < iters; i += 8) {
        const uint32_t off = (mix(uint32_t(i)) % uint32_t(kLdsBytes)) & ~(align - 1) & keep;
        if constexpr (MODE == 0) {
            uint4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const uint4 *>(base + (addr[j] ^ off));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
        } else if constexpr (MODE == 3) {
            uint4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v[j] = make_uint4(0u, 0u, 0u, 0u);
                if (act[j]) v[j] = *reinterpret_cast<const uint4 *>(base + (addr[j] ^ off));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
        } else {
            uint32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const uint32_t *>(base + (addr[j] ^ off));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc ^= v[j];
        }
    }
    sink[blockIdx.x * blockDim.x + t] = acc;
}

}  // namespace

extern "C" {

// Returns 0 when queued, else the hipError_t of the launch.  sink holds blocks * 256 words.
int ceil_stream_read(const void *src, int64_t nbytes, int blocks, void *sink, void *stream) {
    if (blocks < 1 || nbytes < 16) return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), nbytes / 16, static_cast<uint32_t *>(sink));
    return int(hipGetLastError());
}

// table_bytes a power of two >= 16; gathers = blocks * 256 * per_thread.
int ceil_l2_gather(const void *table, int64_t table_bytes, int blocks, int per_thread, void *sink,
                   void *stream) {
    if (table_bytes < 16 || (table_bytes & (table_bytes - 1)) || blocks < 1 || per_thread < 8 ||
        per_thread % 8)
        return int(hipErrorInvalidValue);
    hipLaunchKernelGGL(l2_gather_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(table), uint32_t(table_bytes / 16 - 1), per_thread,
                       static_cast<uint32_t *>(sink));
    return int(hipGetLastError());
}

// mode 0..3 as lds_read_kernel; sink holds blocks * 1024 words.
int ceil_lds_read(int mode, int blocks, int iters, void *sink, void *stream) {
    if (blocks < 1 || iters < 8 || iters % 8) return int(hipErrorInvalidValue);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *k = static_cast<uint32_t *>(sink);
    if (mode == 0) hipLaunchKernelGGL(lds_read_kernel<0>, dim3(blocks), dim3(1024), 0, s, iters, k);
    else if (mode == 1) hipLaunchKernelGGL(lds_read_kernel<1>, dim3(blocks), dim3(1024), 0, s, iters, k);
    else if (mode == 2) hipLaunchKernelGGL(lds_read_kernel<2>, dim3(blocks), dim3(1024), 0, s, iters, k);
    else if (mode == 3) hipLaunchKernelGGL(lds_read_kernel<3>, dim3(blocks), dim3(1024), 0, s, iters, k);
    else return int(hipErrorInvalidValue);
    return int(hipGetLastError());
}

}  // extern "C"
