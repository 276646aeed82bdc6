// 16-bit-code GEMV with the codebook split by vector position (gfx950).
//
// The 8-wide dot product of the additive decode (page "AQLM (Additive
// Quantization for LLMs)", section "Niveau intermediaire") splits over its 8
// positions t:
//     y[b][o] = sum_t sum_k sum_j C_k[i_k(o,j)][t] * x[b][8j + t].
// The whole 1 MiB codebook does not fit the LDS of a CU, but 128 KiB of it does.
// So a workgroup owns one slice of it and one range of rows: it streams every code
// of its rows and turns each into an LDS read, instead of a 16-byte gather through
// L2, whose request rate caps the plain 16-bit kernel.
//
// * Codebooks are taken pre-packed as position pairs, [K][4][65536] x 2 fp16
//   (aqlm_pack_codebooks: a one-time layout change of the weights): word (k, q, c)
//   holds positions 2q and 2q+1 of entry c.
// * Batch <= 4, pair form (one codebook; batch 1, or batch b with b x chunk positions
//   per lane <= 8, e.g. batch 4 with in <= 8192): a
//   workgroup owns positions (2q, 2q+1) of the codebook for one half h of the code
//   space (32768 words = 128 KiB, followed by a zero word).  Every lane looks up
//   every code, at byte min(4*code - h*128 KiB, 128 KiB) (unsigned): a code of the
//   other half lands on the zero word, which all such lanes read at one address (a
//   broadcast).  Measured on MI355X, a 64-lane random 4-byte read with half of the
//   lanes on one address takes 5.4 cycles against 7.3 for 64 random 2-byte reads,
//   and it returns two positions per useful lane, so the lookups of a row cost ~27%
//   fewer LDS cycles than one 2-byte read per position.  The address is two VALU
//   operations (v_mad_u32_u16 picks the code's 16 bits, scales and offsets it; min).
// * Batch <= 4, plane form (otherwise): a workgroup owns position t of codebook k,
//   the 65536-entry plane taken from the pairs while staging, and looks up 2 bytes
//   per code; with several tokens sharing the lookups, one position per workgroup
//   halves the activation bytes each token reads from LDS.
// * The K*8 workgroups of one row range get block ids that are equal modulo 8,
//   so the dispatcher puts them on the same XCD: the codes come from HBM once and
//   from that XCD's L2 for the other planes.
// * The waves of a workgroup take the range's rows in chunks of 4, 2 or 1 rows (fewer
//   as the chunk positions per lane, times the tokens whose activation pairs a lane
//   holds in the pair form, grow from 1-2 to 3-4 to 5-8) from an
//   LDS counter (the waves the LDS serves first take more chunks).  A wave walks a
//   chunk's 16-byte code pieces with the next chunk's in flight (a ring of 4..8
//   loads, issued branch-free) and issues each slot's lookups one slot ahead of its
//   products; each looked-up pair is multiplied with v_dot2_f32_f16 against the
//   matching activation pair x[b][8j + 2q .. +1], staged in LDS (in registers when
//   they fit).  A chunk's rows are summed across lanes by a transposing butterfly.
// * Per-workgroup row sums go to a workspace; a second kernel adds the K*8 parts
//   in order and writes fp16 y.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace aqlm {
namespace {

constexpr int kDsWaves = 16;
constexpr int kEntries = 65536;
constexpr int kHalf = kEntries / 2;     // code-space half of one batch-1 workgroup
constexpr int kXPairs = 7168;           // in/8 activation pairs of one position pair (batch 1)
constexpr int kXPlaneHalves = 14336;    // batch * in/8 activations of one position (batch 2..4)
// words before the tables: the row-chunk counter, kept below 64 KiB (ds_append takes its
// address from m0)
constexpr int kCtrWords = 4;
// LDS words of the batch <= 4 kernel: the larger of its two layouts
constexpr int kDsLdsWords = kCtrWords + ((kHalf + 4 + kXPairs) > (kEntries / 2 + kXPlaneHalves / 2)
                                              ? (kHalf + 4 + kXPairs) : (kEntries / 2 + kXPlaneHalves / 2));
// tokens of the matrix-core form: one 16-token tile (measured on MI355X against unpacking
// and the canonical kernels: 1.3-6x faster at batches 5..8, even at 16, slower from 32)
constexpr int kDsmMaxBatch = 16;

typedef _Float16 hf;

// 4 * (low / high 16 bits of w) + boff in one v_mad_u32_u16 (the two-op shift-and-add
// the compiler emits otherwise makes the VALU, not the LDS, the limit of the lookups)
__device__ __forceinline__ uint32_t pair_byte_lo(uint32_t w, uint32_t boff) {
    uint32_t r;
    asm("v_mad_u32_u16 %0, %1, 4, %2" : "=v"(r) : "v"(w), "s"(boff));
    return r;
}
__device__ __forceinline__ uint32_t pair_byte_hi(uint32_t w, uint32_t boff) {
    uint32_t r;
    asm("v_mad_u32_u16 %0, %1, 4, %2 op_sel:[1,0,0,0]" : "=v"(r) : "v"(w), "s"(boff));
    return r;
}

// Plane t of codebook k (65536 fp16) into LDS from the packed pairs: half (t & 1) of
// each pair word (k, t >> 1, c), 4 entries per 16-byte load, rounds of 8 loads per
// thread, every load of a round issued before its LDS writes.  Called by all threads.
__device__ __forceinline__ void stage_plane(const uint16_t *__restrict__ planes, int k, int t, _Float16 *tab) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        reinterpret_cast<const uint32_t *>(planes) + (size_t(k) * 4 + (t >> 1)) * kEntries);
    uint2 *dst = reinterpret_cast<uint2 *>(tab);
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;   // the high or low halves
    constexpr int kThreads = kDsWaves * kWave;
    constexpr int PER = kEntries / 4 / kThreads;
#pragma unroll
    for (int r0 = 0; r0 < PER; r0 += 8) {
        uint4 tmp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) tmp[i] = src[threadIdx.x + (r0 + i) * kThreads];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[threadIdx.x + (r0 + i) * kThreads] =
                make_uint2(__builtin_amdgcn_perm(tmp[i].y, tmp[i].x, sel),
                           __builtin_amdgcn_perm(tmp[i].w, tmp[i].z, sel));
    }
}

// ds_kernel's pair form: one codebook, batch 1 (activation pairs in registers up to 7
// chunk positions per lane, 117 VGPRs at 7, else read from LDS; measured on MI355X,
// 1x16 8192x28672 with 7: 42.4 against 52.1 us per call) or batch b with b x positions
// <= 8, every token's pairs in registers (measured on MI355X: 1x16 28672x8192 at batch
// 4, 82.9 against 90.7 us per call in the plane form; two codebooks measured slower in
// the pair form: 149 against 144 us per 2x16 7B layer)
constexpr bool ds_pair_form(int K, int nb, int nseg) { return K == 1 && (nb == 1 || nb * nseg <= 8); }
constexpr bool ds_pair_xreg(int nb, int nseg) { return nb == 1 ? nseg <= 7 : nb * nseg <= 8; }

// W = chunk positions x tokens whose activation pairs a lane holds (NSEG in the plane form)
template <int W, int NSEG>
struct DsShape {
    // rows per chunk (reduced together), and code chunks in flight per lane (a multiple
    // of NSEG).  Measured on MI355X at one chunk position (1x16 11008x4096): chunks of 4
    // rows 13.8 us per call, of 8 rows 14.9 (the last round of chunks leaves waves
    // idle longer), of 2 rows 15.1 (too few rows in flight)
    static constexpr int RB = W <= 2 ? 4 : W <= 4 ? 2 : 1;
    static constexpr int D = NSEG * RB;
};

template <int K, int NB, int NSEG, int NS>
__global__ void __launch_bounds__(kDsWaves * kWave)
ds_kernel(const uint8_t *__restrict__ codes1, const uint16_t *__restrict__ planes1,
          const uint16_t *__restrict__ x, float *__restrict__ partial, int out1, int in,
          int batch, int nranges, int rows_per_range, const Segs segs) {
    constexpr int P = K * 8;                 // parts
    constexpr int GPC = 8 / K;               // groups per 16-byte chunk
    constexpr int RB = DsShape<(ds_pair_form(K, NB, NSEG) ? NB : 1) * NSEG, NSEG>::RB;
    constexpr int D = DsShape<(ds_pair_form(K, NB, NSEG) ? NB : 1) * NSEG, NSEG>::D;
    // PAIR (one codebook; batch 1, or batch 2 with NSEG = 1; the activation pairs sit in
    // registers when they fit without spilling, XREG, else they are read from LDS):
    // part (k, q, h) = position pair q of codebook k for code half h; LDS words
    // 0 .. kHalf-1 hold its pairs, word kHalf a zero (the other half's codes), then
    // the activation pairs x[b][8j + 2q .. +1].  Otherwise part (k, t) = position t,
    // the 65536-entry plane taken from the pairs while staging, then the activations
    // x[b][8j + t]: read from LDS per token, one position per part reads half the
    // activation bytes of the pair form.
    constexpr bool PAIR = ds_pair_form(K, NB, NSEG);
    constexpr bool XREG = PAIR && ds_pair_xreg(NB, NSEG);
    // Rows are handed out in chunks of RB from an LDS counter, so the waves that the LDS
    // serves first take more of them (with a fixed share per wave the last waves ended up
    // to 5 us after the first, with the LDS idle meanwhile; 1x16 11008x4096 on MI355X,
    // together with the lookahead below: 15.9 -> 15.3 us per call with the part sums).
    __shared__ __attribute__((aligned(16))) uint32_t lds[kDsLdsWords];
    uint32_t *const tab = lds + kCtrWords;                            // PAIR
    uint32_t *const xs = tab + kHalf + 4;                             // PAIR
    hf *const tabh = reinterpret_cast<hf *>(lds + kCtrWords);         // !PAIR
    hf *const xsh = reinterpret_cast<hf *>(lds + kCtrWords + kEntries / 2);   // !PAIR

    // block -> (part, row range); the parts of a range share id % 8, i.e. an XCD
    const int id = blockIdx.x;
    const int grp = id / (P * 8), rem = id - grp * (P * 8);
    const int p = rem >> 3;
    const int rr = grp * 8 + (rem & 7);
    if (rr >= nranges) return;
    const int k = p >> 3, q = (p >> 1) & 3, h = p & 1, t = p & 7;
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

    // Branch-free loads: the row pointer is wave-uniform (scalar) and each lane adds
    // its chunk offset, clamped into the row; a conditional load would make the
    // compiler wait for it at once.  Clamped lanes and rows are masked where the
    // chunk is used.
    const size_t row_bytes = size_t(NC) * 16u;
    uint32_t lane_off[NSEG];
    bool lane_ok[NSEG];
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
        lane_off[sg] = uint32_t(min(lane + kWave * sg, NC - 1)) * 16u;
        lane_ok[sg] = lane + kWave * sg < NC;
    }

    // The table gates all work, so it is staged first; code loads issued with it
    // would compete for the same bandwidth and delay it (about 2.5 us measured).
    // Every load of a thread (of a round) is issued before its LDS writes.
    if constexpr (PAIR) {
        // 128 KiB of pairs
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint32_t *>(planes) + (size_t(k) * 4 + q) * kEntries + size_t(h) * kHalf);
        uint4 *dst = reinterpret_cast<uint4 *>(tab);
        constexpr int PER = kHalf / 4 / (kDsWaves * kWave);
        // straight from global memory into LDS (global_load_lds_dwordx4: lane l's 16
        // bytes land at the wave's LDS base + 16 l), no round trip through registers
#pragma unroll
        for (int i = 0; i < PER; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + threadIdx.x + i * kDsWaves * kWave),
                (__attribute__((address_space(3))) void *)(dst + (threadIdx.x & ~(kWave - 1)) + i * kDsWaves * kWave),
                16, 0, 0);
        if (threadIdx.x == 0) tab[kHalf] = 0u;
    } else {
        stage_plane(planes, k, t, tabh);
    }
    // activations: x[b][8j + 2q .. +1] (PAIR) or x[b][8j + t]
    if constexpr (PAIR && NB == 1) {
        for (int j = threadIdx.x; j < G; j += blockDim.x)
            xs[j] = *reinterpret_cast<const uint32_t *>(x + size_t(j) * kGroup + 2 * q);
    } else {
        for (int b = 0; b < batch; ++b)
            for (int j = threadIdx.x; j < G; j += blockDim.x) {
                const uint16_t *src = x + size_t(b) * in + size_t(j) * kGroup;
                if constexpr (PAIR) xs[b * G + j] = *reinterpret_cast<const uint32_t *>(src + 2 * q);
                else xsh[b * G + j] = __builtin_bit_cast(hf, src[t]);
            }
    }
    if (threadIdx.x == 0) lds[0] = 2 * kDsWaves * kWave;   // next free row chunk x 64
    __syncthreads();
    // byte address of a code's pair: 4*code - h*128 KiB, clamped to the zero word
    const uint32_t boff = h ? uint32_t(0) - uint32_t(kHalf * 4) : 0u;
    const char *tabb = reinterpret_cast<const char *>(tab);
    // Wave w starts with chunks w and w + 16; each chunk takes the counter's next one for
    // two chunks ahead, and the current next chunk's codes refill the ring slot by slot.
    // The counter's value is read only after the chunk's last lookups: an atomic read at
    // once waits for every LDS read queued before it, the other waves' included.  It is
    // a ds_append (adds the 64 active lanes), which the compiler's atomic rewriting, with
    // its immediate read of the result, leaves alone.  The first chunk is unconditional
    // (clamped loads, masked stores): a loop entered behind a trip-count test lets the
    // compiler sink the ring loads below the barrier.
    const int nchunks = (r_end - r_begin + RB - 1) / RB;
    uint32_t *const ctr = lds;
    auto load_chunk = [&](int chunk, int s) -> u32x4 {
        const int row = min(r_begin + min(chunk, nchunks - 1) * RB + s / NSEG, r_end - 1);
        const uint8_t *rp = codes + size_t(row) * row_bytes;
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rp + lane_off[s % NSEG]));
    };
    u32x4 ring[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        ring[s] = load_chunk(wave, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    // XREG: each lane's activation pairs (GPC per chunk position and token) stay in
    // registers; a token past the batch repeats the last one (its sums are not stored),
    // so the loads need no condition (a conditional one becomes a branch per load)
    uint32_t xr[XREG ? NSEG : 1][GPC][XREG ? NB : 1];
    if constexpr (XREG) {
#pragma unroll
        for (int sg = 0; sg < NSEG; ++sg) {
            const int c = min(lane + kWave * sg, NC - 1);
#pragma unroll
            for (int g = 0; g < GPC; ++g)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    xr[sg][g][b] = xs[(NB == 1 ? 0 : min(b, batch - 1)) * G + c * GPC + g];
        }
    }
    const uint32_t ksh = 16u * uint32_t(k);   // K = 2: codebook k's code is half k of a word
    // looked-up values of one slot: pairs (PAIR) or plane halves
    using VT = std::conditional_t<PAIR, uint32_t, hf>;

    int cur = wave, nxt = wave + kDsWaves;
    do {
        const int nx = __builtin_amdgcn_ds_append((__attribute__((address_space(3))) int *)(ctr));
        __builtin_amdgcn_sched_barrier(0);
        float acc[NB][RB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < RB; ++r) acc[b][r] = 0.0f;
        // The lookups of slot s + 1 are issued before the products of slot s, so each wave
        // keeps two slots of LDS reads in flight.  A slot is refilled with the next
        // chunk's codes once its own are consumed, in place: a refill issued while the old
        // value is still in use makes the compiler rotate the ring through register
        // copies, and each copy waits for its load (measured: every iteration then waited
        // for nearly the whole ring, 16.7 against 15.9 us per 11008x4096 1x16 call).
        VT vb[2][GPC];
        auto look = [&](int s, VT *v) {
            const u32x4 cw = ring[s];
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                if constexpr (PAIR) {
                    // pair of this code (codebook k of group g), zero for the other half;
                    // code n = g*K + k of the chunk: word n/2 is g/2 (K = 1) or g (K = 2)
                    uint32_t byte;
                    if constexpr (K == 1)
                        byte = (g & 1) ? pair_byte_hi(cw[g >> 1], boff) : pair_byte_lo(cw[g >> 1], boff);
                    else   // the low 16 bits after the shift are codebook k's code
                        byte = pair_byte_lo(cw[g] >> ksh, boff);
                    byte = min(byte, uint32_t(kHalf * 4));
                    v[g] = *reinterpret_cast<const uint32_t *>(tabb + byte);
                } else {
                    uint32_t code;
                    if constexpr (K == 1) {
                        const uint32_t w = cw[g >> 1];
                        code = (g & 1) ? (w >> 16) : (w & 0xFFFFu);
                    } else {
                        code = (cw[g] >> (16 * k)) & 0xFFFFu;
                    }
                    v[g] = tabh[code];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            ring[s] = load_chunk(nxt, s);
            __builtin_amdgcn_sched_barrier(0);
        };
        look(0, vb[0]);
#pragma unroll
        for (int s = 0; s < D; ++s) {
            if (s + 1 < D) look(s + 1, vb[(s + 1) & 1]);
            const VT *v = vb[s & 1];
            const int seg = s % NSEG;
            const int c = min(lane + kWave * seg, NC - 1);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float d = 0.0f;
                if constexpr (XREG) {
#pragma unroll
                    for (int g = 0; g < GPC; ++g)
                        d = __builtin_amdgcn_fdot2(as_h2(v[g]), as_h2(xr[seg][g][b]), d, false);
                } else if constexpr (PAIR) {
                    // GPC * 4 bytes, 16-byte aligned (G is a multiple of GPC)
                    const uint4 *xq = reinterpret_cast<const uint4 *>(xs + b * G + c * GPC);
#pragma unroll
                    for (int i = 0; i < GPC / 4; ++i) {
                        const uint4 t4 = xq[i];
                        d = __builtin_amdgcn_fdot2(as_h2(v[4 * i]), as_h2(t4.x), d, false);
                        d = __builtin_amdgcn_fdot2(as_h2(v[4 * i + 1]), as_h2(t4.y), d, false);
                        d = __builtin_amdgcn_fdot2(as_h2(v[4 * i + 2]), as_h2(t4.z), d, false);
                        d = __builtin_amdgcn_fdot2(as_h2(v[4 * i + 3]), as_h2(t4.w), d, false);
                    }
                } else if (b < batch) {
                    const hf *xp = xsh + b * G + c * GPC;
#pragma unroll
                    for (int g = 0; g < GPC; g += 2)
                        d = __builtin_amdgcn_fdot2(half2v{v[g], v[g + 1]}, half2v{xp[g], xp[g + 1]}, d, false);
                }
                acc[b][s / NSEG] += lane_ok[seg] ? d : 0.0f;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int nxt2 = __builtin_amdgcn_readfirstlane(nx) / kWave;
        // rows of chunk cur, RB of them reduced together
        const int row = r_begin + cur * RB + lane / (kWave / RB);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (NB == 1 || b < batch) {
                const float sum = transpose_reduce<RB>(acc[b], lane);
                if ((lane & (kWave / RB - 1)) == 0 && row < r_end)
                    partial[(size_t(p) * (NB == 1 ? 1 : batch) + b) * T + orow0 + row] = sum;
            }
        }
        cur = nxt;
        nxt = nxt2;
    } while (cur < nchunks);
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

    stage_plane(planes, k, t, tab);   // plane t (128 KiB) from the pairs
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

// Packed codebooks: W = 1 (8-bit codes): planes[k][t][c] = codebooks[k][c][t] (fp16);
// W = 2 (16-bit codes): pairs[k][q][c] = codebooks[k][c][2q .. 2q+1] (32-bit words).
template <int W>
__global__ void __launch_bounds__(256)
pack_kernel(const uint16_t *__restrict__ cb, uint16_t *__restrict__ packed, int K, int entries) {
    using U = typename std::conditional<W == 1, uint16_t, uint32_t>::type;
    constexpr int N = 8 / W;   // units per entry
    const U *__restrict__ src = reinterpret_cast<const U *>(cb);
    U *__restrict__ dst = reinterpret_cast<U *>(packed);
    const int64_t n = int64_t(K) * entries;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t kk = i / entries, c = i - kk * entries;
#pragma unroll
        for (int t = 0; t < N; ++t) dst[(kk * N + t) * entries + c] = src[i * N + t];
    }
}

// pack_kernel<2> for the codebooks of the matrices of segs (blockIdx.y = matrix m),
// written to dst + m * K * 65536 * 8 halves
__global__ void __launch_bounds__(256)
pack_pairs_segs_kernel(const Segs segs, uint32_t *__restrict__ dst, int K) {
    const int m = blockIdx.y;
    const uint32_t *__restrict__ src = static_cast<const uint32_t *>(pick(segs.cb, m));
    uint32_t *__restrict__ out = dst + size_t(m) * K * kEntries * 4;
    const int64_t n = int64_t(K) * kEntries;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t kk = i / kEntries, c = i - kk * kEntries;
        const uint4 v = reinterpret_cast<const uint4 *>(src)[i];   // entry c: 4 pairs
        out[(kk * 4 + 0) * kEntries + c] = v.x;
        out[(kk * 4 + 1) * kEntries + c] = v.y;
        out[(kk * 4 + 2) * kEntries + c] = v.z;
        out[(kk * 4 + 3) * kEntries + c] = v.w;
    }
}

// the inverse of pack_kernel<W>
template <int W>
__global__ void __launch_bounds__(256)
unpack_kernel(const uint16_t *__restrict__ packed, uint16_t *__restrict__ cb, int K, int entries) {
    using U = typename std::conditional<W == 1, uint16_t, uint32_t>::type;
    constexpr int N = 8 / W;
    const U *__restrict__ src = reinterpret_cast<const U *>(packed);
    U *__restrict__ dst = reinterpret_cast<U *>(cb);
    const int64_t n = int64_t(K) * entries;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t kk = i / entries, c = i - kk * entries;
#pragma unroll
        for (int t = 0; t < N; ++t) dst[i * N + t] = src[(kk * N + t) * entries + c];
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

namespace {

// The parts of one matrix added in order, each workgroup on the XCD that ran its row range
// (range rr: block ids equal to rr modulo 8 in ds_kernel), so that it finds the parts in
// that XCD's L2.  One wave per workgroup, 64 rows of one range, token blockIdx.y; every
// part's load is issued before the first add.  Measured on MI355X (1x16 4096 x 11008,
// batch 1, packed): 14.15 against 14.85 us per call with the rows handed out in order.
template <int P>
__global__ void __launch_bounds__(64)
ds_partial_sum_kernel(const float *__restrict__ partial, uint16_t *__restrict__ y, int out,
                      int batch, int rows_per_range, int nranges, int chunks) {
    const int b = blockIdx.x;
    const int rest = b >> 3;
    const int c = rest % chunks;
    const int rr = (rest / chunks) * 8 + (b & 7);
    if (rr >= nranges) return;
    const int row = rr * rows_per_range + c * 64 + int(threadIdx.x);
    if (row >= min(out, (rr + 1) * rows_per_range)) return;
    const int tok = blockIdx.y;
    float v[P];
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = partial[(size_t(q) * batch + tok) * out + row];
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < P; ++q) s += v[q];
    y[size_t(tok) * out + row] = f2h_bits(s);
}

hipError_t launch_ds_partial_sum(const Problem &p, const DsCfg &c, const Segs &segs, const float *partial) {
    if (segs.n > 1) return launch_partial_sum_segs(partial, segs, p.batch, p.K * 8, p.stream);
    const int chunks = (c.rows_per_range + 63) / 64;
    const dim3 g(unsigned(c.nranges_padded * chunks), unsigned(p.batch)), b(64);
    uint16_t *y = static_cast<uint16_t *>(segs.y[0]);
    const int out = segs.row0[1];
    if (p.K == 1)
        hipLaunchKernelGGL(ds_partial_sum_kernel<8>, g, b, 0, p.stream, partial, y, out, p.batch,
                           c.rows_per_range, c.nranges, chunks);
    else
        hipLaunchKernelGGL(ds_partial_sum_kernel<16>, g, b, 0, p.stream, partial, y, out, p.batch,
                           c.rows_per_range, c.nranges, chunks);
    return hipGetLastError();
}

}  // namespace

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
    return launch_ds_partial_sum(p, c, segs, partial);
}

bool ds_supported(const Problem &p) {
    if (p.B != 16 || (p.K != 1 && p.K != 2)) return false;
    if (p.batch < 1 || p.batch > 4) return false;
    const int64_t G = p.in / kGroup;
    if (G % (8 / p.K)) return false;
    const int64_t NC = G / (8 / p.K);
    const int64_t nseg = (NC + kWave - 1) / kWave;
    if (nseg > 8) return false;
    // the kernel's two LDS layouts (see ds_kernel)
    const int nb = p.batch <= 1 ? 1 : p.batch <= 2 ? 2 : 4;
    if (int64_t(p.batch) * G > (ds_pair_form(p.K, nb, int(nseg)) ? kXPairs : kXPlaneHalves)) return false;
    if (p.out > (1 << 28)) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.codes) |
                        reinterpret_cast<uintptr_t>(p.codebooks);
    // activation pairs are staged with 4-byte loads
    return (a & 15u) == 0 && (reinterpret_cast<uintptr_t>(p.x) & 3u) == 0;
}

size_t ds_workspace_bytes(const Problem &p) {
    return size_t(p.K) * 8 * size_t(p.batch) * size_t(p.out) * sizeof(float);
}

// segs.cb holds the packed pairs [K][4][65536]; workspace: K*8 x batch x T fp32
hipError_t launch_ds(const Problem &p, void *workspace) {
    Segs segs = p.segs;
    const DsCfg c = ds_cfg(p, &segs);
    float *partial = static_cast<float *>(workspace);
    hipError_t e = p.K == 1 ? launch1<1>(p, c, segs, partial) : launch1<2>(p, c, segs, partial);
    if (e != hipSuccess) return e;
    return launch_ds_partial_sum(p, c, segs, partial);
}

size_t split_canonical_pack_bytes(const Problem &p) {
    return size_t(p.segs.n) * size_t(p.K) * kEntries * 16;
}

size_t split_canonical_workspace_bytes(const Problem &p) {
    return split_canonical_pack_bytes(p) + ds_workspace_bytes(p);
}

// Canonical codebooks: each matrix's codebook is packed into position pairs in the
// workspace (one launch for all matrices), then the split kernel runs on them.
hipError_t launch_split_canonical(const Problem &p, void *workspace) {
    uint32_t *pairs = static_cast<uint32_t *>(workspace);
    const int64_t n = int64_t(p.K) * kEntries;
    const int blocks = int((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(pack_pairs_segs_kernel, dim3(blocks, unsigned(p.segs.n)), dim3(256), 0,
                       p.stream, p.segs, pairs, p.K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    Problem q = p;
    for (int m = 0; m < p.segs.n; ++m) q.segs.cb[m] = pairs + size_t(m) * p.K * kEntries * 4;
    q.codebooks = q.segs.cb[0];
    return launch_ds(q, static_cast<char *>(workspace) + split_canonical_pack_bytes(p));
}

hipError_t launch_pack_codebooks(const void *cb, void *planes, int K, int B, hipStream_t s) {
    const int entries = 1 << B;
    const int64_t n = int64_t(K) * entries;
    const int blocks = int((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (B == 16)
        hipLaunchKernelGGL(pack_kernel<2>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(cb), static_cast<uint16_t *>(planes), K,
                           entries);
    else
        hipLaunchKernelGGL(pack_kernel<1>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(cb), static_cast<uint16_t *>(planes), K,
                           entries);
    return hipGetLastError();
}

hipError_t launch_unpack_codebooks(const void *planes, void *cb, int K, int B, hipStream_t s) {
    const int entries = 1 << B;
    const int64_t n = int64_t(K) * entries;
    const int blocks = int((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (B == 16)
        hipLaunchKernelGGL(unpack_kernel<2>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(planes), static_cast<uint16_t *>(cb), K,
                           entries);
    else
        hipLaunchKernelGGL(unpack_kernel<1>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(planes), static_cast<uint16_t *>(cb), K,
                           entries);
    return hipGetLastError();
}

}  // namespace aqlm
