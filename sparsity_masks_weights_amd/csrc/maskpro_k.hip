// maskpro_k.hip -- gfx950 kernels of the linear-space N:M mask learner
// (MaskPro summary page, "Approach"): M logits per block of M weights, an
// ordered draw of N positions without replacement (Gumbel-top-k on the noise
// contract of maskgs_device.hpp), the hard-masked weights, the policy
// gradient of the draw's log-likelihood, and the initial logits.
//
// One lane per block.  A block's logits are 16 B (2:4) or 32 B (4:8) and its
// weights 8 or 16 B (bf16), so consecutive lanes read consecutive 16-byte
// vectors: every load and store is a coalesced dwordx2/dwordx4.  There is no
// reuse between blocks; LDS holds only the noise contract's coefficient
// table, one copy per workgroup.  The work per byte is the Philox stream and
// one table evaluation per position (and, for the gradient drawn again, the
// N rounds of exponentials), which keeps these kernels near the VALU/HBM
// balance point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "maskgs_device.hpp"
#include "maskgs_launch.hpp"
#include "maskpro_launch.hpp"

namespace maskgs {
namespace {

// Lanes per workgroup: 512 against 256 took the 7B sweep's draw 10.44 -> 10.22
// ms, the gradient from the saved order 9.04 -> 8.88 ms and the redrawn one
// 10.31 -> 10.07 ms (three alternating runs), with half as many copies of the
// noise table to load.
constexpr int kThreads = 512;

// ---------------------------------------------------------------------------
// Vector access to one block of M elements of T.
// ---------------------------------------------------------------------------
template <typename T, int M>
struct BlockIo;

template <>
struct BlockIo<float, 4> {
    static __device__ __forceinline__ void load(const void *base, int64_t b, float (&v)[4]) {
        const float4 x = reinterpret_cast<const float4 *>(base)[b];
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
    static __device__ __forceinline__ void store(void *base, int64_t b, const float (&v)[4]) {
        reinterpret_cast<float4 *>(base)[b] = make_float4(v[0], v[1], v[2], v[3]);
    }
    static __device__ __forceinline__ void load_raw(const void *base, int64_t b,
                                                    uint32_t (&r)[4]) {
        const uint4 x = reinterpret_cast<const uint4 *>(base)[b];
        r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
    }
    static __device__ __forceinline__ void store_raw(void *base, int64_t b,
                                                     const uint32_t (&r)[4]) {
        reinterpret_cast<uint4 *>(base)[b] = make_uint4(r[0], r[1], r[2], r[3]);
    }
};

template <>
struct BlockIo<float, 8> {
    static __device__ __forceinline__ void load(const void *base, int64_t b, float (&v)[8]) {
        const float4 *p = reinterpret_cast<const float4 *>(base) + 2 * b;
        const float4 x = p[0], y = p[1];
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    }
    static __device__ __forceinline__ void store(void *base, int64_t b, const float (&v)[8]) {
        float4 *p = reinterpret_cast<float4 *>(base) + 2 * b;
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    static __device__ __forceinline__ void load_raw(const void *base, int64_t b,
                                                    uint32_t (&r)[8]) {
        const uint4 *p = reinterpret_cast<const uint4 *>(base) + 2 * b;
        const uint4 x = p[0], y = p[1];
        r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
        r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
    }
    static __device__ __forceinline__ void store_raw(void *base, int64_t b,
                                                     const uint32_t (&r)[8]) {
        uint4 *p = reinterpret_cast<uint4 *>(base) + 2 * b;
        p[0] = make_uint4(r[0], r[1], r[2], r[3]);
        p[1] = make_uint4(r[4], r[5], r[6], r[7]);
    }
};

// bf16 blocks as raw 16-bit patterns, two per dword.
template <>
struct BlockIo<bf16_t, 4> {
    static __device__ __forceinline__ void load_raw(const void *base, int64_t b,
                                                    uint32_t (&r)[4]) {
        const uint2 x = reinterpret_cast<const uint2 *>(base)[b];
        r[0] = x.x & 0xFFFFu; r[1] = x.x >> 16; r[2] = x.y & 0xFFFFu; r[3] = x.y >> 16;
    }
    static __device__ __forceinline__ void store_raw(void *base, int64_t b,
                                                     const uint32_t (&r)[4]) {
        reinterpret_cast<uint2 *>(base)[b] = make_uint2(r[0] | (r[1] << 16), r[2] | (r[3] << 16));
    }
};

template <>
struct BlockIo<bf16_t, 8> {
    static __device__ __forceinline__ void load_raw(const void *base, int64_t b,
                                                    uint32_t (&r)[8]) {
        const uint4 x = reinterpret_cast<const uint4 *>(base)[b];
        const uint32_t d[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[2 * i] = d[i] & 0xFFFFu;
            r[2 * i + 1] = d[i] >> 16;
        }
    }
    static __device__ __forceinline__ void store_raw(void *base, int64_t b,
                                                     const uint32_t (&r)[8]) {
        reinterpret_cast<uint4 *>(base)[b] =
            make_uint4(r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16),
                       r[6] | (r[7] << 16));
    }
};

// Raw element -> |w| ordering key (sign cleared) and -> output element.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static __device__ __forceinline__ uint32_t magnitude(uint32_t r) { return r & 0x7FFFFFFFu; }
    // raw fp32 -> raw of the output type
    static __device__ __forceinline__ uint32_t to_bf16(uint32_t r) {
        return bf16_rne(__uint_as_float(r));
    }
    static __device__ __forceinline__ uint32_t to_f32(uint32_t r) { return r; }
};

template <>
struct Elem<bf16_t> {
    static __device__ __forceinline__ uint32_t magnitude(uint32_t r) { return r & 0x7FFFu; }
    static __device__ __forceinline__ uint32_t to_bf16(uint32_t r) { return r; }
    static __device__ __forceinline__ uint32_t to_f32(uint32_t r) { return r << 16; }
};

// ---------------------------------------------------------------------------
// The draw: keys a_j = fp32(pi_j + g_j) (g_j from Philox word gb*M + j), then
// N rounds of "first largest key among the positions not yet drawn" (strict
// '>' from the lowest position, so ties and NaN keys go to the lower one).
// The draw is returned as ranks: rank_j = k for the position drawn in round k
// (k < N); every position not drawn has a rank >= N.
// gtab: the noise coefficient table in LDS.
// ---------------------------------------------------------------------------

// For keys that are neither NaN nor infinite the rounds order the positions
// by key, larger first and equal keys lower position first, so
//   rank_j = #{l < j : key_l >= key_j} + #{l > j : key_l > key_j}.
// Every pair l < j contributes one sign bit, that of key_l - key_j, set
// exactly when key_j > key_l (the keys have -0 turned into +0 first, so equal
// keys differ by +0): then j goes before l.  Three dual-issue instructions per
// pair instead of a compare and selects per position and round.  Returns
// false if some key is NaN or infinite (the caller then runs the rounds).
template <int M>
__device__ __forceinline__ bool ranks_by_key(const float (&key)[M], uint32_t (&rank)[M]) {
    float k[M];
    float probe = 0.0f;
#pragma unroll
    for (int j = 0; j < M; ++j) {
        k[j] = key[j] + 0.0f;
        probe = __builtin_fmaf(k[j], 0.0f, probe);  // NaN iff some key is NaN or infinite
    }
    uint32_t after[M], before[M];
#pragma unroll
    for (int j = 0; j < M; ++j) after[j] = before[j] = 0u;
#pragma unroll
    for (int j = 1; j < M; ++j) {
#pragma unroll
        for (int l = 0; l < j; ++l) {
            const uint32_t g = f32_to_bits(k[l] - k[j]) >> 31;  // key_j > key_l
            after[j] += g;   // l that j goes before, among l < j
            before[l] += g;  // j that go before l, among j > l
        }
    }
#pragma unroll
    for (int j = 0; j < M; ++j) rank[j] = static_cast<uint32_t>(j) - after[j] + before[j];
    return probe == 0.0f;
}

// The rounds themselves: ord[k] is the position drawn in round k.
template <int N, int M>
__device__ __forceinline__ void draw_rounds(const float (&key)[M], uint32_t (&rank)[M]) {
    int ord[N];
    uint32_t taken = 0;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        int best = -1;
        float bv = 0.0f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const bool take = !((taken >> j) & 1u) && (best < 0 || key[j] > bv);
            best = take ? j : best;
            bv = take ? key[j] : bv;
        }
        ord[k] = best;
        taken |= 1u << best;
    }
#pragma unroll
    for (int j = 0; j < M; ++j) {
        uint32_t r = N;
#pragma unroll
        for (int k = 0; k < N; ++k) r = (ord[k] == j) ? static_cast<uint32_t>(k) : r;
        rank[j] = r;
    }
}

// Returns the packed set of drawn positions (bit j = position j drawn).
template <int N, int M>
__device__ __forceinline__ uint32_t draw(const float (&p)[M], uint64_t gb, const MpArgs &a,
                                         const float4 *gtab, uint32_t (&rank)[M]) {
    float key[M];
    if (a.no_noise) {
#pragma unroll
        for (int j = 0; j < M; ++j) key[j] = p[j];
    } else {
        uint32_t wd[M];
        stream_words<M, 0>(gb * static_cast<uint64_t>(M / 4), a.step, a.tensor_id, a.k0, a.k1,
                           wd);
#pragma unroll
        for (int j = 0; j < M; ++j) key[j] = p[j] + gumbel_lds(wd[j], gtab);
    }
    if (!ranks_by_key<M>(key, rank)) draw_rounds<N, M>(key, rank);
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) taken |= (rank[j] < static_cast<uint32_t>(N) ? 1u : 0u) << j;
    return taken;
}

// Draw order packed kBits per round, round 0 lowest.
template <int N, int M>
__device__ __forceinline__ uint32_t pack_order(const uint32_t (&rank)[M]) {
    constexpr uint32_t kBits = (M == 4) ? 2 : 3;
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < M; ++j)
        v |= rank[j] < static_cast<uint32_t>(N) ? static_cast<uint32_t>(j) << (kBits * rank[j]) : 0u;
    return v;
}

// ---------------------------------------------------------------------------
// Forward: draw, masked weights, packed mask and draw order.
// ---------------------------------------------------------------------------
template <int N, int M, typename WT, typename OT>
__global__ __launch_bounds__(kThreads) void mp_fwd_kernel(MpArgs a) {
    __shared__ float4 gtab[kGumbelRows];
    load_gumbel_table<kThreads>(gtab);
    __syncthreads();
    // grid-stride over workgroup-sized spans of blocks (the span base is
    // uniform, so every lane of a wave reaches the cross-lane swap below)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads; base < a.nblocks;
         base += stride) {
        const int64_t b = base + threadIdx.x;
        const bool live = b < a.nblocks;
        uint32_t keep = 0;
        if (live) {
            float p[M];
            BlockIo<float, M>::load(a.pi, b, p);
            uint32_t rank[M];
            keep = draw<N, M>(p, a.block_offset + static_cast<uint64_t>(b), a, gtab, rank);
            if (a.out) {
                uint32_t r[M], o[M];
                BlockIo<WT, M>::load_raw(a.w, b, r);
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    const uint32_t v = (sizeof(OT) == 2) ? Elem<WT>::to_bf16(r[j])
                                                         : Elem<WT>::to_f32(r[j]);
                    o[j] = ((keep >> j) & 1u) ? v : 0u;
                }
                BlockIo<OT, M>::store_raw(a.out, b, o);
            }
            if (a.order) {
                if (M == 4)
                    static_cast<uint8_t *>(a.order)[b] = static_cast<uint8_t>(pack_order<N, M>(rank));
                else
                    static_cast<uint16_t *>(a.order)[b] =
                        static_cast<uint16_t>(pack_order<N, M>(rank));
            }
        }
        if (a.bits) {
            if (M == 8) {
                if (live) a.bits[b] = static_cast<uint8_t>(keep);
            } else {
                // two 4-bit masks per byte: the even lane of each pair stores both
                // (every lane of the wave reaches the shuffle; dead lanes give 0)
                const uint32_t hi = __shfl_xor(keep, 1);
                if (live && !(b & 1)) a.bits[b >> 1] = static_cast<uint8_t>(keep | (hi << 4));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Policy gradient of the ordered draw.  Round k (k = 1..N) runs over the
// positions not yet drawn, whose logits q_l are the inputs while drawn ones
// are set to -inf (exp then gives exactly 0, so no per-position select):
//   mx = max_l q_l,  e_l = exp(q_l - mx),  Z = sum e_l (in [1, M]),
//   acc_l -= e_l / Z  for every position,
// then the drawn position's logit becomes -inf.  Forming each round against
// its own largest open logit keeps the dominant terms accurate whatever the
// spread of the block.  Finally every drawn position gets its +1 (the
// derivative of pi_{j_k}); the cancellation in 1 - e/Z is an absolute error
// of one ulp of 1.  dpi = A * acc (+ dpi when accumulating).
// ---------------------------------------------------------------------------
template <int N, int M, bool ORDER_IN>
__device__ __forceinline__ void mp_bwd_block(const MpArgs &a, int64_t b, const float4 *gtab) {
    float q[M];
    BlockIo<float, M>::load(a.pi, b, q);
    // the position closed after round k: ord[k] from the saved order, or the
    // one of rank k from the draw
    int ord[N];
    uint32_t rank[M];
    if (ORDER_IN) {
        constexpr int kBits = (M == 4) ? 2 : 3;
        const uint32_t v = (M == 4) ? static_cast<const uint8_t *>(a.order_in)[b]
                                    : static_cast<const uint16_t *>(a.order_in)[b];
#pragma unroll
        for (int k = 0; k < N; ++k) ord[k] = (v >> (kBits * k)) & ((1u << kBits) - 1u);
    } else {
        draw<N, M>(q, a.block_offset + static_cast<uint64_t>(b), a, gtab, rank);
    }
    float acc[M];
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        float mx = q[0];
#pragma unroll
        for (int l = 1; l < M; ++l) mx = __builtin_fmaxf(mx, q[l]);
        // e_l = 2^((q_l - mx) log2 e) as one fused multiply-add per position:
        // the rounding of the shared offset scales every e_l alike and cancels
        // in e_l / Z
        const float off = -mx * 1.44269504088896341f;
        float e[M];
        float z = 0.0f;
#pragma unroll
        for (int l = 0; l < M; ++l) {
            e[l] = __builtin_amdgcn_exp2f(__builtin_fmaf(q[l], 1.44269504088896341f, off));
            z += e[l];
        }
        const float inv = __builtin_amdgcn_rcpf(z);
#pragma unroll
        for (int l = 0; l < M; ++l) acc[l] = __builtin_fmaf(-e[l], inv, acc[l]);
        if (k + 1 < N) {
#pragma unroll
            for (int l = 0; l < M; ++l) {
                const bool closed = ORDER_IN ? l == ord[k] : rank[l] == static_cast<uint32_t>(k);
                q[l] = closed ? -__builtin_huge_valf() : q[l];
            }
        }
    }
#pragma unroll
    for (int l = 0; l < M; ++l) {
        bool drawn;
        if (ORDER_IN) {
            drawn = false;
#pragma unroll
            for (int k = 0; k < N; ++k) drawn = drawn || l == ord[k];
        } else {
            drawn = rank[l] < static_cast<uint32_t>(N);
        }
        acc[l] += drawn ? 1.0f : 0.0f;
    }
    float d[M];
    if (a.accumulate) {
        BlockIo<float, M>::load(a.dpi, b, d);
#pragma unroll
        for (int j = 0; j < M; ++j) d[j] = d[j] + a.adv * acc[j];
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) d[j] = a.adv * acc[j];
    }
    BlockIo<float, M>::store(a.dpi, b, d);
}

template <int N, int M, bool ORDER_IN>
__global__ __launch_bounds__(kThreads) void mp_bwd_kernel(MpArgs a) {
    __shared__ float4 gtab[ORDER_IN ? 1 : kGumbelRows];
    if constexpr (!ORDER_IN) {
        load_gumbel_table<kThreads>(gtab);
        __syncthreads();
    }
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < a.nblocks;
         b += stride)
        mp_bwd_block<N, M, ORDER_IN>(a, b, gtab);
}

// ---------------------------------------------------------------------------
// Initial logits: c at the kept positions of the initial mask, 0 elsewhere.
// The mask is the packed prior (LSB-first, M bits per block) or the magnitude
// top-N of w (N rounds of "first largest |w| not yet kept").
// ---------------------------------------------------------------------------
template <int N, int M, typename WT>
__device__ __forceinline__ void mp_init_block(const MpInitArgs &a, int64_t b) {
    uint32_t keep = 0;
    if (a.prior_bits) {
        if (M == 8)
            keep = a.prior_bits[b];
        else
            keep = (a.prior_bits[b >> 1] >> (4 * (b & 1))) & 0xFu;
    } else {
        uint32_t r[M], mag[M];
        BlockIo<WT, M>::load_raw(a.w, b, r);
#pragma unroll
        for (int j = 0; j < M; ++j) mag[j] = Elem<WT>::magnitude(r[j]);
#pragma unroll
        for (int k = 0; k < N; ++k) {
            int best = -1;
            uint32_t bv = 0;
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const bool take = !((keep >> j) & 1u) && (best < 0 || mag[j] > bv);
                best = take ? j : best;
                bv = take ? mag[j] : bv;
            }
            keep |= 1u << best;
        }
    }
    float v[M];
#pragma unroll
    for (int j = 0; j < M; ++j) v[j] = ((keep >> j) & 1u) ? a.c : 0.0f;
    BlockIo<float, M>::store(a.pi, b, v);
}

template <int N, int M, typename WT>
__global__ __launch_bounds__(kThreads) void mp_init_kernel(MpInitArgs a) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < a.nblocks;
         b += stride)
        mp_init_block<N, M, WT>(a, b);
}

// One thread per block up to 2^20 workgroups (5.4e8 blocks); larger tensors
// loop, which keeps the grid inside its 32-bit dimension.
unsigned blocks_for(int64_t nblocks) {
    const int64_t want = (nblocks + kThreads - 1) / kThreads;
    return static_cast<unsigned>(want < (INT64_C(1) << 20) ? want : (INT64_C(1) << 20));
}

// The kernels that draw noise first copy the 24 KB coefficient table into
// LDS, so their grids stop at the workgroups that fit the CUs at once (three
// of 512 lanes per CU by registers) and loop over the rest: the table is read
// once per resident workgroup instead of once per 512 blocks.
constexpr int kNoiseWgPerCU = 3;
unsigned noise_blocks_for(int64_t nblocks) {
    const int64_t want = (nblocks + kThreads - 1) / kThreads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * kNoiseWgPerCU;
    const int64_t g = want < cap ? want : cap;
    return static_cast<unsigned>(g < 1 ? 1 : g);
}

template <int N, int M, typename WT>
hipError_t fwd_out(const MpArgs &a, maskgs_dtype out_dt, hipStream_t s) {
    if (out_dt == MASKGS_BF16)
        hipLaunchKernelGGL((mp_fwd_kernel<N, M, WT, bf16_t>), dim3(noise_blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mp_fwd_kernel<N, M, WT, float>), dim3(noise_blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int N, int M>
hipError_t fwd_nm(const MpArgs &a, maskgs_dtype w_dt, maskgs_dtype out_dt, hipStream_t s) {
    if (w_dt == MASKGS_F32) return fwd_out<N, M, float>(a, out_dt, s);
    return fwd_out<N, M, bf16_t>(a, out_dt, s);
}

template <int N, int M>
hipError_t bwd_nm(const MpArgs &a, hipStream_t s) {
    if (a.order_in)
        hipLaunchKernelGGL((mp_bwd_kernel<N, M, true>), dim3(blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mp_bwd_kernel<N, M, false>), dim3(noise_blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int N, int M>
hipError_t init_nm(const MpInitArgs &a, maskgs_dtype w_dt, hipStream_t s) {
    if (a.prior_bits || w_dt == MASKGS_BF16)
        hipLaunchKernelGGL((mp_init_kernel<N, M, bf16_t>), dim3(blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mp_init_kernel<N, M, float>), dim3(blocks_for(a.nblocks)),
                           dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mp_fwd(const MpArgs &a, int m, maskgs_dtype w_dt, maskgs_dtype out_dt,
                         hipStream_t s) {
    // without an output the weight type is irrelevant: use one instantiation
    if (!a.out) w_dt = out_dt = MASKGS_BF16;
    return m == 4 ? fwd_nm<2, 4>(a, w_dt, out_dt, s) : fwd_nm<4, 8>(a, w_dt, out_dt, s);
}

hipError_t launch_mp_bwd(const MpArgs &a, int m, hipStream_t s) {
    return m == 4 ? bwd_nm<2, 4>(a, s) : bwd_nm<4, 8>(a, s);
}

hipError_t launch_mp_init(const MpInitArgs &a, int m, maskgs_dtype w_dt, hipStream_t s) {
    return m == 4 ? init_nm<2, 4>(a, w_dt, s) : init_nm<4, 8>(a, w_dt, s);
}

}  // namespace maskgs
