// maskgs_k24.hip -- 2:4 kernels of libmaskgs for gfx950.
//
// Work item = one pair of consecutive blocks (2p, 2p+1) handled by one lane:
//   weights   8 bf16 = one 16 B load (fp32: two),   logits 12 fp32 = three 16 B loads,
//   and the pair's 12 noise words come from 3 Philox calls when the pair starts
//   at an even global block (4 calls otherwise; PHASE is uniform per launch).
// A workgroup walks tiles of kThreads consecutive pairs (grid-stride, the same
// trip count for every lane).  Inputs are read directly (lanes 48 B apart,
// three 16 B loads each), and the pair's noise, which depends only on the
// counters, is drawn while those loads are in flight; 48-byte-per-lane outputs
// (soft index, logit gradient, seeded logits) are transposed through LDS so
// that every global store is a fully coalesced, non-temporal 16 B-per-lane
// stream.
// The path is an HBM/VALU streaming path: no matrix cores are involved.
#include <hip/hip_runtime.h>

#include "maskgs_device.hpp"
#include "maskgs_launch.hpp"

namespace maskgs {
namespace {

#ifndef MASKGS_K24_THREADS
#define MASKGS_K24_THREADS 512
#endif
constexpr int kThreads = MASKGS_K24_THREADS;
#ifndef MASKGS_K24_WG_PER_CU
#define MASKGS_K24_WG_PER_CU 8
#endif
constexpr int kWgPerCU = MASKGS_K24_WG_PER_CU;  // grid cap: workgroups of kThreads lanes per CU
// The cap of the kernels without noise or end-of-workgroup atomics (hard
// extract, prior seeding, the backward fused with AdamW): a grid well past the
// resident set keeps each workgroup's share, and so the launch's tail, short.
// Measured on the 7B sweep against the cap of 8: hard extract 11.4 -> 10.7 ms,
// prior seeding 16.8 -> 15.8 ms, training backward 46.8 -> 45.6 ms; the
// 512-lane forward and backward measured best at 8 (the step's two kernels
// use the shapes below).
constexpr int kWgPerCUStream = 64;
// Lanes per workgroup and grid cap of the backward that draws the soft index
// again (without the fused update): 1024-lane workgroups, one resident per CU
// (72 KB of LDS, 75 registers), took the 7B step's backward phase from 18.8
// to 18.3 ms against 512-lane ones (grid caps of 2, 4 and 8 per CU within
// 0.5% of each other).
constexpr int kBwdRcThreads = 1024;
constexpr int kBwdRcWgPerCU = 4;
// The same for the forward that saves no soft index (the step's forward):
// 768-lane workgroups, 2 per CU, both resident (24 waves), 13.51 -> 13.31 ms
// over the 7B step's forward phase in three alternating runs against 512
// lanes and 8 per CU (256 lanes and 8 per CU: 13.38; 384 and 1024 lanes:
// 14.3-14.4).
constexpr int kFwdNoYThreads = 768;
constexpr int kFwdNoYWgPerCU = 2;
using C24 = Cands<2, 4>;

// ---------------------------------------------------------------------------
// Pair loads and stores.  `two` is false only for the last pair of an odd
// block count; then only block 2p exists and only its bytes are touched.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack_bf16x2(uint32_t v, float &lo, float &hi) {
    lo = __uint_as_float(v << 16);
    hi = __uint_as_float(v & 0xFFFF0000u);
}

// Selects among four register values without indexing an array (which would
// place the array in scratch memory).
__device__ __forceinline__ uint32_t pick4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                          uint32_t pos) {
    return pos == 0 ? r0 : pos == 1 ? r1 : pos == 2 ? r2 : r3;
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <typename T>
struct Io;

template <>
struct Io<bf16_t> {
    static __device__ __forceinline__ void load8(const void *base, int64_t p, bool two,
                                                 float (&v)[8]) {
        const uint16_t *ptr = static_cast<const uint16_t *>(base) + p * 8;
        if (two) {
            const uint4 u = *reinterpret_cast<const uint4 *>(ptr);
            unpack_bf16x2(u.x, v[0], v[1]);
            unpack_bf16x2(u.y, v[2], v[3]);
            unpack_bf16x2(u.z, v[4], v[5]);
            unpack_bf16x2(u.w, v[6], v[7]);
        } else {
            const uint2 u = *reinterpret_cast<const uint2 *>(ptr);
            unpack_bf16x2(u.x, v[0], v[1]);
            unpack_bf16x2(u.y, v[2], v[3]);
            v[4] = v[5] = v[6] = v[7] = 0.0f;
        }
    }
    // load8 that also keeps the words as loaded: d[0..3] hold the pair's bf16
    // values two per word (d[4..7] unused)
    static __device__ __forceinline__ void load8(const void *base, int64_t p, bool two,
                                                 float (&v)[8], uint32_t (&d)[8]) {
        const uint16_t *ptr = static_cast<const uint16_t *>(base) + p * 8;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (two) {
            u = *reinterpret_cast<const uint4 *>(ptr);
        } else {
            const uint2 h = *reinterpret_cast<const uint2 *>(ptr);
            u.x = h.x;
            u.y = h.y;
        }
        unpack_bf16x2(u.x, v[0], v[1]);
        unpack_bf16x2(u.y, v[2], v[3]);
        unpack_bf16x2(u.z, v[4], v[5]);
        unpack_bf16x2(u.w, v[6], v[7]);
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
        d[4] = d[5] = d[6] = d[7] = 0u;
    }
    // raw bit patterns, widened to 32 bits (one per position)
    static __device__ __forceinline__ void load8_raw(const void *base, int64_t p, bool two,
                                                     uint32_t (&r)[8]) {
        uint32_t d[8];
        load8_words(base, p, two, d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[2 * i] = d[i] & 0xFFFFu;
            r[2 * i + 1] = d[i] >> 16;
        }
    }
    // the words as loaded (the form load8 keeps), for the hard-mask pass
    static __device__ __forceinline__ void load8_words(const void *base, int64_t p, bool two,
                                                       uint32_t (&d)[8]) {
        const uint16_t *ptr = static_cast<const uint16_t *>(base) + p * 8;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (two) {
            u = *reinterpret_cast<const uint4 *>(ptr);
        } else {
            const uint2 h = *reinterpret_cast<const uint2 *>(ptr);
            u.x = h.x;
            u.y = h.y;
        }
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
        d[4] = d[5] = d[6] = d[7] = 0u;
    }
    static __device__ __forceinline__ uint32_t magnitude(uint32_t raw) { return raw & 0x7FFFu; }
    // |w| ordering keys (sign cleared) of the 8 positions, from the loaded words
    static __device__ __forceinline__ void mags8(const uint32_t (&d)[8], uint32_t (&mag)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mag[2 * i] = d[i] & 0x7FFFu;
            mag[2 * i + 1] = (d[i] >> 16) & 0x7FFFu;
        }
    }
    static __device__ __forceinline__ void store8(void *base, int64_t p, bool two,
                                                  const float (&v)[8]) {
        uint16_t *ptr = static_cast<uint16_t *>(base) + p * 8;
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = static_cast<uint32_t>(bf16_rne(v[2 * i])) |
                   (static_cast<uint32_t>(bf16_rne(v[2 * i + 1])) << 16);
        if (two)
            __builtin_nontemporal_store(v4u{u[0], u[1], u[2], u[3]}, reinterpret_cast<v4u *>(ptr));
        else
            *reinterpret_cast<uint2 *>(ptr) = make_uint2(u[0], u[1]);
    }
    // The 2 kept values of each block (positions lo < hi, given as the nibble
    // lo | hi << 2) in ascending position, from the words as loaded: one
    // byte permute per block picks bytes 2lo, 2lo+1, 2hi, 2hi+1 of its two
    // words, so the output word is w_lo | w_hi << 16.
    static __device__ __forceinline__ void store_values(void *base, int64_t p, bool two,
                                                        const uint32_t (&d)[8], uint32_t lohi0,
                                                        uint32_t lohi1) {
        uint16_t *ptr = static_cast<uint16_t *>(base) + p * 4;
        const uint32_t s0 = 0x01000100u + (lohi0 & 3u) * 0x0202u + (lohi0 >> 2) * 0x02020000u;
        const uint32_t a = __builtin_amdgcn_perm(d[1], d[0], s0);
        if (two) {
            const uint32_t s1 = 0x01000100u + (lohi1 & 3u) * 0x0202u + (lohi1 >> 2) * 0x02020000u;
            *reinterpret_cast<uint2 *>(ptr) = make_uint2(a, __builtin_amdgcn_perm(d[3], d[2], s1));
        } else {
            *reinterpret_cast<uint32_t *>(ptr) = a;
        }
    }
};

template <>
struct Io<float> {
    static __device__ __forceinline__ void load8(const void *base, int64_t p, bool two,
                                                 float (&v)[8]) {
        const float *ptr = static_cast<const float *>(base) + p * 8;
        const float4 a = *reinterpret_cast<const float4 *>(ptr);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        if (two) {
            const float4 b = *reinterpret_cast<const float4 *>(ptr + 4);
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            v[4] = v[5] = v[6] = v[7] = 0.0f;
        }
    }
    static __device__ __forceinline__ void load8_raw(const void *base, int64_t p, bool two,
                                                     uint32_t (&r)[8]) {
        float v[8];
        load8(base, p, two, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __float_as_uint(v[i]);
    }
    static __device__ __forceinline__ void load8_words(const void *base, int64_t p, bool two,
                                                       uint32_t (&d)[8]) {
        load8_raw(base, p, two, d);
    }
    static __device__ __forceinline__ void load8(const void *base, int64_t p, bool two,
                                                 float (&v)[8], uint32_t (&d)[8]) {
        load8(base, p, two, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = __float_as_uint(v[i]);
    }
    static __device__ __forceinline__ uint32_t magnitude(uint32_t raw) {
        return raw & 0x7FFFFFFFu;
    }
    static __device__ __forceinline__ void mags8(const uint32_t (&d)[8], uint32_t (&mag)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) mag[i] = d[i] & 0x7FFFFFFFu;
    }
    static __device__ __forceinline__ void store8(void *base, int64_t p, bool two,
                                                  const float (&v)[8]) {
        float *ptr = static_cast<float *>(base) + p * 8;
        *reinterpret_cast<float4 *>(ptr) = make_float4(v[0], v[1], v[2], v[3]);
        if (two) *reinterpret_cast<float4 *>(ptr + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    // The 2 kept values of each block (nibble lo | hi << 2), ascending.
    static __device__ __forceinline__ void store_values(void *base, int64_t p, bool two,
                                                        const uint32_t (&d)[8], uint32_t lohi0,
                                                        uint32_t lohi1) {
        uint32_t *ptr = static_cast<uint32_t *>(base) + p * 4;
        const uint32_t a = pick4(d[0], d[1], d[2], d[3], lohi0 & 3u);
        const uint32_t b = pick4(d[0], d[1], d[2], d[3], lohi0 >> 2);
        if (two)
            *reinterpret_cast<uint4 *>(ptr) =
                make_uint4(a, b, pick4(d[4], d[5], d[6], d[7], lohi1 & 3u),
                           pick4(d[4], d[5], d[6], d[7], lohi1 >> 2));
        else
            *reinterpret_cast<uint2 *>(ptr) = make_uint2(a, b);
    }
};

// 12 fp32 per pair ([2, 6] logits, soft indices or logit gradients)
__device__ __forceinline__ void load12(const float *base, int64_t p, bool two, float (&v)[12]) {
    const float *ptr = base + p * 12;
    const float4 a = *reinterpret_cast<const float4 *>(ptr);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    if (two) {
        const float4 b = *reinterpret_cast<const float4 *>(ptr + 4);
        const float4 c = *reinterpret_cast<const float4 *>(ptr + 8);
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        v[8] = c.x; v[9] = c.y; v[10] = c.z; v[11] = c.w;
    } else {
        const float2 b = *reinterpret_cast<const float2 *>(ptr + 4);
        v[4] = b.x; v[5] = b.y;
        v[6] = v[7] = v[8] = v[9] = v[10] = v[11] = 0.0f;
    }
}

__device__ __forceinline__ void nt_store(float4 *p, float4 v) {
    __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f *>(p));
}

// Writes a lane's 12 values to its slot of the LDS tile (pair order).
__device__ __forceinline__ void stage12(const float (&v)[12], float4 *lds) {
    const int t = threadIdx.x;
    lds[3 * t] = make_float4(v[0], v[1], v[2], v[3]);
    lds[3 * t + 1] = make_float4(v[4], v[5], v[6], v[7]);
    lds[3 * t + 2] = make_float4(v[8], v[9], v[10], v[11]);
}

// Stores 12 floats per lane for the pairs [base, base + kThreads) of the
// workgroup with coalesced 16 B stores, through LDS.  The 64 pairs of one wave
// are one contiguous 3 KB span of the output and its own slice of the LDS
// tile, so each wave transposes and stores its span alone: a wave's LDS
// operations complete in order, and no workgroup barrier holds the other waves
// (measured 2-9% faster than a workgroup-wide transpose in the forward and
// backward).  Called by every lane of the wave.
__device__ __forceinline__ void store12_wave(float *g, int64_t base, int64_t nblocks,
                                             const float (&v)[12], float4 *lds) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    stage12(v, lds);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t wbase = base + 64 * wv;  // first pair of this wave
    const int64_t end = 2 * (wbase + 64) < nblocks ? 2 * (wbase + 64) : nblocks;
    const int nf = end > 2 * wbase ? static_cast<int>((end - 2 * wbase) * 6) : 0;
    const int n4 = nf >> 2;
    float4 *dst = reinterpret_cast<float4 *>(g + wbase * 12);
    const float4 *src = lds + 3 * 64 * wv;
    for (int i = lane; i < n4; i += 64) nt_store(dst + i, src[i]);
    if ((nf & 3) && lane == 0)
        reinterpret_cast<float2 *>(dst)[2 * n4] = reinterpret_cast<const float2 *>(src)[2 * n4];
    // the next stage12 of this wave must not overtake these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same store with a workgroup-wide transpose (two barriers); prior seeding,
// which rewrites the logits it has just read, measured faster with it.
__device__ __forceinline__ void store12_tile(float *g, int64_t base, int64_t nblocks,
                                             const float (&v)[12], float4 *lds) {
    const int t = threadIdx.x;
    stage12(v, lds);
    __syncthreads();
    const int64_t end = 2 * (base + kThreads) < nblocks ? 2 * (base + kThreads) : nblocks;
    const int nf = static_cast<int>((end - 2 * base) * 6);
    const int n4 = nf >> 2;
    float4 *dst = reinterpret_cast<float4 *>(g + base * 12);
    for (int i = t; i < n4; i += kThreads) nt_store(dst + i, lds[i]);
    if ((nf & 3) && t == 0)
        reinterpret_cast<float2 *>(dst)[2 * n4] = reinterpret_cast<const float2 *>(lds)[2 * n4];
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Sampling (MaskLLM summary, section 3.4, Eqs. 5-7, Algorithm 1).
// ---------------------------------------------------------------------------
// Noise words of the pair starting at global block gb0 (PHASE = (6*gb0) % 4).
template <int PHASE>
__device__ __forceinline__ void pair_words(const Geometry &g, const Noise &nz, int64_t p,
                                           uint32_t (&wd)[12]) {
    const uint64_t gb0 = g.block_offset + 2 * static_cast<uint64_t>(p);
    stream_words<12, PHASE>((gb0 * 6u) >> 2, nz.step, g.tensor_id, nz.k0, nz.k1, wd);
}

// Soft index of one block from its perturbed logits: y = softmax(a) in fp32
// (max-shifted, hardware exp2 and reciprocal).  The exponentials are taken
// 2^64 too large, so that terms down to 2^-190 stay normal through the exp2
// (which flushes subnormal results); the product with the reciprocal of the
// (equally scaled) sum then rounds small soft-index values, subnormal ones
// included, correctly.
__device__ __forceinline__ void softmax6(const float *a, float *y) {
    float e[6];
    float amax = a[0];
#pragma unroll
    for (int i = 1; i < 6; ++i) amax = fmaxf(amax, a[i]);
    // exponent (a_i - amax) log2(e) + 64 as one fused multiply-add per
    // candidate: the rounding of the shared offset scales every exponential
    // alike and cancels in the normalisation
    const float off = __builtin_fmaf(-amax, 1.44269504088896341f, 64.0f);
#pragma unroll
    for (int i = 0; i < 6; ++i)
        e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(a[i], 1.44269504088896341f, off));
    const float s = ((e[0] + e[1]) + (e[2] + e[3])) + (e[4] + e[5]);
    const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < 6; ++i) y[i] = e[i] * inv;
}

// Soft mask m_j = sum_i y_i S_ij (Eq. 7), candidates in table order.
__device__ __forceinline__ void soft_mask4(const float *y, float *m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = 0.0f;
        bool first = true;
#pragma unroll
        for (int i = 0; i < 6; ++i)
            if ((C24::mask[i] >> j) & 1u) {
                s = first ? y[i] : s + y[i];
                first = false;
            }
        m[j] = s;
    }
}

// Hard mask (section 3.2 inference flow; Algorithm 1 step 3): first index of
// the largest logit, its candidate mask, kept positions and values.
__device__ __forceinline__ int first_argmax6(const float *z) {
    int best = 0;
    float bv = z[0];
#pragma unroll
    for (int i = 1; i < 6; ++i)
        if (z[i] > bv) {
            bv = z[i];
            best = i;
        }
    return best;
}

// The six candidate masks packed as nibbles (nibble i = mask i), so that a
// runtime candidate index selects its mask with one shift.
constexpr uint32_t pack_nibbles24() {
    uint32_t v = 0;
    for (int i = 0; i < 6; ++i) v |= static_cast<uint32_t>(C24::mask[i]) << (4 * i);
    return v;
}
constexpr uint32_t kMaskNibbles24 = pack_nibbles24();

__device__ __forceinline__ uint32_t cand_mask6(int k) { return (kMaskNibbles24 >> (4 * k)) & 0xFu; }

// The kept positions lo < hi of each candidate as the nibble lo | hi << 2 (the
// 2-bit index format), packed like kMaskNibbles24.
constexpr uint32_t pack_lohi24() {
    uint32_t v = 0;
    for (int i = 0; i < 6; ++i) {
        int lo = -1, hi = -1;
        for (int j = 0; j < 4; ++j)
            if ((C24::mask[i] >> j) & 1u) {
                if (lo < 0)
                    lo = j;
                else
                    hi = j;
            }
        v |= static_cast<uint32_t>(lo | (hi << 2)) << (4 * i);
    }
    return v;
}
constexpr uint32_t kLoHi24 = pack_lohi24();
static_assert(kLoHi24 == 0xE9DC84u, "kept positions of the page-order 2:4 candidates");

__device__ __forceinline__ uint32_t cand_lohi6(int k) { return (kLoHi24 >> (4 * k)) & 0xFu; }

// Hard mask of one pair from its logits z and the pair's weight words d (as
// Io<WT>::load8_words gives them; read only when values are requested).
template <typename WT>
__device__ __forceinline__ void hard_pair(uint8_t *idx, uint8_t *bits, void *values,
                                          uint8_t *val_idx, int64_t p, bool two,
                                          const float (&z)[12], const uint32_t (&d)[8]) {
    const int k0 = first_argmax6(z), k1 = first_argmax6(z + 6);
    const uint32_t m0 = cand_mask6(k0), m1 = two ? cand_mask6(k1) : 0u;
    if (idx) {
        if (two)
            *reinterpret_cast<uint16_t *>(idx + 2 * p) = static_cast<uint16_t>(k0 | (k1 << 8));
        else
            idx[2 * p] = static_cast<uint8_t>(k0);
    }
    if (bits) bits[p] = static_cast<uint8_t>(m0 | (m1 << 4));
    const uint32_t lh0 = cand_lohi6(k0), lh1 = two ? cand_lohi6(k1) : 0u;
    if (val_idx) val_idx[p] = static_cast<uint8_t>(lh0 | (lh1 << 4));
    if (values) Io<WT>::store_values(values, p, two, d, lh0, lh1);
}

// Gumbel noise of a pair (section 3.4, Eq. 5): g_i of the contract for its
// twelve candidates from the contract's coefficient table in LDS (gtab), +0
// with the noise switched off.  It depends only on the counters, so the
// kernels draw it right after requesting the pair's loads and the memory
// latency passes under the noise arithmetic.  The noise flag is uniform, so
// the twelve Gumbel evaluations form one straight-line block the scheduler can
// interleave.
template <int PHASE>
__device__ __forceinline__ void pair_noise(const Geometry &g, const Noise &nz, int64_t p,
                                           const float4 *gtab, float (&g12)[12]) {
    if (nz.no_noise) {
#pragma unroll
        for (int i = 0; i < 12; ++i) g12[i] = 0.0f;
    } else {
        uint32_t wd[12];
        pair_words<PHASE>(g, nz, p, wd);
#pragma unroll
        for (int i = 0; i < 12; ++i) g12[i] = gumbel_lds(wd[i], gtab);
    }
}

// Perturbed logits of a pair (section 3.4, Eq. 6 and Algorithm 1 steps 1-2):
// a_i = fp32(fp32(kappa z_i + g_i) * fp32(1/tau)).
__device__ __forceinline__ void pair_logits(const Noise &nz, const float (&z)[12],
                                            const float (&g12)[12], float (&a12)[12]) {
    // kappa and 1/tau in vector registers: an instruction that reads a scalar
    // register does not dual-issue
    float kappa = nz.kappa, tau_inv = nz.tau_inv;
    asm volatile("" : "+v"(kappa), "+v"(tau_inv));
#pragma unroll
    for (int i = 0; i < 12; ++i) a12[i] = __builtin_fmaf(kappa, z[i], g12[i]) * tau_inv;
}

// Soft index of a pair from its logits and noise and, under the hard-sample
// flag, the masks of its two Gumbel-max samples S[first argmax a] (0
// otherwise).
// need_y false skips the soft index under the hard sample (a forward that
// applies the sample and saves no soft index has no use for it).
__device__ __forceinline__ void pair_sample(const Noise &nz, const float (&z)[12],
                                            const float (&g12)[12], float (&y)[12],
                                            uint32_t (&hm)[2], bool need_y = true) {
    float a12[12];
    pair_logits(nz, z, g12, a12);
    hm[0] = hm[1] = 0u;
    if (nz.hard_sample) {
        hm[0] = cand_mask6(first_argmax6(a12));
        hm[1] = cand_mask6(first_argmax6(a12 + 6));
        if (!need_y) return;
    }
    softmax6(a12, y);
    softmax6(a12 + 6, y + 6);
}

// The mask the forward applies to a block: the soft mask y.S (Eq. 7), or the
// hard sample's 0/1 mask.
__device__ __forceinline__ void applied_mask4(const float *y6, uint32_t hm, bool hard,
                                              float (&m)[4]) {
    if (hard) {
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = ((hm >> j) & 1u) ? 1.0f : 0.0f;
    } else {
        soft_mask4(y6, m);
    }
}

// Workgroup sum of one double per lane, added atomically to *dst.
template <int T = kThreads>
__device__ __forceinline__ void reduce_add(double v, double *dst) {
    __shared__ double part[T / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) part[wid] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < T / 64; ++i) s += part[i];
        atomicAdd(dst, s);
    }
}

// ---------------------------------------------------------------------------
// Forward: W (.) M~, optional soft index and regulariser value.
// ---------------------------------------------------------------------------
template <int PHASE, typename WT, typename OT, bool YSAVE, int T>
__global__ __launch_bounds__(T) void fwd24_kernel(FwdArgs a) {
    __shared__ float4 stage[YSAVE ? 3 * T : 1];
    __shared__ float4 gtab[kGumbelRows];
    load_gumbel_table<T>(gtab);
    __syncthreads();
    const bool hard = a.idx || a.bits || a.values || a.val_idx;
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * T;
    double reg = 0.0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * T; base < npairs;
         base += stride) {
        const int64_t p = base + threadIdx.x;
        float y[12];
        if (p < npairs) {
            const bool two = 2 * p + 1 < a.g.nblocks;
            float w[8], z[12], out[8];
            uint32_t wd[8];
            Io<WT>::load8(a.w, p, two, w, wd);
            load12(a.z, p, two, z);
            float g12[12];
            pair_noise<PHASE>(a.g, a.nz, p, gtab, g12);
            if (hard) {
                // hard mask of the same logits (argmax of z, not of the sample)
                hard_pair<WT>(a.idx, a.bits, a.values, a.val_idx, p, two, z, wd);
            }
            uint32_t hm[2];
            pair_sample(a.nz, z, g12, y, hm, YSAVE);
            float racc = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float m[4];
                applied_mask4(y + 6 * h, hm[h], a.nz.hard_sample, m);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float u = w[4 * h + j] * m[j];
                    out[4 * h + j] = u;
                    racc = __builtin_fmaf(u, u, racc);
                }
            }
            reg += static_cast<double>(racc);
            Io<OT>::store8(a.out, p, two, out);
        }
        if constexpr (YSAVE) store12_wave(a.y, base, a.g.nblocks, y, stage);
    }
    if (a.reg) reduce_add<T>(reg, a.reg);
}

// ---------------------------------------------------------------------------
// Backward to the logits (section 3.2 information flow; section 3.4 Eq. 8):
//   dm_j = G_j w_j - 2 lambda w_j (w_j m_j),  dy_i = sum_j S_ij dm_j,
//   dz_i = (kappa/tau) y_i (dy_i - sum_k y_k dy_k).
// With m_j = sum of y_k over the candidates that keep position j and mb_j the
// sum over those that drop it, dy_i - sum_k y_k dy_k (for sum_k y_k = 1) is
//   t_i = sum_{j in S_i} mb_j dm_j - sum_{j not in S_i} m_j dm_j,
// four products of fp32 values whose factors mb_j, m_j are small exactly
// where dy_i - sum y dy cancels (the dominant candidate: every y_k but its
// own is small), so t_i is formed in fp32 without that cancellation.
// ---------------------------------------------------------------------------
// mb_j: sum of y_i over the candidates that drop position j.
__device__ __forceinline__ void soft_mask4_complement(const float *y, float *mb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = 0.0f;
        bool first = true;
#pragma unroll
        for (int i = 0; i < 6; ++i)
            if (!((C24::mask[i] >> j) & 1u)) {
                s = first ? y[i] : s + y[i];
                first = false;
            }
        mb[j] = s;
    }
}

template <int PHASE, typename WT, typename GT, bool SAVED, bool ADAMW, int T>
__global__ __launch_bounds__(T) void bwd24_kernel(BwdArgs a) {
    __shared__ float4 stage[3 * T];
    __shared__ float4 gtab[SAVED ? 1 : kGumbelRows];
    if constexpr (!SAVED) {
        load_gumbel_table<T>(gtab);
        __syncthreads();
    }
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * T;
    const float two_lambda = static_cast<float>(2.0 * a.lambda);
    const float gscale = static_cast<float>(a.nz.grad_scale);
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * T; base < npairs;
         base += stride) {
        const int64_t p = base + threadIdx.x;
        float dz[12];
        if (p < npairs) {
            const bool two = 2 * p + 1 < a.g.nblocks;
            float w[8], G[8], y[12];
            uint32_t hm[2] = {0u, 0u};
            Io<WT>::load8(a.w, p, two, w);
            Io<GT>::load8(a.dout, p, two, G);
            if (SAVED) {
                load12(a.y, p, two, y);
            } else {
                float z[12], g12[12];
                load12(a.z, p, two, z);
                pair_noise<PHASE>(a.g, a.nz, p, gtab, g12);
                pair_sample(a.nz, z, g12, y, hm);
            }
            float prev[12];
            if (a.accumulate) load12(a.dz, p, two, prev);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float *yh = y + 6 * h;
                float m[4], mb[4];
                soft_mask4(yh, m);
                soft_mask4_complement(yh, mb);
                // the regulariser term is that of the applied mask (straight-
                // through under the hard sample); the Jacobian is y's
                float ma[4];
                applied_mask4(yh, hm[h], !SAVED && a.nz.hard_sample, ma);
                float pk[4], qd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float wj = w[4 * h + j];
                    const float u = wj * ma[j];
                    const float dm = __builtin_fmaf(G[4 * h + j], wj, -(two_lambda * wj) * u);
                    pk[j] = mb[j] * dm;
                    qd[j] = m[j] * dm;
                }
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    // S_i = {lo, hi}, its complement {c0, c1} (compile-time)
                    int kp[2] = {0, 0}, dp[2] = {0, 0}, nk = 0, nd = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if ((C24::mask[i] >> j) & 1u) kp[nk++] = j;
                        else dp[nd++] = j;
                    }
                    const float t = (pk[kp[0]] + pk[kp[1]]) - (qd[dp[0]] + qd[dp[1]]);
                    const float sy = gscale * yh[i];
                    dz[6 * h + i] = a.accumulate ? __builtin_fmaf(sy, t, prev[6 * h + i]) : sy * t;
                }
            }
        }
        if (ADAMW) {
            // the gradient goes through LDS into the AdamW update of the same
            // logits (coalesced float4 streams of z and both moments); each
            // wave updates its own contiguous span, as in store12_wave
            stage12(dz, stage);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int lane = threadIdx.x & 63;
            const int wv = threadIdx.x >> 6;
            const int64_t wbase = base + 64 * wv;
            const int64_t end = 2 * (wbase + 64) < a.g.nblocks ? 2 * (wbase + 64) : a.g.nblocks;
            const int nf = end > 2 * wbase ? static_cast<int>((end - 2 * wbase) * 6) : 0;
            adamw_span<64, 3 * 64, 3>(a.zu + wbase * 12, a.m1 + wbase * 12, a.m2 + wbase * 12,
                                      reinterpret_cast<const float *>(stage + 3 * 64 * wv), nf,
                                      a.adam, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        } else {
            store12_wave(a.dz, base, a.g.nblocks, dz, stage);
        }
    }
}

// ---------------------------------------------------------------------------
// Regulariser value alone (section 3.4, Eq. 8).
// ---------------------------------------------------------------------------
template <int PHASE, typename WT, bool SAVED>
__global__ __launch_bounds__(kThreads) void reg24_kernel(RegArgs a) {
    __shared__ float4 gtab[SAVED ? 1 : kGumbelRows];
    if constexpr (!SAVED) {
        load_gumbel_table<kThreads>(gtab);
        __syncthreads();
    }
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    double reg = 0.0;
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; p < npairs;
         p += stride) {
        const bool two = 2 * p + 1 < a.g.nblocks;
        float w[8], y[12];
        uint32_t hm[2] = {0u, 0u};
        Io<WT>::load8(a.w, p, two, w);
        if (SAVED) {
            load12(a.y, p, two, y);
        } else {
            float z[12], g12[12];
            load12(a.z, p, two, z);
            pair_noise<PHASE>(a.g, a.nz, p, gtab, g12);
            // the regulariser of a hard sample needs only its mask
            pair_sample(a.nz, z, g12, y, hm, false);
        }
        float racc = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float m[4];
            applied_mask4(y + 6 * h, hm[h], !SAVED && a.nz.hard_sample, m);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float u = w[4 * h + j] * m[j];
                racc = __builtin_fmaf(u, u, racc);
            }
        }
        reg += static_cast<double>(racc);
    }
    reduce_add(reg, a.reg);
}

// ---------------------------------------------------------------------------
// Hard mask: argmax, packed bits, 2:4 values and 2-bit indices (section 3.2
// inference flow; Algorithm 1 step 3), as a pass of its own.
// ---------------------------------------------------------------------------
template <typename WT>
__global__ __launch_bounds__(kThreads) void hard24_kernel(HardArgs a) {
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; p < npairs;
         p += stride) {
        const bool two = 2 * p + 1 < a.g.nblocks;
        // both streams are requested before any use, so their latencies overlap
        float z[12];
        uint32_t r[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        load12(a.z, p, two, z);
        if (a.values) Io<WT>::load8_words(a.w, p, two, r);
        hard_pair<WT>(a.idx, a.bits, a.values, a.val_idx, p, two, z, r);
    }
}

// ---------------------------------------------------------------------------
// Prior seeding (section 3.4, Mask Prior, Eqs. 9-10).
// ---------------------------------------------------------------------------
// Magnitude top-2 of 4 magnitudes: position j is kept when fewer than 2
// positions beat it (larger magnitude, or equal magnitude at a lower position).
__device__ __forceinline__ uint32_t top2_of4(const uint32_t *mag) {
    uint32_t keep = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int beat = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (i != j) beat += (mag[i] > mag[j]) || (mag[i] == mag[j] && i < j);
        if (beat < 2) keep |= 1u << j;
    }
    return keep;
}

__device__ __forceinline__ void prior_block6(float *z, uint32_t m0, double alpha, int mode) {
    int dot[6], dsum = 0;
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        dot[i] = __builtin_popcount(m0 & C24::mask[i]);
        dsum += dot[i];
    }
    if (mode == 0) {
        const double mean = static_cast<double>(dsum) / 6.0;
        double mu = 0.0;
#pragma unroll
        for (int i = 0; i < 6; ++i) mu += static_cast<double>(z[i]);
        mu /= 6.0;
        double var = 0.0;
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const double d = static_cast<double>(z[i]) - mu;
            var += d * d;
        }
        const double sigma = sqrt(var / 6.0);
#pragma unroll
        for (int i = 0; i < 6; ++i)
            z[i] = static_cast<float>(static_cast<double>(z[i]) +
                                      alpha * sigma * (static_cast<double>(dot[i]) - mean));
    } else {
#pragma unroll
        for (int i = 0; i < 6; ++i)
            if (C24::mask[i] == m0) z[i] = static_cast<float>(static_cast<double>(z[i]) + alpha);
    }
}

template <typename WT, bool BITS>
__global__ __launch_bounds__(kThreads) void prior24_kernel(PriorArgs a) {
    __shared__ float4 stage[3 * kThreads];
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads; base < npairs;
         base += stride) {
        const int64_t p = base + threadIdx.x;
        float z[12];
        if (p < npairs) {
            const bool two = 2 * p + 1 < a.g.nblocks;
            load12(a.z, p, two, z);
            uint32_t m0, m1;
            if (BITS) {
                const uint32_t byte = a.prior_bits[p];
                m0 = byte & 0xFu;
                m1 = byte >> 4;
            } else {
                uint32_t r[8], mag[8];
                Io<WT>::load8_raw(a.w, p, two, r);
#pragma unroll
                for (int j = 0; j < 8; ++j) mag[j] = Io<WT>::magnitude(r[j]);
                m0 = top2_of4(mag);
                m1 = top2_of4(mag + 4);
            }
            prior_block6(z, m0, a.alpha, a.mode);
            prior_block6(z + 6, m1, a.alpha, a.mode);
        }
        // in place: store12_tile's barrier orders every lane's loads before the stores
        store12_tile(a.z, base, a.g.nblocks, z, stage);
    }
}

// ---------------------------------------------------------------------------
// Launch helpers.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Training diagnostics (section 3.4 kappa discussion / Figure 5, Figures 6 and
// 8, Table 14): per-lane sums over block pairs, one set of atomics per
// workgroup.
// ---------------------------------------------------------------------------
// max_i softmax(kappa z)_i of one block = 1 / sum_i exp(kappa (z_i - zmax)).
__device__ __forceinline__ float max_prob6(const float *z, float kappa_log2e) {
    float zmax = z[0];
#pragma unroll
    for (int i = 1; i < 6; ++i) zmax = fmaxf(zmax, z[i]);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 6; ++i) s += __builtin_amdgcn_exp2f((z[i] - zmax) * kappa_log2e);
    return 1.0f / s;
}

// Sum of |w| over the positions kept by `keep` (bit j = position j).
__device__ __forceinline__ double kept_abs4(const float *w, uint32_t keep) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if ((keep >> j) & 1u) s += static_cast<double>(fabsf(w[j]));
    return s;
}

// Workgroup sums of five per-lane values; thread 0 adds them to the stats.
__device__ __forceinline__ void stats_flush(double (&v)[5], maskgs_stats *st) {
    __shared__ double part[5][kThreads / 64];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off);
        if (lane == 0) part[k][wid] = v[k];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < 5; ++k)
#pragma unroll
            for (int i = 0; i < kThreads / 64; ++i) t[k] += part[k][i];
        if (t[0] != 0.0)
            atomicAdd(reinterpret_cast<unsigned long long *>(&st->changed),
                      static_cast<unsigned long long>(t[0]));
        atomicAdd(&st->max_prob, t[1]);
        if (t[2] != 0.0 || t[3] != 0.0) {
            atomicAdd(&st->kept_l1, t[2]);
            atomicAdd(&st->magnitude_l1, t[3]);
        }
        if (t[4] != 0.0) atomicAdd(&st->grad_sq, t[4]);
    }
}

template <int PHASE, typename WT, bool SAMPLED>
__global__ __launch_bounds__(kThreads) void stats24_kernel(StatsArgs a) {
    __shared__ float4 gtab[SAMPLED ? kGumbelRows : 1];
    if constexpr (SAMPLED) {
        load_gumbel_table<kThreads>(gtab);
        __syncthreads();
    }
    const int64_t npairs = (a.g.nblocks + 1) >> 1;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    double acc[5] = {0.0, 0.0, 0.0, 0.0, 0.0};  // changed, max_prob, kept, magnitude, grad^2
    for (int64_t p = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; p < npairs;
         p += stride) {
        const bool two = 2 * p + 1 < a.g.nblocks;
        // every stream of the pair is requested before any is used, so one
        // memory latency covers them (the pointer tests are uniform)
        float z[12], d[12], w[8];
        uint32_t wd[8];
        uint32_t rb = 0;
        load12(a.z, p, two, z);
        if (a.w) Io<WT>::load8(a.w, p, two, w, wd);
        if (a.dz) load12(a.dz, p, two, d);
        if (a.ref_bits) rb = a.ref_bits[p];
        int k0, k1;
        if (SAMPLED) {
            float a12[12], g12[12];
            pair_noise<PHASE>(a.g, a.nz, p, gtab, g12);
            pair_logits(a.nz, z, g12, a12);
            k0 = first_argmax6(a12);
            k1 = first_argmax6(a12 + 6);
        } else {
            k0 = first_argmax6(z);
            k1 = first_argmax6(z + 6);
        }
        const uint32_t m0 = cand_mask6(k0), m1 = cand_mask6(k1);
        if (a.ref_bits)
            acc[0] += static_cast<double>(((rb & 0xFu) != m0) + (two && ((rb >> 4) != m1)));
        acc[1] += static_cast<double>(max_prob6(z, a.kappa_log2e));
        if (two) acc[1] += static_cast<double>(max_prob6(z + 6, a.kappa_log2e));
        if (a.w) {
            uint32_t mag[8];
            Io<WT>::mags8(wd, mag);
            acc[2] += kept_abs4(w, m0);
            acc[3] += kept_abs4(w, top2_of4(mag));
            if (two) {
                acc[2] += kept_abs4(w + 4, m1);
                acc[3] += kept_abs4(w + 4, top2_of4(mag + 4));
            }
        }
        if (a.dz) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < 12; ++i) s += static_cast<double>(d[i]) * static_cast<double>(d[i]);
            acc[4] += s;
        }
    }
    stats_flush(acc, a.stats);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        atomicAdd(reinterpret_cast<unsigned long long *>(&a.stats->blocks),
                  static_cast<unsigned long long>(a.g.nblocks));
}

template <int T = kThreads, typename K, typename A>
hipError_t go(K kernel, const A &args, int64_t items, hipStream_t s,
              int wg_per_cu = kWgPerCU) {
    const unsigned grid = grid_for(items, T, wg_per_cu);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(T), 0, s, args);
    return hipGetLastError();
}

// The diagnostics pass ends every workgroup with five fp64 atomics into one
// 48-byte struct, which serialise at its L2 line: 2 workgroups per CU
// (measured 125 us on 11008x4096) against 175 us at the grid cap of the
// streaming kernels and 279 us at 16.
constexpr int kStatsWgPerCU = 2;

int phase_of(uint64_t block_offset) { return (block_offset & 1u) ? 2 : 0; }

template <int PHASE, bool YSAVE>
hipError_t fwd24_dispatch(const FwdArgs &a, maskgs_dtype w_dt, maskgs_dtype o_dt,
                          hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    constexpr int T = YSAVE ? kThreads : kFwdNoYThreads;
    const int c = YSAVE ? kWgPerCU : kFwdNoYWgPerCU;
    if (w_dt == MASKGS_BF16 && o_dt == MASKGS_BF16)
        return go<T>(fwd24_kernel<PHASE, bf16_t, bf16_t, YSAVE, T>, a, np, s, c);
    if (w_dt == MASKGS_BF16 && o_dt == MASKGS_F32)
        return go<T>(fwd24_kernel<PHASE, bf16_t, float, YSAVE, T>, a, np, s, c);
    if (w_dt == MASKGS_F32 && o_dt == MASKGS_BF16)
        return go<T>(fwd24_kernel<PHASE, float, bf16_t, YSAVE, T>, a, np, s, c);
    return go<T>(fwd24_kernel<PHASE, float, float, YSAVE, T>, a, np, s, c);
}

template <int PHASE, bool SAVED, bool ADAMW>
hipError_t bwd24_dispatch(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    constexpr bool rc = !SAVED && !ADAMW;
    constexpr int T = rc ? kBwdRcThreads : kThreads;
    const int c = ADAMW ? kWgPerCUStream : (rc ? kBwdRcWgPerCU : kWgPerCU);
    if (w_dt == MASKGS_BF16 && g_dt == MASKGS_BF16)
        return go<T>(bwd24_kernel<PHASE, bf16_t, bf16_t, SAVED, ADAMW, T>, a, np, s, c);
    if (w_dt == MASKGS_BF16)
        return go<T>(bwd24_kernel<PHASE, bf16_t, float, SAVED, ADAMW, T>, a, np, s, c);
    if (g_dt == MASKGS_BF16)
        return go<T>(bwd24_kernel<PHASE, float, bf16_t, SAVED, ADAMW, T>, a, np, s, c);
    return go<T>(bwd24_kernel<PHASE, float, float, SAVED, ADAMW, T>, a, np, s, c);
}

template <bool ADAMW>
hipError_t bwd24_phase(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s) {
    const bool even = phase_of(a.g.block_offset) == 0;
    if (a.y) return even ? bwd24_dispatch<0, true, ADAMW>(a, w_dt, g_dt, s)
                         : bwd24_dispatch<2, true, ADAMW>(a, w_dt, g_dt, s);
    return even ? bwd24_dispatch<0, false, ADAMW>(a, w_dt, g_dt, s)
                : bwd24_dispatch<2, false, ADAMW>(a, w_dt, g_dt, s);
}

template <int PHASE, bool SAVED>
hipError_t reg24_dispatch(const RegArgs &a, maskgs_dtype w_dt, hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    if (w_dt == MASKGS_BF16) return go(reg24_kernel<PHASE, bf16_t, SAVED>, a, np, s);
    return go(reg24_kernel<PHASE, float, SAVED>, a, np, s);
}

}  // namespace

hipError_t launch_fwd24(const FwdArgs &a, maskgs_dtype w_dt, maskgs_dtype out_dt, hipStream_t s) {
    const bool even = phase_of(a.g.block_offset) == 0;
    if (a.y) return even ? fwd24_dispatch<0, true>(a, w_dt, out_dt, s)
                         : fwd24_dispatch<2, true>(a, w_dt, out_dt, s);
    return even ? fwd24_dispatch<0, false>(a, w_dt, out_dt, s)
                : fwd24_dispatch<2, false>(a, w_dt, out_dt, s);
}

hipError_t launch_bwd24(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s) {
    return a.m1 ? bwd24_phase<true>(a, w_dt, g_dt, s) : bwd24_phase<false>(a, w_dt, g_dt, s);
}

hipError_t launch_reg24(const RegArgs &a, maskgs_dtype w_dt, hipStream_t s) {
    const bool even = phase_of(a.g.block_offset) == 0;
    if (a.y) return even ? reg24_dispatch<0, true>(a, w_dt, s) : reg24_dispatch<2, true>(a, w_dt, s);
    return even ? reg24_dispatch<0, false>(a, w_dt, s) : reg24_dispatch<2, false>(a, w_dt, s);
}

hipError_t launch_hard24(const HardArgs &a, maskgs_dtype w_dt, hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    if (a.values && w_dt == MASKGS_F32) return go(hard24_kernel<float>, a, np, s, kWgPerCUStream);
    return go(hard24_kernel<bf16_t>, a, np, s, kWgPerCUStream);
}

hipError_t launch_prior24(const PriorArgs &a, maskgs_dtype w_dt, hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    const int c = kWgPerCUStream;
    if (a.prior_bits) return go(prior24_kernel<bf16_t, true>, a, np, s, c);
    if (w_dt == MASKGS_F32) return go(prior24_kernel<float, false>, a, np, s, c);
    return go(prior24_kernel<bf16_t, false>, a, np, s, c);
}

template <int PHASE>
hipError_t stats24_dispatch(const StatsArgs &a, bool sampled, maskgs_dtype w_dt, hipStream_t s) {
    const int64_t np = (a.g.nblocks + 1) >> 1;
    const int c = kStatsWgPerCU;
    if (sampled)
        return w_dt == MASKGS_F32 ? go(stats24_kernel<PHASE, float, true>, a, np, s, c)
                                  : go(stats24_kernel<PHASE, bf16_t, true>, a, np, s, c);
    return w_dt == MASKGS_F32 ? go(stats24_kernel<PHASE, float, false>, a, np, s, c)
                              : go(stats24_kernel<PHASE, bf16_t, false>, a, np, s, c);
}

hipError_t launch_stats24(const StatsArgs &a, bool sampled, maskgs_dtype w_dt, hipStream_t s) {
    return phase_of(a.g.block_offset) == 0 ? stats24_dispatch<0>(a, sampled, w_dt, s)
                                           : stats24_dispatch<2>(a, sampled, w_dt, s);
}

}  // namespace maskgs
