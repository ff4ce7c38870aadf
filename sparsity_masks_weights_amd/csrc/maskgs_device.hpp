// maskgs_device.hpp -- device building blocks of libmaskgs (gfx950): candidate
// tables, the Philox4x32-10 stream, the fp32 Gumbel noise contract and the
// bf16 store.  The Philox stream and the element helpers are __host__
// __device__, so they can also be exercised on the CPU.
//
// Compile with -ffp-contract=off: the noise contract fixes every rounding, and
// the only fused multiply-adds are the explicit __builtin_fmaf calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MASKGS_HD __host__ __device__ __forceinline__

namespace maskgs {

// ---------------------------------------------------------------------------
// Candidate masks (MaskLLM summary, section 3.2 candidate set S_2:4; section
// 3.4 Eq. 7).  Bit j = keep position j of the block.
// ---------------------------------------------------------------------------
template <int N, int M>
struct Cands;

// 2:4 in the order the page lists the patterns:
// [1,1,0,0] [1,0,1,0] [1,0,0,1] [0,1,0,1] [0,1,1,0] [0,0,1,1]
template <>
struct Cands<2, 4> {
    static constexpr int K = 6;
    static constexpr uint8_t mask[6] = {0x3, 0x5, 0x9, 0xA, 0x6, 0xC};
};

// Lexicographic N-subsets of M positions, built by advancing the rightmost
// position that can still move (the classic next-combination step).
template <int N, int M, int K>
struct LexTable {
    uint8_t v[K];
    constexpr LexTable() : v() {
        int pos[N] = {};
        for (int i = 0; i < N; ++i) pos[i] = i;
        for (int k = 0; k < K; ++k) {
            uint8_t b = 0;
            for (int i = 0; i < N; ++i) b = static_cast<uint8_t>(b | (1u << pos[i]));
            v[k] = b;
            int i = N - 1;
            while (i >= 0 && pos[i] == M - N + i) --i;
            if (i < 0) break;
            ++pos[i];
            for (int t = i + 1; t < N; ++t) pos[t] = pos[t - 1] + 1;
        }
    }
};

template <>
struct Cands<4, 8> {
    static constexpr int K = 70;
    static constexpr LexTable<4, 8, 70> table{};
    static constexpr uint8_t at(int i) { return table.v[i]; }
};

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11).  The key is uniform across a launch, so the
// compiler keeps its schedule in scalar registers (the xor3 operand).
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// a ^ b ^ c.  On gfx950 one v_bitop3_b32 (truth table 0x96 is the three-input
// xor); the compiler forms it for some bit patterns but not for a chained xor,
// which would cost two instructions per Philox output word.
MASKGS_HD uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
    return a ^ b ^ c;
#endif
}

MASKGS_HD void philox10(uint32_t &c0, uint32_t &c1, uint32_t &c2, uint32_t &c3, uint32_t k0,
                        uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // 32x32 -> 64-bit products: one v_mad_u64_u32 each on gfx950
        const uint64_t p0 = static_cast<uint64_t>(c0) * kPhiloxM0;
        const uint64_t p1 = static_cast<uint64_t>(c2) * kPhiloxM1;
        const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
}

// Words j = 0..NW-1 of the stream starting at word index 4*q0 + PHASE: word j
// is output (PHASE+j)%4 of the call with counter q0 + (PHASE+j)/4.
template <int NW, int PHASE>
MASKGS_HD void stream_words(uint64_t q0, uint32_t step, uint32_t tensor_id, uint32_t k0,
                            uint32_t k1, uint32_t (&wd)[NW]) {
    constexpr int NC = (PHASE + NW + 3) / 4;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint64_t q = q0 + static_cast<uint64_t>(c);
        uint32_t x0 = static_cast<uint32_t>(q), x1 = static_cast<uint32_t>(q >> 32);
        uint32_t x2 = step, x3 = tensor_id;
        philox10(x0, x1, x2, x3, k0, k1);
        const uint32_t xs[4] = {x0, x1, x2, x3};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * c + u - PHASE;
            if (j >= 0 && j < NW) wd[j] = xs[u];
        }
    }
}

MASKGS_HD float bits_to_f32(uint32_t u) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __uint_as_float(u);
#else
    float f;
    __builtin_memcpy(&f, &u, 4);
    return f;
#endif
}

MASKGS_HD uint32_t f32_to_bits(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __float_as_uint(f);
#else
    uint32_t u;
    __builtin_memcpy(&u, &f, 4);
    return u;
#endif
}

// ---------------------------------------------------------------------------
// Noise contract: the Gumbel value of a Philox word (MaskLLM summary, section
// 3.4, Eq. 5: g = -ln(-ln eps) for a uniform eps).
// eps = k2 * 2^-24 with k2 = 2*(x >> 9) + 1, exact and inside (0, 1).  Below
// 1/2 (side 0) v = k2, above (side 1) v = 2^24 - k2, the same integer for
// 1 - eps; v in [2^b, 2^(b+1)).  g is a cubic in the offset d of v / 2^b from
// the centre of its segment (32 per binade): the Taylor coefficients of
// -ln(-ln eps) about that centre, one fp32 row (c0, c1, c2, c3) per
// (side, binade, segment), generated into maskgs_gumbel_table.inc.  Within
// 1.25 ulp of max(|g|, 1) of the exact value for all 2^23 uniforms.
// ---------------------------------------------------------------------------
constexpr int kGumbelRows = 2 * 24 * 32;

// The coefficient table in device memory; kernels copy it into LDS (24 KB)
// and evaluate the noise from there.
static __constant__ __attribute__((aligned(16))) float kGumbelTable[kGumbelRows][4] = {
#include "maskgs_gumbel_table.inc"
};

// Copies the table into LDS; all THREADS lanes of the workgroup call it and
// pass a barrier before the first gumbel_lds.
template <int THREADS>
__device__ __forceinline__ void load_gumbel_table(float4 *lds) {
    const float4 *src = reinterpret_cast<const float4 *>(kGumbelTable);
    for (int i = threadIdx.x; i < kGumbelRows; i += THREADS) lds[i] = src[i];
}

// A plain register copy the compiler does not fold away.  The polynomial's
// last fused multiply-add accumulates into the register that held c0, one of
// the four registers of the LDS read; left there, every noise value (and the
// logit built on it) kept a 4-aligned register slot, which took the 2:4
// forward from 58 to 72 VGPRs and made the 4:8 kernels spill.
__device__ __forceinline__ float fresh_reg(float x) {
    float r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// g of the contract for Philox word x.  With spread = x >> 31 (arithmetic:
// all ones on side 1), v = min(k2, 2^24 - k2) is ((x ^ spread) >> 8) | 1: on
// side 1 the complemented word gives 2^24 - k2 (for k2 = (x >> 8) | 1, the
// complement's (~x >> 8) | 1 is 2^24 - k2 whatever the parity of x >> 8).
// The row is side * 768 + b * 32 + q, read off the exponent and the top 5
// mantissa bits of fp32(v) (exact), and addressed in bytes: (f >> 14) masked
// is 16 (127 * 32 + b * 32 + q); the low 18 mantissa bits give
// d = v / 2^b - 1 - (q + 1/2)/32, also exact.
__device__ __forceinline__ float gumbel_lds(uint32_t x, const float4 *tab) {
    // shift and mask (dual-issue instructions) rather than a compare and a
    // select for the side; kept from being turned into one by the compiler
    int32_t spread = static_cast<int32_t>(x) >> 31;
    asm("" : "+v"(spread));
    const uint32_t v = ((x ^ static_cast<uint32_t>(spread)) >> 8) | 1u;
    const uint32_t f = f32_to_bits(static_cast<float>(v));
    const uint32_t side_bytes = static_cast<uint32_t>(spread) & (24u * 32u * 16u);
    const uint32_t off = ((f >> 14) & 0x1FFF0u) + side_bytes;
    const float d = bits_to_f32((f & 0x3FFFFu) | 0x3F800000u) - 1.015625f;
    const float4 c = *reinterpret_cast<const float4 *>(
        reinterpret_cast<const char *>(tab) + off - (127u << 5) * 16u);
    return fresh_reg(
        __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c.w, d, c.z), d, c.y), d, c.x));
}

// ---------------------------------------------------------------------------
// Element access.
// ---------------------------------------------------------------------------
struct bf16_t {
    uint16_t bits;
};

MASKGS_HD float widen(bf16_t v) { return bits_to_f32(static_cast<uint32_t>(v.bits) << 16); }
MASKGS_HD float widen(float v) { return v; }

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
MASKGS_HD uint16_t bf16_rne(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
#else
    const uint32_t u = f32_to_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
#endif
}

}  // namespace maskgs
