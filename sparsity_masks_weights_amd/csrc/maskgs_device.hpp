// maskgs_device.hpp -- device building blocks of libmaskgs (gfx950): candidate
// tables, the Philox4x32-10 stream, the fp32 Gumbel noise contract and the
// bf16 store.  Functions are __host__ __device__ so that the noise contract
// can also be exercised on the CPU.
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

// ---------------------------------------------------------------------------
// Noise contract.
// Uniform: eps = (2*(x>>9) + 1) * 2^-24, exact, inside (0, 1).
// Natural log ln_c: Cephes (S. L. Moshier) single-precision logarithm with a
// fixed operation order: reduce x = 2^e * X with X in [sqrt(1/2), sqrt(2))
// (the bit pattern 0x3F3504F3 of fp32 sqrt(1/2) splits the binade), f = X - 1,
// ln(1+f) = f - f^2/2 + f^3 P(f) with Cephes' degree-8 P (Horner, fmaf), and
// e*ln 2 added as 0.693359375*e plus -2.12194440e-4*e.
// Gumbel (MaskLLM summary, section 3.4, Eq. 5): g = -ln_c(-ln_c(eps)).
// ---------------------------------------------------------------------------
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

// ln_c on a pre-offset exponent/mantissa word ix = bits(x) - bits(sqrt(1/2)):
// e = ix >> 23 (arithmetic), X = mantissa of ix re-based on sqrt(1/2).
MASKGS_HD float ln_core(uint32_t ixu) {
    const int32_t ix = static_cast<int32_t>(ixu);
    const int32_t e = ix >> 23;  // exponent relative to [sqrt(1/2), sqrt(2))
    const float X = bits_to_f32((ixu & 0x007FFFFFu) + 0x3F3504F3u);
    const float f = X - 1.0f;
    const float z = f * f;
    float p = 7.0376836292e-2f;
    p = __builtin_fmaf(p, f, -1.1514610310e-1f);
    p = __builtin_fmaf(p, f, 1.1676998740e-1f);
    p = __builtin_fmaf(p, f, -1.2420140846e-1f);
    p = __builtin_fmaf(p, f, 1.4249322787e-1f);
    p = __builtin_fmaf(p, f, -1.6668057665e-1f);
    p = __builtin_fmaf(p, f, 2.0000714765e-1f);
    p = __builtin_fmaf(p, f, -2.4999993993e-1f);
    p = __builtin_fmaf(p, f, 3.3333331174e-1f);
    float y = (p * f) * z;
    const float fe = static_cast<float>(e);
    y = __builtin_fmaf(fe, -2.12194440e-4f, y);
    y = __builtin_fmaf(-0.5f, z, y);
    float r = f + y;
    r = __builtin_fmaf(fe, 0.693359375f, r);
    return r;
}

MASKGS_HD float ln_contract(float x) { return ln_core(f32_to_bits(x) - 0x3F3504F3u); }

MASKGS_HD float uniform_open(uint32_t x) {
    return static_cast<float>(((x >> 9) << 1) | 1u) * 0x1p-24f;
}

// -ln_c(-ln_c(eps)), evaluated on exactly the same operands as the contract:
//  - eps = (2k+1) * 2^-24 differs from the integer-valued float (2k+1) only in
//    its exponent field (by 24), so ln_c(eps) reads the bits of (2k+1) with
//    24 << 23 removed from the offset word;
//  - t = -r1 flips only the sign bit of r1, which is the same as adding
//    0x80000000 to its bit pattern.
MASKGS_HD float neg_gumbel(uint32_t x) {  // returns -g
    const float odd = static_cast<float>((x >> 8) | 1u);  // 2k+1, exact
    const float r1 = ln_core(f32_to_bits(odd) - (0x3F3504F3u + (24u << 23)));
    return ln_core(f32_to_bits(r1) + (0x80000000u - 0x3F3504F3u));
}

MASKGS_HD float gumbel(uint32_t x) { return -neg_gumbel(x); }

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
