// roofline_probe.hip -- calibration kernels behind the roofline figures that
// the benchmark reports for libmaskgs on MI355X (gfx950).
//
//  hbm   streams of known size over 4 GiB buffers (far beyond the 256 MB
//        last-level cache), 16 bytes per lane per access, fully coalesced:
//        pure read, pure write (plain and non-temporal stores), copy, and
//        mixed read/write streams in the byte ratios of the mask kernels.
//        Prints the best of several launch shapes: the HBM rate a kernel
//        with that traffic mix can reach on this chip.
//  valu  loops of known VALU instruction count: 8 independent chains of one
//        instruction class, 1024 iterations, so every wave issues exactly
//        8192 instructions of that class (plus a few dozen of set-up and
//        folding).  Prints wave instructions per microsecond per class; run
//        under rocprofv3 with SQ_INSTS_VALU it shows what that counter
//        counts (wave-level instructions) and, with SQ_ACTIVE_INST_VALU2,
//        which classes issue two per cycle pair.
//  read | write | copy   one stream kernel alone (warm-up plus 5 launches),
//        for FETCH_SIZE / WRITE_SIZE counter runs against known bytes.
//
// Usage: roofline_probe hbm|valu|read|write|copy
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#define CHECK(x)                                                                     \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), \
                         __LINE__);                                                  \
            std::exit(1);                                                            \
        }                                                                            \
    } while (0)

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMagic = 0x9E3779B9u;

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold4(float4 v) {
    return __float_as_uint(v.x) ^ __float_as_uint(v.y) ^ __float_as_uint(v.z) ^
           __float_as_uint(v.w);
}

// ---------------------------------------------------------------------------
// HBM streams.  Each kernel walks its float4 index range grid-stride.  A read
// result is kept live by a store that happens only if the running xor equals
// a fixed constant (practically never): no write traffic.
// ---------------------------------------------------------------------------
// A float4 load, non-temporal (NTL) or plain.
template <bool NTL>
__device__ __forceinline__ float4 load4(const float4 *p) {
    if constexpr (NTL) {
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

template <int U, bool NTL = false>
__global__ __launch_bounds__(kThreads) void read_kernel(const float4 *src, int64_t n4,
                                                        uint32_t *sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * U;
    uint32_t acc = 0;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kThreads * U + threadIdx.x; i0 < n4;
         i0 += stride) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = i0 + u * kThreads < n4 ? load4<NTL>(src + i0 + u * kThreads)
                                          : make_float4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold4(v[u]);
    }
    if (acc == kMagic) sink[0] = acc;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void write_kernel(float4 *dst, int64_t n4) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n4;
         i += stride) {
        const float f = static_cast<float>(i & 0xFFFF);
        if (NT)
            __builtin_nontemporal_store(v4f{f, f, f, f}, reinterpret_cast<v4f *>(dst + i));
        else
            dst[i] = make_float4(f, f, f, f);
    }
}

// Copy, U float4 per lane in flight per iteration (loads first, then stores);
// non-temporal or plain stores.  Every access is bounds-checked.
template <int U, bool NT, bool NTL = false>
__global__ __launch_bounds__(kThreads) void copy_kernel(const float4 *src, float4 *dst,
                                                        int64_t n4) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * U;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kThreads * U + threadIdx.x; i0 < n4;
         i0 += stride) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = i0 + u * kThreads < n4 ? load4<NTL>(src + i0 + u * kThreads)
                                          : make_float4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u * kThreads >= n4) continue;
            if (NT)
                __builtin_nontemporal_store(v4f{v[u].x, v[u].y, v[u].z, v[u].w},
                                            reinterpret_cast<v4f *>(dst + i0 + u * kThreads));
            else
                dst[i0 + u * kThreads] = v[u];
        }
    }
}

// R read streams and W write streams of n4 float4 each, one float4 of every
// stream per index: R*16 bytes read and W*16 bytes written per index.
template <int R, int W>
__global__ __launch_bounds__(kThreads) void rw_kernel(const float4 *src, float4 *dst,
                                                      int64_t n4, uint32_t *sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    uint32_t acc = 0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n4;
         i += stride) {
        float4 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = src[r * n4 + i];
        float4 s = v[0];
#pragma unroll
        for (int r = 1; r < R; ++r) {
            s.x += v[r].x;
            s.y += v[r].y;
            s.z += v[r].z;
            s.w += v[r].w;
        }
        acc ^= fold4(s);
#pragma unroll
        for (int w = 0; w < W; ++w)
            __builtin_nontemporal_store(v4f{s.x, s.y, s.z, s.w + static_cast<float>(w)},
                                        reinterpret_cast<v4f *>(dst + w * n4 + i));
    }
    if (acc == kMagic) sink[0] = acc;
}

// ---------------------------------------------------------------------------
// VALU issue loops.  Each class: 8 independent chains, kIters iterations of
// one inline-assembly instruction per chain, the loop counter uniform (scalar
// instructions only), so a wave issues exactly 8 * kIters instructions of the
// class inside the loop.
// ---------------------------------------------------------------------------
constexpr int kIters = 1024;
constexpr int kChains = 8;

enum Op {
    kAddU32,       // v_add_u32 v, v, v
    kFmaF32,       // v_fma_f32 v, v, v, v
    kFmaF32Sgpr,   // v_fma_f32 v, v, s, v (one scalar operand)
    kBitop3,       // v_bitop3_b32 v, v, v, v (three-input xor)
    kMadU64,       // v_mad_u64_u32 v[2], vcc, v, v, v[2]
    kCvtF32U32,    // v_cvt_f32_u32 v, v
    kExpF32,       // v_exp_f32 v, v
    kRcpF32,       // v_rcp_f32 v, v
    kFmaF64,       // v_fma_f64 v[2], v[2], v[2], v[2]
    kBitop3Sgpr,   // v_bitop3_b32 v, v, v, s (one scalar operand)
    kCndmaskVcc,   // v_cndmask_b32 v, v, v, vcc
    kCmpVcc,       // v_cmp_gt_f32 vcc, v, v
    kMovSgpr,      // v_mov_b32 v, s
    kMax3F32,      // v_max3_f32 v, v, v, v
    kMin3U32,      // v_min3_u32 v, v, v, v
    kAndOrB32,     // v_and_or_b32 v, v, v, v
    kOrLiteral,    // v_or_b32 v, literal, v
    kCmpCndmask,   // v_cmp_gt_f32 vcc, v, v then v_cndmask_b32 v, v, v, vcc (a pair)
    kCndmaskSgpr,  // v_cndmask_b32 v, v, v, s[2] (VOP3 form, mask in a scalar pair)
    kMaxF32,       // v_max_f32 v, v, v
    kMulF32,       // v_mul_f32 v, v, v
    kBfiB32,       // v_bfi_b32 v, v, v, v
    kNumOps
};

const char *op_name(int op) {
    static const char *names[] = {"v_add_u32 (vgpr)",  "v_fma_f32 (vgpr)", "v_fma_f32 (sgpr)",
                                  "v_bitop3_b32",      "v_mad_u64_u32",    "v_cvt_f32_u32",
                                  "v_exp_f32",         "v_rcp_f32",        "v_fma_f64",
                                  "v_bitop3_b32 (sgpr)", "v_cndmask_b32 (vcc)", "v_cmp_gt_f32 (vcc)",
                                  "v_mov_b32 (sgpr)",  "v_max3_f32",       "v_min3_u32",
                                  "v_and_or_b32",      "v_or_b32 (literal)",
                                  "cmp+cndmask (vcc)", "v_cndmask_b32 (s[2])", "v_max_f32",
                                  "v_mul_f32",         "v_bfi_b32"};
    return names[op];
}

template <int OP>
__global__ __launch_bounds__(kThreads) void valu_kernel(uint32_t *sink, uint32_t seed,
                                                        float fs) {
    const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
    uint32_t u[kChains];
    float f[kChains];
    double d[kChains];
    uint64_t q[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        u[c] = t * 2654435761u + seed + static_cast<uint32_t>(c);
        f[c] = 0.5f + static_cast<float>(u[c] & 1023u) * 1e-3f;
        d[c] = static_cast<double>(f[c]);
        q[c] = (static_cast<uint64_t>(u[c]) << 32) | (u[c] ^ seed);
    }
    uint32_t ku = 0x9E3779B9u ^ t, kv = 0xD2511F53u + t;
    float fa = 0.9999f, fb = 1e-4f;
    double da = 0.9999, db = 1e-4;
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (OP == kAddU32)
                asm volatile("v_add_u32 %0, %0, %1" : "+v"(u[c]) : "v"(ku));
            if constexpr (OP == kFmaF32)
                asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[c]) : "v"(fa), "v"(fb));
            if constexpr (OP == kFmaF32Sgpr)
                asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[c]) : "s"(fs), "v"(fb));
            if constexpr (OP == kBitop3)
                asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96"
                             : "+v"(u[c])
                             : "v"(ku), "v"(kv));
            if constexpr (OP == kMadU64)
                asm volatile("v_mad_u64_u32 %0, vcc, %1, %2, %0"
                             : "+v"(q[c])
                             : "v"(u[c]), "v"(kv)
                             : "vcc");
            if constexpr (OP == kCvtF32U32)
                asm volatile("v_cvt_f32_u32 %0, %1" : "=v"(f[c]) : "v"(u[c]));
            if constexpr (OP == kExpF32) asm volatile("v_exp_f32 %0, %0" : "+v"(f[c]));
            if constexpr (OP == kRcpF32) asm volatile("v_rcp_f32 %0, %0" : "+v"(f[c]));
            if constexpr (OP == kFmaF64)
                asm volatile("v_fma_f64 %0, %0, %1, %2" : "+v"(d[c]) : "v"(da), "v"(db));
            if constexpr (OP == kBitop3Sgpr)
                asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96"
                             : "+v"(u[c])
                             : "v"(ku), "s"(seed));
            if constexpr (OP == kCndmaskVcc)
                asm volatile("v_cndmask_b32 %0, %0, %1, vcc" : "+v"(u[c]) : "v"(ku));
            if constexpr (OP == kCmpVcc)
                asm volatile("v_cmp_gt_f32 vcc, %0, %1" : : "v"(f[c]), "v"(fa) : "vcc");
            if constexpr (OP == kMovSgpr)
                asm volatile("v_mov_b32 %0, %1" : "=v"(u[c]) : "s"(seed + static_cast<uint32_t>(c)));
            if constexpr (OP == kMax3F32)
                asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(f[c]) : "v"(fa), "v"(fb));
            if constexpr (OP == kMin3U32)
                asm volatile("v_min3_u32 %0, %0, %1, %2" : "+v"(u[c]) : "v"(ku), "v"(kv));
            if constexpr (OP == kAndOrB32)
                asm volatile("v_and_or_b32 %0, %0, %1, %2" : "+v"(u[c]) : "v"(ku), "v"(kv));
            if constexpr (OP == kOrLiteral)
                asm volatile("v_or_b32 %0, 0x12345, %0" : "+v"(u[c]));
            if constexpr (OP == kCmpCndmask)
                asm volatile("v_cmp_gt_f32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
                             : "+v"(u[c])
                             : "v"(f[c]), "v"(fa), "v"(ku)
                             : "vcc");
            if constexpr (OP == kCndmaskSgpr)
                asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2"
                             : "+v"(u[c])
                             : "v"(ku), "s"(static_cast<uint64_t>(seed) * 0x9E3779B97F4A7C15ull));
            if constexpr (OP == kMaxF32)
                asm volatile("v_max_f32 %0, %0, %1" : "+v"(f[c]) : "v"(fa));
            if constexpr (OP == kMulF32)
                asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[c]) : "v"(fa));
            if constexpr (OP == kBfiB32)
                asm volatile("v_bfi_b32 %0, %1, %0, %2" : "+v"(u[c]) : "v"(ku), "v"(kv));
        }
    }
    uint32_t r = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        uint64_t db64;
        std::memcpy(&db64, &d[c], 8);
        r ^= u[c] ^ __float_as_uint(f[c]) ^ static_cast<uint32_t>(q[c]) ^
             static_cast<uint32_t>(q[c] >> 32) ^ static_cast<uint32_t>(db64);
    }
    if (r == kMagic) sink[t] = r;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Timer {
    hipEvent_t a, b;
    Timer() {
        CHECK(hipEventCreate(&a));
        CHECK(hipEventCreate(&b));
    }
    ~Timer() {
        (void)hipEventDestroy(a);
        (void)hipEventDestroy(b);
    }
};

int cu_count() {
    int dev = 0, n = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev));
    return n;
}

// Best time (ms) of `reps` launches of fn(grid) after one warm-up, over the
// given grid sizes; returns the best and the grid that gave it.
template <typename F>
double best_ms(F fn, const std::vector<unsigned> &grids, int reps, unsigned *best_grid) {
    Timer t;
    double best = 1e30;
    for (unsigned g : grids) {
        fn(g);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
        for (int r = 0; r < reps; ++r) {
            CHECK(hipEventRecord(t.a));
            fn(g);
            CHECK(hipEventRecord(t.b));
            CHECK(hipEventSynchronize(t.b));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, t.a, t.b));
            if (ms < best) {
                best = ms;
                *best_grid = g;
            }
        }
    }
    return best;
}

void report(const char *what, double bytes, double ms, unsigned grid) {
    std::printf("%-34s %8.3f GiB  %9.1f us  %7.1f GB/s  (grid %u x %d)\n", what,
                bytes / (1024.0 * 1024.0 * 1024.0), ms * 1e3, bytes / (ms * 1e-3) / 1e9, grid,
                kThreads);
}

constexpr int64_t kGiB = INT64_C(1) << 30;

void run_hbm() {
    const int cus = cu_count();
    std::vector<unsigned> grids = {static_cast<unsigned>(cus) * 4, static_cast<unsigned>(cus) * 8,
                                   static_cast<unsigned>(cus) * 16,
                                   static_cast<unsigned>(cus) * 32};
    const int64_t bytes = 4 * kGiB;
    const int64_t n4 = bytes / 16;
    float4 *a = nullptr, *b = nullptr;
    uint32_t *sink = nullptr;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&sink, 64));
    CHECK(hipMemset(a, 0x3c, bytes));
    CHECK(hipMemset(b, 0, bytes));
    CHECK(hipDeviceSynchronize());
    unsigned g = 0;
    double ms;
    ms = best_ms([&](unsigned gr) { read_kernel<1><<<gr, kThreads>>>(a, n4, sink); }, grids, 5,
                 &g);
    report("read", static_cast<double>(bytes), ms, g);
    ms = best_ms([&](unsigned gr) { read_kernel<4><<<gr, kThreads>>>(a, n4, sink); }, grids, 5,
                 &g);
    report("read (4 in flight per lane)", static_cast<double>(bytes), ms, g);
    ms = best_ms([&](unsigned gr) { read_kernel<1, true><<<gr, kThreads>>>(a, n4, sink); }, grids,
                 5, &g);
    report("read (non-temporal loads)", static_cast<double>(bytes), ms, g);
    ms = best_ms([&](unsigned gr) { write_kernel<false><<<gr, kThreads>>>(b, n4); }, grids, 5, &g);
    report("write", static_cast<double>(bytes), ms, g);
    ms = best_ms([&](unsigned gr) { write_kernel<true><<<gr, kThreads>>>(b, n4); }, grids, 5, &g);
    report("write (non-temporal)", static_cast<double>(bytes), ms, g);
    {
        // 2 GiB each way
        const int64_t h4 = n4 / 2;
        ms = best_ms([&](unsigned gr) { copy_kernel<1, true><<<gr, kThreads>>>(a, b, h4); }, grids,
                     5, &g);
        report("copy (nt stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms([&](unsigned gr) { copy_kernel<1, false><<<gr, kThreads>>>(a, b, h4); },
                     grids, 5, &g);
        report("copy (plain stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms([&](unsigned gr) { copy_kernel<4, true><<<gr, kThreads>>>(a, b, h4); }, grids,
                     5, &g);
        report("copy (4 in flight, nt stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms([&](unsigned gr) { copy_kernel<4, false><<<gr, kThreads>>>(a, b, h4); },
                     grids, 5, &g);
        report("copy (4 in flight, plain stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms([&](unsigned gr) { copy_kernel<1, true, true><<<gr, kThreads>>>(a, b, h4); },
                     grids, 5, &g);
        report("copy (nt loads, nt stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms([&](unsigned gr) { copy_kernel<1, false, true><<<gr, kThreads>>>(a, b, h4); },
                     grids, 5, &g);
        report("copy (nt loads, plain stores)", 2.0 * 16 * h4, ms, g);
        ms = best_ms(
            [&](unsigned) { CHECK(hipMemcpyAsync(b, a, 16 * h4, hipMemcpyDeviceToDevice, 0)); },
            {0u}, 5, &g);
        report("hipMemcpyAsync device to device", 2.0 * 16 * h4, ms, g);
    }
    // mixed streams over the same 4 GiB buffers: each stream n4/(R or W) long
    {
        const int64_t m = n4 / 5;
        ms = best_ms([&](unsigned gr) { rw_kernel<5, 2><<<gr, kThreads>>>(a, b, m, sink); }, grids,
                     5, &g);
        report("read 5 : write 2 streams", 7.0 * 16 * m, ms, g);
        ms = best_ms([&](unsigned gr) { rw_kernel<5, 3><<<gr, kThreads>>>(a, b, m, sink); }, grids,
                     5, &g);
        report("read 5 : write 3 streams", 8.0 * 16 * m, ms, g);
        ms = best_ms([&](unsigned gr) { rw_kernel<2, 2><<<gr, kThreads>>>(a, b, m, sink); }, grids,
                     5, &g);
        report("read 2 : write 2 streams", 4.0 * 16 * m, ms, g);
    }
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(sink));
}

// One stream kernel alone: warm-up plus 5 launches on 1 GiB, grid 8 per CU.
void run_one(const std::string &mode) {
    const int cus = cu_count();
    const unsigned grid = static_cast<unsigned>(cus) * 8;
    const int64_t bytes = kGiB;
    const int64_t n4 = bytes / 16;
    float4 *a = nullptr, *b = nullptr;
    uint32_t *sink = nullptr;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&sink, 64));
    CHECK(hipMemset(a, 0x3c, bytes));
    CHECK(hipDeviceSynchronize());
    unsigned g = 0;
    double ms = 0.0, moved = 0.0;
    if (mode == "read") {
        ms = best_ms([&](unsigned gr) { read_kernel<1><<<gr, kThreads>>>(a, n4, sink); }, {grid}, 5,
                     &g);
        moved = static_cast<double>(bytes);
    } else if (mode == "write") {
        ms = best_ms([&](unsigned gr) { write_kernel<true><<<gr, kThreads>>>(b, n4); }, {grid}, 5,
                     &g);
        moved = static_cast<double>(bytes);
    } else {
        ms = best_ms([&](unsigned gr) { copy_kernel<1, true><<<gr, kThreads>>>(a, b, n4); }, {grid},
                     5, &g);
        moved = 2.0 * bytes;
    }
    report(mode.c_str(), moved, ms, g);
    std::printf("bytes read per launch %lld, written per launch %lld\n",
                static_cast<long long>(mode == "write" ? 0 : bytes),
                static_cast<long long>(mode == "read" ? 0 : bytes));
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(sink));
}

template <int OP>
void valu_one(uint32_t *sink, unsigned grid) {
    unsigned g = 0;
    const double ms = best_ms(
        [&](unsigned gr) { valu_kernel<OP><<<gr, kThreads>>>(sink, 1u, 0.9999f); }, {grid}, 3, &g);
    const double waves = static_cast<double>(grid) * (kThreads / 64);
    const double insts = waves * kChains * kIters * (OP == kCmpCndmask ? 2 : 1);
    const double rate = insts / (ms * 1e3);  // wave instructions per microsecond
    std::printf("%-20s %9.1f us  %8.1f k wave-instr/us  %.2f cycles per instruction per SIMD "
                "at 2.4 GHz\n",
                op_name(OP), ms * 1e3, rate / 1e3,
                (ms * 1e-3) * 2.4e9 * cu_count() * 4 / insts);
}

template <int... OPS>
void valu_all(uint32_t *sink, unsigned grid, std::integer_sequence<int, OPS...>) {
    (valu_one<OPS>(sink, grid), ...);
}

void run_valu() {
    const unsigned grid = static_cast<unsigned>(cu_count()) * 32;  // 32 waves per CU
    uint32_t *sink = nullptr;
    CHECK(hipMalloc(&sink, static_cast<size_t>(grid) * kThreads * 4));
    std::printf("%u workgroups of %d lanes, %d instructions of the class per wave\n", grid,
                kThreads, kChains * kIters);
    valu_all(sink, grid, std::make_integer_sequence<int, kNumOps>{});
    CHECK(hipFree(sink));
}

}  // namespace

int main(int argc, char **argv) {
    const std::string mode = argc > 1 ? argv[1] : "";
    if (mode == "hbm") {
        run_hbm();
    } else if (mode == "valu") {
        run_valu();
    } else if (mode == "read" || mode == "write" || mode == "copy") {
        run_one(mode);
    } else {
        std::fprintf(stderr, "usage: %s hbm|valu|read|write|copy\n", argv[0]);
        return 2;
    }
    return 0;
}
