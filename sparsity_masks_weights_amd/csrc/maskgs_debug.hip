// maskgs_debug.hip -- test hooks of libmaskgs: raw Philox words of the noise
// stream and the fp32 Gumbel contract applied to given words.
#include <hip/hip_runtime.h>

#include "maskgs_device.hpp"
#include "maskgs_launch.hpp"

namespace maskgs {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void philox_words_kernel(uint32_t k0, uint32_t k1,
                                                                uint32_t step, uint32_t tid,
                                                                uint64_t n0, int64_t count,
                                                                uint32_t *out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < count;
         t += stride) {
        const uint64_t n = n0 + static_cast<uint64_t>(t);
        const uint64_t q = n >> 2;
        uint32_t x0 = static_cast<uint32_t>(q), x1 = static_cast<uint32_t>(q >> 32);
        uint32_t x2 = step, x3 = tid;
        philox10(x0, x1, x2, x3, k0, k1);
        const uint32_t r = n & 3u;
        out[t] = r == 0 ? x0 : r == 1 ? x1 : r == 2 ? x2 : x3;
    }
}

__global__ __launch_bounds__(kThreads) void gumbel_kernel(const uint32_t *words, int64_t n,
                                                          float *g) {
    __shared__ float4 gtab[kGumbelRows];
    load_gumbel_table<kThreads>(gtab);
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; t < n;
         t += stride)
        g[t] = gumbel_lds(words[t], gtab);
}

}  // namespace

hipError_t launch_debug_philox(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                               int64_t count, uint32_t *words, hipStream_t s) {
    const unsigned grid = grid_for(count, kThreads, 8);
    hipLaunchKernelGGL(philox_words_kernel, dim3(grid), dim3(kThreads), 0, s,
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32), step,
                       tensor_id, n0, count, words);
    return hipGetLastError();
}

hipError_t launch_debug_gumbel(const uint32_t *words, int64_t n, float *g, hipStream_t s) {
    const unsigned grid = grid_for(n, kThreads, 8);
    hipLaunchKernelGGL(gumbel_kernel, dim3(grid), dim3(kThreads), 0, s, words, n, g);
    return hipGetLastError();
}

}  // namespace maskgs
