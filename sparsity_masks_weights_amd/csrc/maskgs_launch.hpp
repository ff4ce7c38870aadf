// maskgs_launch.hpp -- kernel argument blocks and launchers shared by the C-ABI
// layer and the kernel files of libmaskgs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "maskgs.h"

namespace maskgs {

// Geometry of one call: K = C(m, n) candidates, nblocks = rows*cols/m blocks,
// block 0 of the call is global block block_offset.
struct Geometry {
    int32_t n, m, k;
    int64_t nblocks;
    uint64_t block_offset;
    uint32_t tensor_id;
};

// Sampling scalars, prepared on the host: Philox key words, step, kappa,
// fp32(1/tau) for the logit step, kappa/tau in fp64 for the gradient.
struct Noise {
    uint32_t k0, k1, step;
    float kappa, tau_inv;
    double grad_scale;
    uint32_t no_noise;
};

struct FwdArgs {
    const void *w;
    const float *z;
    void *out;
    float *y;     // nullable
    double *reg;  // nullable
    Geometry g;
    Noise nz;
    // hard mask of the same logits (maskgs_fwd_hard), all nullable
    uint8_t *idx = nullptr;
    uint8_t *bits = nullptr;
    void *values = nullptr;
    uint8_t *val_idx = nullptr;
};

struct BwdArgs {
    const void *w;
    const float *z;  // nullable when y is given
    const float *y;  // nullable: recompute
    const void *dout;
    float *dz;
    double lambda;
    bool accumulate;
    Geometry g;
    Noise nz;
};

struct RegArgs {
    const void *w;
    const float *z;
    const float *y;
    double *reg;
    Geometry g;
    Noise nz;
};

struct HardArgs {
    const float *z;
    const void *w;
    uint8_t *idx;
    uint8_t *bits;
    void *values;
    uint8_t *val_idx;
    Geometry g;
};

struct PriorArgs {
    float *z;
    const uint8_t *prior_bits;
    const void *w;
    double alpha;
    int32_t mode;
    Geometry g;
};

int device_cu_count();

// Grid size for a grid-stride kernel over `items` work items.
inline unsigned grid_for(int64_t items, int threads, int waves_per_cu) {
    const int64_t want = (items + threads - 1) / threads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * waves_per_cu;
    const int64_t g = want < cap ? want : cap;
    return static_cast<unsigned>(g < 1 ? 1 : g);
}

hipError_t launch_fwd24(const FwdArgs &a, maskgs_dtype w_dt, maskgs_dtype out_dt, hipStream_t s);
hipError_t launch_bwd24(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s);
hipError_t launch_reg24(const RegArgs &a, maskgs_dtype w_dt, hipStream_t s);
hipError_t launch_hard24(const HardArgs &a, maskgs_dtype w_dt, hipStream_t s);
hipError_t launch_prior24(const PriorArgs &a, maskgs_dtype w_dt, hipStream_t s);

hipError_t launch_fwd48(const FwdArgs &a, maskgs_dtype w_dt, maskgs_dtype out_dt, hipStream_t s);
hipError_t launch_bwd48(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s);
hipError_t launch_reg48(const RegArgs &a, maskgs_dtype w_dt, hipStream_t s);
hipError_t launch_hard48(const HardArgs &a, hipStream_t s);
hipError_t launch_prior48(const PriorArgs &a, maskgs_dtype w_dt, hipStream_t s);

hipError_t launch_debug_philox(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                               int64_t count, uint32_t *words, hipStream_t s);
hipError_t launch_debug_gumbel(const uint32_t *words, int64_t n, float *g, hipStream_t s);

}  // namespace maskgs
