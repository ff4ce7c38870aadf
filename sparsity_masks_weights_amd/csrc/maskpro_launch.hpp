// maskpro_launch.hpp -- kernel argument blocks and launchers of the
// linear-space mask learner (maskpro.h), shared by the C-ABI layer and
// maskpro_k.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "maskgs.h"

namespace maskgs {

// One forward or backward call: M logits per block, the draw's Philox key,
// step and tensor id, and the outputs (each nullable where maskpro.h says so).
struct MpArgs {
    const void *w;
    const float *pi;
    void *out;
    uint8_t *bits;
    void *order;           // forward: draw order out
    const void *order_in;  // backward: draw order in (nullptr: draw again)
    float *dpi;
    float adv;
    uint32_t accumulate;
    int64_t nblocks;
    uint64_t block_offset;
    uint32_t tensor_id;
    uint32_t k0, k1, step;
    uint32_t no_noise;
};

struct MpInitArgs {
    const uint8_t *prior_bits;  // nullable: magnitude top-N of w
    const void *w;
    float c;
    float *pi;
    int64_t nblocks;
};

hipError_t launch_mp_fwd(const MpArgs &a, int m, maskgs_dtype w_dt, maskgs_dtype out_dt,
                         hipStream_t s);
hipError_t launch_mp_bwd(const MpArgs &a, int m, hipStream_t s);
hipError_t launch_mp_init(const MpInitArgs &a, int m, maskgs_dtype w_dt, hipStream_t s);

}  // namespace maskgs
