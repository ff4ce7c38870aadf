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
    uint32_t hard_sample;  // apply S[first argmax a] (straight-through backward)
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

// AdamW constants of one update, prepared on the host: 1 - beta and the
// reciprocal bias corrections 1/(1 - beta^t) rounded to fp32.
struct Adam {
    float lr, b1, omb1, b2, omb2, ibc1, ibc2, eps, wd;
};

struct BwdArgs {
    const void *w;
    const float *z;  // nullable when y is given
    const float *y;  // nullable: recompute
    const void *dout;
    float *dz;       // the logit gradient (nullptr under the fused AdamW update)
    double lambda;
    bool accumulate;
    Geometry g;
    Noise nz;
    // fused AdamW update (maskgs_bwd_adamw): the logits updated in place (the
    // same array as z) and the two moments; all nullptr otherwise
    float *zu = nullptr;
    float *m1 = nullptr;
    float *m2 = nullptr;
    Adam adam{};
};

struct StatsArgs {
    const float *z;
    const uint8_t *ref_bits;  // nullable
    const void *w;            // nullable
    const float *dz;          // nullable
    maskgs_stats *stats;
    float kappa_log2e;        // kappa * log2(e), for max softmax(kappa z)
    Geometry g;
    Noise nz;                 // the draw of the sampled hard mask (when sampled)
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

// One AdamW step of one logit (section 3.4, Algorithm 1 "update logits"), in
// fp32: m and v advance, z moves by lr (mh/(sqrt(vh)+eps) + wd z) with z the
// value before this step.
__device__ __forceinline__ void adam_step(float &z, float &m, float &v, float g, const Adam &a) {
    m = __builtin_fmaf(a.b1, m, a.omb1 * g);
    v = __builtin_fmaf(a.b2, v, a.omb2 * (g * g));
    const float den = __builtin_sqrtf(v * a.ibc2) + a.eps;
    const float upd = (m * a.ibc1) / den;
    z = z - a.lr * __builtin_fmaf(a.wd, z, upd);
}

__device__ __forceinline__ void adam_step4(float4 &z, float4 &m, float4 &v, float4 g,
                                           const Adam &a) {
    adam_step(z.x, m.x, v.x, g.x, a);
    adam_step(z.y, m.y, v.y, g.y, a);
    adam_step(z.z, m.z, v.z, g.z, a);
    adam_step(z.w, m.w, v.w, g.w, a);
}

// AdamW update of nf consecutive logits z[0..nf) (16-byte aligned, at most CAP
// float4) whose gradients are at g[0..nf) in LDS, with their moments m1, m2.
// Float4 number k*THREADS + t is handled by lane t of the THREADS lanes that
// share the span; the loads of BATCH such rounds are issued before any of them
// is used.  An odd float pair at the end is handled by lane 0.  Every lane of
// the span calls this once g is visible to all of them.
template <int THREADS, int CAP, int BATCH>
__device__ __forceinline__ void adamw_span(float *z, float *m1, float *m2, const float *g, int nf,
                                           const Adam &a, int t) {
    const int n4 = nf >> 2;
    constexpr int kRounds = (CAP + THREADS - 1) / THREADS;
    for (int r0 = 0; r0 < kRounds; r0 += BATCH) {
        float4 zz[BATCH], mm[BATCH], vv[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int i = (r0 + k) * THREADS + t;
            if (i < n4) {
                zz[k] = reinterpret_cast<const float4 *>(z)[i];
                mm[k] = reinterpret_cast<const float4 *>(m1)[i];
                vv[k] = reinterpret_cast<const float4 *>(m2)[i];
            }
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int i = (r0 + k) * THREADS + t;
            if (i < n4) {
                adam_step4(zz[k], mm[k], vv[k], reinterpret_cast<const float4 *>(g)[i], a);
                reinterpret_cast<float4 *>(z)[i] = zz[k];
                reinterpret_cast<float4 *>(m1)[i] = mm[k];
                reinterpret_cast<float4 *>(m2)[i] = vv[k];
            }
        }
    }
    if ((nf & 3) && t == 0) {
        const int i = 2 * n4;
        float2 zz = reinterpret_cast<float2 *>(z)[i], mm = reinterpret_cast<float2 *>(m1)[i];
        float2 vv = reinterpret_cast<float2 *>(m2)[i];
        const float2 gg = reinterpret_cast<const float2 *>(g)[i];
        adam_step(zz.x, mm.x, vv.x, gg.x, a);
        adam_step(zz.y, mm.y, vv.y, gg.y, a);
        reinterpret_cast<float2 *>(z)[i] = zz;
        reinterpret_cast<float2 *>(m1)[i] = mm;
        reinterpret_cast<float2 *>(m2)[i] = vv;
    }
}

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
hipError_t launch_stats24(const StatsArgs &a, bool sampled, maskgs_dtype w_dt, hipStream_t s);

hipError_t launch_fwd48(const FwdArgs &a, maskgs_dtype w_dt, maskgs_dtype out_dt, hipStream_t s);
hipError_t launch_bwd48(const BwdArgs &a, maskgs_dtype w_dt, maskgs_dtype g_dt, hipStream_t s);
hipError_t launch_reg48(const RegArgs &a, maskgs_dtype w_dt, hipStream_t s);
hipError_t launch_hard48(const HardArgs &a, hipStream_t s);
hipError_t launch_prior48(const PriorArgs &a, maskgs_dtype w_dt, hipStream_t s);
hipError_t launch_stats48(const StatsArgs &a, bool sampled, maskgs_dtype w_dt, hipStream_t s);

hipError_t launch_debug_philox(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                               int64_t count, uint32_t *words, hipStream_t s);
hipError_t launch_debug_gumbel(const uint32_t *words, int64_t n, float *g, hipStream_t s);

}  // namespace maskgs
