// maskgs_api.hip -- C ABI of libmaskgs: argument checks, launch geometry and
// dispatch to the gfx950 kernels (maskgs_k24.hip: 2:4, maskgs_k48.hip: 4:8).
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "maskgs.h"
#include "maskgs_device.hpp"
#include "maskgs_launch.hpp"
#include "maskpro.h"
#include "maskpro_launch.hpp"

namespace maskgs {

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace maskgs

using namespace maskgs;

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool valid_dtype(maskgs_dtype d) { return d == MASKGS_F32 || d == MASKGS_BF16; }

// Checks a tensor description; fills the geometry on success.
int check_desc(const maskgs_tensor_desc *t, Geometry *g) {
    if (!t) return MASKGS_E_NULL;
    if (!((t->n == 2 && t->m == 4) || (t->n == 4 && t->m == 8))) return MASKGS_E_UNSUPPORTED;
    if (t->rows < 0 || t->cols < 0 || t->cols % t->m != 0) return MASKGS_E_SHAPE;
    const int64_t bpr = t->cols / t->m;
    // rows * bpr * 80 <= 2^56, tested without forming a product that could
    // overflow: bpr is bounded first, so bpr * 80 <= 2^56 below
    constexpr int64_t kLimit = INT64_C(1) << 56;
    if (bpr > kLimit / 80) return MASKGS_E_SHAPE;
    if (bpr != 0 && t->rows > kLimit / (bpr * 80)) return MASKGS_E_SHAPE;
    g->n = t->n;
    g->m = t->m;
    g->k = (t->m == 4) ? 6 : 70;
    g->nblocks = t->rows * bpr;
    g->block_offset = t->block_offset;
    g->tensor_id = t->tensor_id;
    if (t->block_offset > (UINT64_C(1) << 56)) return MASKGS_E_SHAPE;
    return MASKGS_OK;
}

int check_params(const maskgs_sample_params *p, Noise *nz) {
    if (!p) return MASKGS_E_NULL;
    if (!std::isfinite(p->kappa) || !std::isfinite(p->tau) || !(p->kappa > 0.0f) ||
        !(p->tau > 0.0f))
        return MASKGS_E_RANGE;
    const float tau_inv = 1.0f / p->tau;
    if (!std::isfinite(tau_inv)) return MASKGS_E_RANGE;
    nz->k0 = static_cast<uint32_t>(p->seed);
    nz->k1 = static_cast<uint32_t>(p->seed >> 32);
    nz->step = p->step;
    nz->kappa = p->kappa;
    nz->tau_inv = tau_inv;
    nz->grad_scale = static_cast<double>(p->kappa) / static_cast<double>(p->tau);
    nz->no_noise = (p->flags & MASKGS_NO_NOISE) ? 1u : 0u;
    nz->hard_sample = (p->flags & MASKGS_HARD_SAMPLE) ? 1u : 0u;
    return MASKGS_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MASKGS_OK : MASKGS_E_HIP; }

}  // namespace

extern "C" {

int maskgs_abi_version(void) { return MASKGS_ABI_VERSION; }

const char *maskgs_status_str(int status) {
    switch (status) {
        case MASKGS_OK: return "ok";
        case MASKGS_E_NULL: return "a required pointer is NULL";
        case MASKGS_E_SHAPE: return "invalid shape (negative size, cols not a multiple of M, or too large)";
        case MASKGS_E_UNSUPPORTED: return "unsupported N:M pattern, output for this pattern, or argument combination";
        case MASKGS_E_DTYPE: return "invalid dtype code";
        case MASKGS_E_ALIGN: return "a device pointer is not 16-byte aligned";
        case MASKGS_E_RANGE: return "scalar argument out of range (kappa, tau > 0; lambda, alpha >= 0; finite; mode 0/1)";
        case MASKGS_E_HIP: return "HIP runtime error at launch";
        case MASKGS_E_CAPACITY: return "host output buffer too small";
        default: return "unknown status";
    }
}

int maskgs_candidates(int32_t n, int32_t m, uint8_t *masks_host, int32_t capacity,
                      int32_t *k_out) {
    if (!masks_host) return MASKGS_E_NULL;
    if (n == 2 && m == 4) {
        if (capacity < 6) return MASKGS_E_CAPACITY;
        for (int i = 0; i < 6; ++i) masks_host[i] = Cands<2, 4>::mask[i];
        if (k_out) *k_out = 6;
        return MASKGS_OK;
    }
    if (n == 4 && m == 8) {
        if (capacity < 70) return MASKGS_E_CAPACITY;
        for (int i = 0; i < 70; ++i) masks_host[i] = Cands<4, 8>::at(i);
        if (k_out) *k_out = 70;
        return MASKGS_OK;
    }
    return MASKGS_E_UNSUPPORTED;
}

int maskgs_fwd(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
               maskgs_dtype w_dt, const float *z, void *out, maskgs_dtype out_dt, float *y_save,
               double *reg_accum, hipStream_t stream) {
    Geometry g;
    Noise nz;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((rc = check_params(p, &nz))) return rc;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!w || !z || !out) return MASKGS_E_NULL;
    if (!valid_dtype(w_dt) || !valid_dtype(out_dt)) return MASKGS_E_DTYPE;
    if (misaligned(w) || misaligned(z) || misaligned(out) || misaligned(y_save) ||
        misaligned(reg_accum))
        return MASKGS_E_ALIGN;
    FwdArgs a{w, z, out, y_save, reg_accum, g, nz};
    if (g.m == 4) return launch_status(launch_fwd24(a, w_dt, out_dt, stream));
    return launch_status(launch_fwd48(a, w_dt, out_dt, stream));
}

int maskgs_fwd_hard(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                    maskgs_dtype w_dt, const float *z, void *out, maskgs_dtype out_dt,
                    float *y_save, double *reg_accum, uint8_t *idx, uint8_t *mask_bits,
                    void *values, uint8_t *val_idx, hipStream_t stream) {
    Geometry g;
    Noise nz;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((rc = check_params(p, &nz))) return rc;
    if ((values || val_idx) && g.m != 4) return MASKGS_E_UNSUPPORTED;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!w || !z || !out) return MASKGS_E_NULL;
    if (!valid_dtype(w_dt) || !valid_dtype(out_dt)) return MASKGS_E_DTYPE;
    if (misaligned(w) || misaligned(z) || misaligned(out) || misaligned(y_save) ||
        misaligned(reg_accum) || misaligned(idx) || misaligned(mask_bits) || misaligned(values) ||
        misaligned(val_idx))
        return MASKGS_E_ALIGN;
    FwdArgs a{w, z, out, y_save, reg_accum, g, nz, idx, mask_bits, values, val_idx};
    if (g.m == 4) return launch_status(launch_fwd24(a, w_dt, out_dt, stream));
    return launch_status(launch_fwd48(a, w_dt, out_dt, stream));
}

int maskgs_bwd(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
               maskgs_dtype w_dt, const float *z, const float *y_saved, const void *dout,
               maskgs_dtype dout_dt, float lambda, float *dz, int32_t accumulate,
               hipStream_t stream) {
    Geometry g;
    Noise nz;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((rc = check_params(p, &nz))) return rc;
    if (!std::isfinite(lambda) || lambda < 0.0f) return MASKGS_E_RANGE;
    if (nz.hard_sample && y_saved) return MASKGS_E_UNSUPPORTED;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!w || !dout || !dz || (!z && !y_saved)) return MASKGS_E_NULL;
    if (!valid_dtype(w_dt) || !valid_dtype(dout_dt)) return MASKGS_E_DTYPE;
    if (misaligned(w) || misaligned(z) || misaligned(y_saved) || misaligned(dout) ||
        misaligned(dz))
        return MASKGS_E_ALIGN;
    BwdArgs a{w, z, y_saved, dout, dz, static_cast<double>(lambda), accumulate != 0, g, nz};
    if (g.m == 4) return launch_status(launch_bwd24(a, w_dt, dout_dt, stream));
    return launch_status(launch_bwd48(a, w_dt, dout_dt, stream));
}

int maskgs_bwd_adamw(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                     maskgs_dtype w_dt, float *z, const float *y_saved, const void *dout,
                     maskgs_dtype dout_dt, float lambda, float *exp_avg, float *exp_avg_sq,
                     const maskgs_adamw_params *opt, hipStream_t stream) {
    Geometry g;
    Noise nz;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((rc = check_params(p, &nz))) return rc;
    if (!opt) return MASKGS_E_NULL;
    if (!std::isfinite(lambda) || lambda < 0.0f) return MASKGS_E_RANGE;
    const float vals[5] = {opt->lr, opt->beta1, opt->beta2, opt->eps, opt->weight_decay};
    for (float v : vals)
        if (!std::isfinite(v)) return MASKGS_E_RANGE;
    if (opt->lr < 0.0f || !(opt->beta1 >= 0.0f && opt->beta1 < 1.0f) ||
        !(opt->beta2 >= 0.0f && opt->beta2 < 1.0f) || !(opt->eps > 0.0f) ||
        opt->weight_decay < 0.0f || opt->t == 0)
        return MASKGS_E_RANGE;
    if (nz.hard_sample && y_saved) return MASKGS_E_UNSUPPORTED;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!w || !dout || !z || !exp_avg || !exp_avg_sq) return MASKGS_E_NULL;
    if (!valid_dtype(w_dt) || !valid_dtype(dout_dt)) return MASKGS_E_DTYPE;
    if (misaligned(w) || misaligned(z) || misaligned(y_saved) || misaligned(dout) ||
        misaligned(exp_avg) || misaligned(exp_avg_sq))
        return MASKGS_E_ALIGN;
    BwdArgs a{w, z, y_saved, dout, nullptr, static_cast<double>(lambda), false, g, nz};
    a.zu = z;
    a.m1 = exp_avg;
    a.m2 = exp_avg_sq;
    const double t_d = static_cast<double>(opt->t);
    a.adam.lr = opt->lr;
    a.adam.b1 = opt->beta1;
    a.adam.omb1 = static_cast<float>(1.0 - static_cast<double>(opt->beta1));
    a.adam.b2 = opt->beta2;
    a.adam.omb2 = static_cast<float>(1.0 - static_cast<double>(opt->beta2));
    a.adam.ibc1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(opt->beta1), t_d)));
    a.adam.ibc2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(opt->beta2), t_d)));
    a.adam.eps = opt->eps;
    a.adam.wd = opt->weight_decay;
    if (!std::isfinite(a.adam.ibc1) || !std::isfinite(a.adam.ibc2)) return MASKGS_E_RANGE;
    if (g.m == 4) return launch_status(launch_bwd24(a, w_dt, dout_dt, stream));
    return launch_status(launch_bwd48(a, w_dt, dout_dt, stream));
}

int maskgs_mask_stats(const maskgs_tensor_desc *t, const float *z, float kappa,
                      const maskgs_sample_params *sample, const uint8_t *ref_bits, const void *w,
                      maskgs_dtype w_dt, const float *dz, maskgs_stats *stats,
                      hipStream_t stream) {
    Geometry g;
    Noise nz{};
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if (sample && (rc = check_params(sample, &nz))) return rc;
    if (!std::isfinite(kappa) || kappa < 0.0f) return MASKGS_E_RANGE;
    if (!stats) return MASKGS_E_NULL;
    if (misaligned(stats)) return MASKGS_E_ALIGN;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!z) return MASKGS_E_NULL;
    if (w && !valid_dtype(w_dt)) return MASKGS_E_DTYPE;
    if (misaligned(z) || misaligned(ref_bits) || misaligned(w) || misaligned(dz))
        return MASKGS_E_ALIGN;
    StatsArgs a{z, ref_bits, w, dz, stats, kappa * 1.44269504088896341f, g, nz};
    if (g.m == 4) return launch_status(launch_stats24(a, sample != nullptr, w_dt, stream));
    return launch_status(launch_stats48(a, sample != nullptr, w_dt, stream));
}

int maskgs_reg_reduce(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                      maskgs_dtype w_dt, const float *z, const float *y_saved,
                      double *reg_accum, hipStream_t stream) {
    Geometry g;
    Noise nz;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((rc = check_params(p, &nz))) return rc;
    if (nz.hard_sample && y_saved) return MASKGS_E_UNSUPPORTED;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!w || !reg_accum || (!z && !y_saved)) return MASKGS_E_NULL;
    if (!valid_dtype(w_dt)) return MASKGS_E_DTYPE;
    if (misaligned(w) || misaligned(z) || misaligned(y_saved) || misaligned(reg_accum))
        return MASKGS_E_ALIGN;
    RegArgs a{w, z, y_saved, reg_accum, g, nz};
    if (g.m == 4) return launch_status(launch_reg24(a, w_dt, stream));
    return launch_status(launch_reg48(a, w_dt, stream));
}

int maskgs_hard_extract(const maskgs_tensor_desc *t, const float *z, const void *w,
                        maskgs_dtype w_dt, uint8_t *idx, uint8_t *mask_bits, void *values,
                        uint8_t *val_idx, hipStream_t stream) {
    Geometry g;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if ((values || val_idx) && g.m != 4) return MASKGS_E_UNSUPPORTED;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!z) return MASKGS_E_NULL;
    if (values && !w) return MASKGS_E_NULL;
    if (values && !valid_dtype(w_dt)) return MASKGS_E_DTYPE;
    if (misaligned(z) || misaligned(idx) || misaligned(mask_bits) || misaligned(values) ||
        misaligned(val_idx) || (values && misaligned(w)))
        return MASKGS_E_ALIGN;
    HardArgs a{z, w, idx, mask_bits, values, val_idx, g};
    if (g.m == 4) return launch_status(launch_hard24(a, w_dt, stream));
    return launch_status(launch_hard48(a, stream));
}

int maskgs_prior_init(const maskgs_tensor_desc *t, float *z, const uint8_t *prior_bits,
                      const void *w, maskgs_dtype w_dt, float alpha, int32_t mode,
                      hipStream_t stream) {
    Geometry g;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if (!std::isfinite(alpha) || alpha < 0.0f || (mode != 0 && mode != 1)) return MASKGS_E_RANGE;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!z || (!prior_bits && !w)) return MASKGS_E_NULL;
    if (!prior_bits && !valid_dtype(w_dt)) return MASKGS_E_DTYPE;
    if (misaligned(z) || misaligned(prior_bits) || (!prior_bits && misaligned(w)))
        return MASKGS_E_ALIGN;
    PriorArgs a{z, prior_bits, w, static_cast<double>(alpha), mode, g};
    if (g.m == 4) return launch_status(launch_prior24(a, w_dt, stream));
    return launch_status(launch_prior48(a, w_dt, stream));
}

int maskgs_debug_philox(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                        int64_t count, uint32_t *words, hipStream_t stream) {
    if (!words) return MASKGS_E_NULL;
    if (count < 0) return MASKGS_E_SHAPE;
    if (misaligned(words)) return MASKGS_E_ALIGN;
    if (count == 0) return MASKGS_OK;
    return launch_status(launch_debug_philox(seed, step, tensor_id, n0, count, words, stream));
}

int maskgs_debug_gumbel(const uint32_t *words, int64_t n, float *g, hipStream_t stream) {
    if (!words || !g) return MASKGS_E_NULL;
    if (n < 0) return MASKGS_E_SHAPE;
    if (misaligned(words) || misaligned(g)) return MASKGS_E_ALIGN;
    if (n == 0) return MASKGS_OK;
    return launch_status(launch_debug_gumbel(words, n, g, stream));
}

/* ------------------------------------------------------------------------- */
/* Linear-space mask learner (maskpro.h).                                    */
/* ------------------------------------------------------------------------- */

static int mp_common(const maskgs_tensor_desc *t, const maskpro_draw_params *p, MpArgs *a,
                     int *m) {
    Geometry g;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if (!p) return MASKGS_E_NULL;
    *a = MpArgs{};
    a->nblocks = g.nblocks;
    a->block_offset = g.block_offset;
    a->tensor_id = g.tensor_id;
    a->k0 = static_cast<uint32_t>(p->seed);
    a->k1 = static_cast<uint32_t>(p->seed >> 32);
    a->step = p->step;
    a->no_noise = (p->flags & MASKGS_NO_NOISE) ? 1u : 0u;
    *m = g.m;
    return MASKGS_OK;
}

int maskpro_fwd(const maskgs_tensor_desc *t, const maskpro_draw_params *p, const void *w,
                maskgs_dtype w_dt, const float *pi, void *out, maskgs_dtype out_dt,
                uint8_t *mask_bits, void *order, hipStream_t stream) {
    MpArgs a;
    int m = 0;
    int rc = mp_common(t, p, &a, &m);
    if (rc) return rc;
    if (a.nblocks == 0) return MASKGS_OK;
    if (!pi || (out && !w)) return MASKGS_E_NULL;
    if (out && (!valid_dtype(w_dt) || !valid_dtype(out_dt))) return MASKGS_E_DTYPE;
    if (misaligned(pi) || misaligned(mask_bits) || misaligned(order) ||
        (out && (misaligned(out) || misaligned(w))))
        return MASKGS_E_ALIGN;
    if (!out && !mask_bits && !order) return MASKGS_OK;
    a.w = w;
    a.pi = pi;
    a.out = out;
    a.bits = mask_bits;
    a.order = order;
    return launch_status(launch_mp_fwd(a, m, w_dt, out_dt, stream));
}

int maskpro_bwd(const maskgs_tensor_desc *t, const maskpro_draw_params *p, const float *pi,
                const void *order, float advantage, float *dpi, int32_t accumulate,
                hipStream_t stream) {
    MpArgs a;
    int m = 0;
    int rc = mp_common(t, p, &a, &m);
    if (rc) return rc;
    if (!std::isfinite(advantage)) return MASKGS_E_RANGE;
    if (a.nblocks == 0) return MASKGS_OK;
    if (!pi || !dpi) return MASKGS_E_NULL;
    if (misaligned(pi) || misaligned(order) || misaligned(dpi)) return MASKGS_E_ALIGN;
    a.pi = pi;
    a.order_in = order;
    a.dpi = dpi;
    a.adv = advantage;
    a.accumulate = accumulate ? 1u : 0u;
    return launch_status(launch_mp_bwd(a, m, stream));
}

int maskpro_init(const maskgs_tensor_desc *t, const uint8_t *prior_bits, const void *w,
                 maskgs_dtype w_dt, float c, float *pi, hipStream_t stream) {
    Geometry g;
    int rc = check_desc(t, &g);
    if (rc) return rc;
    if (!std::isfinite(c)) return MASKGS_E_RANGE;
    if (g.nblocks == 0) return MASKGS_OK;
    if (!pi || (!prior_bits && !w)) return MASKGS_E_NULL;
    if (!prior_bits && !valid_dtype(w_dt)) return MASKGS_E_DTYPE;
    if (misaligned(pi) || misaligned(prior_bits) || (!prior_bits && misaligned(w)))
        return MASKGS_E_ALIGN;
    MpInitArgs a{prior_bits, w, c, pi, g.nblocks};
    return launch_status(launch_mp_init(a, g.m, w_dt, stream));
}

int maskpro_baseline(double residual, double mu, double *baseline, double *advantage) {
    if (!baseline || !advantage) return MASKGS_E_NULL;
    if (!std::isfinite(residual) || !(mu >= 0.0 && mu <= 1.0) || !std::isfinite(*baseline))
        return MASKGS_E_RANGE;
    const double b = *baseline;
    *advantage = residual - b;
    *baseline = mu * b + (1.0 - mu) * residual;
    return MASKGS_OK;
}

}  // extern "C"
