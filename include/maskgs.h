/*
 * maskgs.h -- C ABI of libmaskgs: the differentiable N:M mask path of MaskLLM
 * ("MaskLLM: Learnable Semi-Structured Sparsity for Large Language Models",
 * arXiv 2409.17481; citations below name sections of its paper-graph-ui
 * summary page) on AMD Instinct MI355X (gfx950).
 *
 * Every block of M consecutive weights of a frozen weight matrix carries K =
 * C(M,N) learnable fp32 logits z (one per candidate N:M mask).  The library
 * draws Gumbel noise for every (block, candidate) from a counter-based Philox
 * stream, forms the soft index y = softmax((kappa*z + g)/tau), the soft mask
 * M~ = y.S and W (.) M~; it maps the upstream gradient plus the sparse-weight
 * regulariser back to dL/dz; it extracts, packs and compacts the hard mask
 * argmax(z); and it seeds logits from a prior mask.
 *
 * Conventions shared by all entry points
 *   Layout.   W, W(.)M~ and the upstream gradient are row-major [rows, cols];
 *             block b = r*(cols/M) + c covers W[r, c*M .. c*M+M-1] (blocks run
 *             along the contiguous, input dimension).  Logits, soft indices and
 *             logit gradients are fp32 [B, K] with K innermost, B = rows*cols/M.
 *   Support.  N:M = 2:4 (K = 6) and 4:8 (K = 70) on the GPU.
 *   Memory.   Every array argument is device memory owned by the caller, except
 *             where a comment says "host".  The library allocates nothing and
 *             keeps no state between calls that affects results (only a cache
 *             of each device's compute-unit count, for launch sizes); calls
 *             are thread safe.
 *             Every device pointer must be 16-byte aligned.  Outputs must not
 *             alias inputs except where stated (prior_init updates z in place,
 *             bwd with accumulate reads and writes dz).
 *   Streams.  Work is enqueued on the given HIP stream (0 = null stream) and
 *             runs asynchronously; faults surface at the caller's synchronise.
 *             Calls may be captured in a HIP graph: every argument, the
 *             sample parameters included, is fixed at capture, and the arrays
 *             are read when the graph runs.
 *   Errors.   Each call returns MASKGS_OK (0) or a MASKGS_E_* status.  All
 *             argument checks run on the host before anything is enqueued: on
 *             an error status nothing has been launched.  The descriptor, the
 *             scalars and the combination of arguments are checked first; a
 *             tensor with no blocks (rows or cols 0) then returns MASKGS_OK
 *             and launches nothing (the array pointers of its data are not
 *             checked).  Data-dependent conditions (NaN logits, priors
 *             matching no candidate) are not errors; their behaviour is stated
 *             per entry point.
 */
#ifndef MASKGS_H
#define MASKGS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MASKGS_ABI_VERSION 2

/* Status codes. */
#define MASKGS_OK 0
#define MASKGS_E_NULL 1        /* a required pointer is NULL                      */
#define MASKGS_E_SHAPE 2       /* rows/cols negative, cols % M != 0, or past the
                                  size limits of maskgs_tensor_desc             */
#define MASKGS_E_UNSUPPORTED 3 /* N:M other than 2:4 / 4:8, a 2:4-only output, or
                                  a saved y under MASKGS_HARD_SAMPLE            */
#define MASKGS_E_DTYPE 4       /* dtype code out of range                         */
#define MASKGS_E_ALIGN 5       /* a device pointer is not 16-byte aligned         */
#define MASKGS_E_RANGE 6       /* kappa<=0, tau<=0, lambda<0, alpha<0, non-finite, bad mode */
#define MASKGS_E_HIP 7         /* the HIP runtime refused a launch                */
#define MASKGS_E_CAPACITY 8    /* a host output buffer is too small               */

/* Element types of weights, masked weights and upstream gradients.  The two
 * sentinels make every int32 value a valid maskgs_dtype for a C++
 * implementation, so that an out-of-range code passed by a C caller is
 * answered with MASKGS_E_DTYPE rather than being undefined; they are not
 * element types. */
typedef enum {
    MASKGS_F32 = 0,
    MASKGS_BF16 = 1,
    MASKGS_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    MASKGS_DTYPE_RANGE_MAX_ = 2147483647
} maskgs_dtype;

/* Sample flags. */
#define MASKGS_NO_NOISE 1u /* g = 0 for every candidate (tests and diagnostics) */
/* Hard Gumbel-max sample with a straight-through gradient (section 3.4, Eq. 5:
 * the first argmax k of the perturbed logits a is a draw from softmax(kappa z)).
 * Forward: W (.) S_k and its regulariser instead of W (.) M~; the soft index y
 * is still computed and saved.  Backward: the softmax Jacobian of y, with the
 * regulariser term taken at S_k.  The backward needs k, so it recomputes y
 * from z: with a saved y it returns MASKGS_E_UNSUPPORTED. */
#define MASKGS_HARD_SAMPLE 2u

/* One weight tensor (or a row range of one).  block_offset is the global index
 * of the first block described: the noise of a block depends on its global
 * index, so a tensor split into row ranges with matching offsets draws exactly
 * the noise of the whole tensor.  tensor_id separates the noise streams of the
 * layers of a model.  Limits (MASKGS_E_SHAPE beyond them): block_offset at most
 * 2^56, and rows * (cols/m) * 80 at most 2^56, so that every element index and
 * Philox word index fits 64 bits. */
typedef struct {
    int32_t n, m;          /* N:M pattern: keep n of every m weights             */
    int64_t rows, cols;    /* weight shape [rows, cols]                          */
    uint64_t block_offset; /* global index of block 0 of this call               */
    uint32_t tensor_id;    /* noise stream of this tensor                        */
} maskgs_tensor_desc;

/* One draw of the Gumbel soft index.  The Philox4x32-10 stream (Salmon et al.,
 * SC'11) gives word n = global_block*K + candidate as output n%4 of the call
 * with counter (lo32(n/4), hi32(n/4), step, tensor_id) and key (lo32(seed),
 * hi32(seed)).  kappa and tau follow the schedules of section 3.4 (kappa
 * 100 -> 500, tau 4 -> 0.05); the caller evaluates the schedule per step. */
typedef struct {
    uint64_t seed;
    uint32_t step;
    float kappa; /* logit scale, > 0 (section 3.4, logit parameterisation)  */
    float tau;   /* temperature, > 0 (section 3.4, Eq. 6)                   */
    uint32_t flags;
} maskgs_sample_params;

/* Library version of this header's ABI (MASKGS_ABI_VERSION). */
int maskgs_abi_version(void);

/* Static text for a status code (never NULL). */
const char *maskgs_status_str(int status);

/* Candidate masks S (section 3.2 candidate set; section 3.4 Eq. 7).  Writes the
 * K = C(m,n) masks to masks_host (HOST memory, capacity entries) as bitmasks,
 * bit j set = keep position j.  Order: for 2:4 the order in which the page
 * lists the six patterns ([1,1,0,0],[1,0,1,0],[1,0,0,1],[0,1,0,1],[0,1,1,0],
 * [0,0,1,1], first position = bit 0); for 4:8 lexicographic order of the sorted
 * kept positions.  *k_out = K (may be NULL).  E_UNSUPPORTED for other N:M,
 * E_CAPACITY if capacity < K (nothing written). */
int maskgs_candidates(int32_t n, int32_t m, uint8_t *masks_host, int32_t capacity, int32_t *k_out);

/* Forward of the mask path (section 3.4, Eqs. 5-7 and Algorithm 1; section 3.2
 * frozen backbone).  Per block: g_i Gumbel noise (Eq. 5), a_i =
 * fp32(fp32(kappa*z_i + g_i) * fp32(1/tau)), y = softmax(a) (Eq. 6),
 * m = y.S (Eq. 7), out = W (.) m.
 *   w        [rows, cols] of w_dt, frozen weight.
 *   z        [B, K] fp32 logits.
 *   out      [rows, cols] of out_dt: W (.) M~ (bf16: round to nearest even).
 *   y_save   NULL, or [B, K] fp32: the soft index, for maskgs_bwd.
 *   reg_accum NULL, or ONE device double to which sum_b ||W_b (.) M~_b||^2 is
 *            added atomically (the regulariser value R of Eq. 8; the loss term
 *            is -lambda*R).  The caller zeroes it.
 * NaN logits propagate to y, out and R. */
int maskgs_fwd(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
               maskgs_dtype w_dt, const float *z, void *out, maskgs_dtype out_dt, float *y_save,
               double *reg_accum, hipStream_t stream);

/* Forward plus the hard mask of the same logits: the outputs of maskgs_fwd and
 * those of maskgs_hard_extract on z (idx, mask_bits, and for 2:4 values and
 * val_idx, each NULL to skip; formats as documented there), bit-identical to
 * the two calls in sequence, with z and w read once.  The per-step hard mask
 * is what the mask-change and maximum-probability diagnostics of section 3.4
 * (kappa sweep, Figure 5) track during training.  values/val_idx for 4:8
 * return MASKGS_E_UNSUPPORTED. */
int maskgs_fwd_hard(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                    maskgs_dtype w_dt, const float *z, void *out, maskgs_dtype out_dt,
                    float *y_save, double *reg_accum, uint8_t *idx, uint8_t *mask_bits,
                    void *values, uint8_t *val_idx, hipStream_t stream);

/* Backward to the logits (section 3.2 information flow; section 3.4 Eq. 8).
 * With G = dL_LM/d(W (.) M~) and W frozen, the gradient of
 * L = L_LM - lambda * sum_b ||W_b (.) M~_b||^2 is, per block,
 *   dm_j = G_j w_j - 2 lambda w_j^2 m_j,   dy_i = sum_j S_ij dm_j,
 *   dz_i = (kappa/tau) y_i (dy_i - sum_k y_k dy_k).
 *   y_saved  NULL (recompute y from z with the same seed/step: bit-identical to
 *            the forward's), or the y_save written by maskgs_fwd.
 *   z        [B, K]; may be NULL when y_saved is given.
 *   dout     [rows, cols] of dout_dt, G.
 *   dz       [B, K] fp32 output; accumulate != 0 adds to its contents. */
int maskgs_bwd(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
               maskgs_dtype w_dt, const float *z, const float *y_saved, const void *dout,
               maskgs_dtype dout_dt, float lambda, float *dz, int32_t accumulate,
               hipStream_t stream);

/* AdamW hyperparameters of maskgs_bwd_adamw (section 3.4, Algorithm 1 "update
 * logits", and the training details: AdamW, lr 5e-4 for LLaMA-2 and Nemotron,
 * 1e-3 for GPT-3, weight decay 0.1).  The pages give no beta1, beta2 or eps;
 * Adam's published defaults are 0.9, 0.999 and 1e-8.  The weight decay is
 * decoupled from the moments and scaled by lr. */
typedef struct {
    float lr;           /* >= 0                                              */
    float beta1, beta2; /* in [0, 1)                                         */
    float eps;          /* > 0                                               */
    float weight_decay; /* >= 0                                              */
    uint32_t t;         /* updates so far including this one (>= 1), for the */
                        /* bias corrections 1 - beta^t                       */
} maskgs_adamw_params;

/* Backward to the logits fused with their AdamW update (section 3.4,
 * Algorithm 1: backpropagate, then update the logits).  dz is computed exactly
 * as maskgs_bwd with accumulate = 0 stores it (fp32) but is never written;
 * instead, per logit,
 *   m = b1 m + (1 - b1) dz,   v = b2 v + (1 - b2) dz^2,
 *   z = z - lr (m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + wd z),
 * with z on the right the logits before this update.
 *   z          [B, K] fp32, in-out: read for the soft index when y_saved is
 *              NULL and for the update, then overwritten with the new logits.
 *   y_saved    NULL (recompute y from z before the update, bit-identical to the
 *              forward's) or the y_save of maskgs_fwd.
 *   exp_avg, exp_avg_sq  [B, K] fp32 first and second moments, in-out (zero
 *              before the first update).
 *   opt        HOST pointer to the hyperparameters.
 * Other arguments as in maskgs_bwd.  E_RANGE for lr < 0, beta outside [0, 1),
 * eps <= 0, weight_decay < 0, t = 0 or a non-finite value.  z, exp_avg and
 * exp_avg_sq must not alias each other or any input. */
int maskgs_bwd_adamw(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                     maskgs_dtype w_dt, float *z, const float *y_saved, const void *dout,
                     maskgs_dtype dout_dt, float lambda, float *exp_avg, float *exp_avg_sq,
                     const maskgs_adamw_params *opt, hipStream_t stream);

/* Training diagnostics of one tensor, as sums that maskgs_mask_stats adds to a
 * DEVICE struct (the caller zeroes it; tensors and steps accumulate).  They are
 * the quantities the pages plot: the mask change between training steps and
 * the maximum probability of the learned distribution (section 3.4, kappa
 * discussion, Figure 5), the weight norm the mask keeps against magnitude
 * pruning (Figure 6), the mask difference between two masks (Figure 8) and the
 * logit gradient norm (Table 14). */
typedef struct {
    uint64_t blocks;     /* blocks counted                                        */
    uint64_t changed;    /* blocks whose hard mask differs from ref_bits          */
    double max_prob;     /* sum over blocks of max_i softmax(kappa z)_i           */
    double kept_l1;      /* sum of |w| at the kept positions of the hard mask     */
    double magnitude_l1; /* sum of |w| at the magnitude top-n positions           */
    double grad_sq;      /* sum of dz^2 over all logits                           */
} maskgs_stats;

/* Adds the diagnostics of one tensor to *stats (device, 16-byte aligned):
 *   z        [B, K] logits (required).  The hard mask of block b is S[k_b],
 *            k_b the first index of the largest z_b,i, or, when sample is not
 *            NULL, the first index of the largest perturbed logit
 *            a_i = fp32(fp32(kappa z_i + g_i) fp32(1/tau)) of that draw (the
 *            Gumbel-max sample, section 3.4 Eq. 5; block_offset and tensor_id of
 *            t select the noise as in maskgs_fwd).
 *   kappa    >= 0, the scale of max_prob's softmax(kappa z).
 *   ref_bits NULL, or packed masks (maskgs_hard_extract's mask_bits format):
 *            changed counts the blocks whose hard mask differs.
 *   w        NULL, or the weight [rows, cols] of w_dt: kept_l1 and magnitude_l1
 *            (magnitude top-n as in maskgs_prior_init).
 *   dz       NULL, or [B, K] fp32 logit gradients: grad_sq.
 * max_prob always accumulates; blocks counts every block of t.  The sums use
 * device atomics, so their fp64 rounding order varies between runs. */
int maskgs_mask_stats(const maskgs_tensor_desc *t, const float *z, float kappa,
                      const maskgs_sample_params *sample, const uint8_t *ref_bits, const void *w,
                      maskgs_dtype w_dt, const float *dz, maskgs_stats *stats,
                      hipStream_t stream);

/* Regulariser value alone (section 3.4, Eq. 8): adds sum_b ||W_b (.) M~_b||^2 to
 * *reg_accum (one device double, atomically) without writing W (.) M~.
 * y_saved as in maskgs_bwd. */
int maskgs_reg_reduce(const maskgs_tensor_desc *t, const maskgs_sample_params *p, const void *w,
                      maskgs_dtype w_dt, const float *z, const float *y_saved,
                      double *reg_accum, hipStream_t stream);

/* Hard mask (section 3.2 inference flow; Algorithm 1 step 3): k_b = the first
 * index of the largest z_b,i (fp32 compare), M*_b = S_k.  Outputs, each NULL
 * to skip:
 *   idx       [B] uint8, k_b.
 *   mask_bits [ceil(B*m/8)] uint8: M*_b at bits [b*m, b*m+m) of an LSB-first
 *             bit stream; the unused bits of the last byte are zero.
 *   values    2:4 only, [B*2] of w_dt: the kept weights of block b in ascending
 *             position at [2b], [2b+1] (bit copies of w; needs w).
 *   val_idx   2:4 only, [ceil(B/2)] uint8: nibble p0 | p1<<2 of the two kept
 *             positions (p0 < p1); block 2i in the low nibble of byte i, block
 *             2i+1 in the high nibble; the unused high nibble is zero.
 * block_offset and tensor_id of t are ignored.  A block whose logits are all
 * NaN selects candidate 0. */
int maskgs_hard_extract(const maskgs_tensor_desc *t, const float *z, const void *w,
                        maskgs_dtype w_dt, uint8_t *idx, uint8_t *mask_bits, void *values,
                        uint8_t *val_idx, hipStream_t stream);

/* Prior seeding (section 3.4, Mask Prior, Eqs. 9-10), z updated in place.
 * The prior M0 of block b is read from prior_bits (the mask_bits format), or,
 * when prior_bits is NULL, is the magnitude top-n of w (|w| compared on the
 * bit pattern with the sign cleared; ties keep the lower position).
 *   mode 0 (Eq. 10): z_i <- z_i + alpha * sigma_b * sim_i, sim_i = <M0,S_i> -
 *          mean_k <M0,S_k>, sigma_b the population std of the block's K logits.
 *   mode 1: z_k0 <- z_k0 + alpha at the candidate S_k0 = M0; a block whose
 *          prior has no equal candidate is left unchanged.
 * alpha >= 0 (alpha = 0 leaves z unchanged). */
int maskgs_prior_init(const maskgs_tensor_desc *t, float *z, const uint8_t *prior_bits,
                      const void *w, maskgs_dtype w_dt, float alpha, int32_t mode,
                      hipStream_t stream);

/* Test hooks.  maskgs_debug_philox writes words n0 .. n0+count-1 of the noise
 * stream of (seed, step, tensor_id) to words (device, count uint32).
 * maskgs_debug_gumbel maps n Philox words to the fp32 Gumbel noise the forward
 * uses (device arrays). */
int maskgs_debug_philox(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                        int64_t count, uint32_t *words, hipStream_t stream);
int maskgs_debug_gumbel(const uint32_t *words, int64_t n, float *g, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MASKGS_H */
