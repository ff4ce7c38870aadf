/*
 * maskpro.h -- C ABI of the linear-space N:M mask learner of libmaskgs,
 * following MaskPro ("MaskPro: Linear-Space Probabilistic Learning for Strict
 * (N:M)-Sparsity on LLMs"; citations below name sections of its atlas.scime.ai
 * summary page) on AMD Instinct MI355X (gfx950).
 *
 * Every block of M consecutive weights carries M fp32 logits pi, one
 * categorical distribution over its positions ("Approach": linear space, one
 * logit per weight, against C(M,N) per block for MaskLLM).  A step draws N of
 * the M positions without replacement, applies that hard mask to the frozen
 * weights, and, given the scalar advantage of the step's loss, forms the
 * policy gradient of the logits.
 *
 * The conventions of maskgs.h hold: layout (block b = r*(cols/M) + c covers
 * W[r, c*M .. c*M+M-1]; logits and their gradients are fp32 [B, M], M
 * innermost), caller-owned 16-byte-aligned device memory, no allocation, no
 * state, asynchronous work on the given stream, MASKGS_* status codes with
 * every check on the host before any launch.  N:M = 2:4 and 4:8.
 *
 * The draw.  Position j of global block gb gets the key
 *   a_j = fp32(pi_j + g_j),
 * g_j the Gumbel variate of maskgs.h's noise contract from Philox word
 * n = gb*M + j of (seed, step, tensor_id).  The drawn positions j_1..j_N are
 * those of the N largest keys in descending order (ties and NaN keys: the
 * lower position first).  This is the Gumbel-top-k construction of a
 * sequential draw without replacement from softmax(pi) (Kool, van Hoof,
 * Welling, ICML 2019), whose ordered outcome has the Plackett-Luce
 * probability p(j_1..j_N) = prod_k softmax(pi restricted to the positions
 * not yet drawn)_{j_k}.
 */
#ifndef MASKPRO_H
#define MASKPRO_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "maskgs.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One draw.  flags: MASKGS_NO_NOISE makes the keys pi itself, so the draw is
 * the N most likely positions in descending order (the deterministic mask,
 * e.g. the initial mask at initialisation or the final mask after training). */
typedef struct {
    uint64_t seed;
    uint32_t step;
    uint32_t flags;
} maskpro_draw_params;

/* Forward ("Approach": N-way sampling without replacement).  Draws the N
 * positions of every block and applies the hard mask.  Outputs, each NULL to
 * skip:
 *   out        [rows, cols] of out_dt: w_j at the drawn positions, 0 elsewhere
 *              (bf16 out of fp32 w: round to nearest even).  Needs w.
 *   mask_bits  [ceil(B*M/8)] uint8, maskgs_hard_extract's format: the drawn
 *              positions of block b at bits [b*M, b*M+M) of an LSB-first
 *              stream; the unused bits of the last byte are zero.
 *   order      the draw order, for maskpro_bwd: 2:4 [B] uint8 with j_k at bits
 *              [2(k-1), 2k); 4:8 [B] uint16 with j_k at bits [3(k-1), 3k);
 *              unused high bits zero.
 *   pi         [B, M] fp32 logits (required).
 *   w          [rows, cols] of w_dt, frozen weights (required when out is).
 * E_NULL without pi, E_DTYPE for a bad w_dt/out_dt where out is given. */
int maskpro_fwd(const maskgs_tensor_desc *t, const maskpro_draw_params *p, const void *w,
                maskgs_dtype w_dt, const float *pi, void *out, maskgs_dtype out_dt,
                uint8_t *mask_bits, void *order, hipStream_t stream);

/* Policy gradient ("Approach": policy gradient on the loss residual against
 * the initial mask, with a moving-average baseline).  For the ordered draw of
 * each block, with Z_k = sum of exp(pi_l) over the positions l not drawn
 * before step k,
 *   dpi_l = A * sum_{k=1..N} ( 1{l = j_k} - 1{l not drawn before k} exp(pi_l)/Z_k ),
 * the gradient of A*log p(j_1..j_N); its expectation over draws is the
 * gradient of the expected loss when A = L(draw) - (any baseline that does
 * not depend on the draw).
 *   order      NULL (draw again from pi and p exactly as maskpro_fwd does:
 *              pi must be the logits of that forward), or maskpro_fwd's order.
 *   advantage  A, finite: the step's loss residual minus the baseline (see
 *              maskpro_baseline).
 *   dpi        [B, M] fp32 output; accumulate != 0 adds to its contents.
 *              Must not alias pi.
 * fp32 arithmetic; each round is formed against the largest logit still in
 * play, so its normaliser lies in [1, M] and no exponential overflows; terms
 * that underflow to 0 are below 2^-126 of that round's largest.  Non-finite
 * logits give non-finite gradients. */
int maskpro_bwd(const maskgs_tensor_desc *t, const maskpro_draw_params *p, const float *pi,
                const void *order, float advantage, float *dpi, int32_t accumulate,
                hipStream_t stream);

/* Initial logits ("Limitations": training starts from a chosen initial mask
 * and a magnitude C): pi_j = c at the kept positions of the initial mask M0,
 * 0 elsewhere, written to pi [B, M].  M0 is prior_bits (the mask_bits format)
 * or, when prior_bits is NULL, the magnitude top-N of w (as in
 * maskgs_prior_init: |w| compared on the bit pattern with the sign cleared,
 * ties keep the lower position).  c finite (E_RANGE otherwise). */
int maskpro_init(const maskgs_tensor_desc *t, const uint8_t *prior_bits, const void *w,
                 maskgs_dtype w_dt, float c, float *pi, hipStream_t stream);

/* Moving-average baseline of the loss residual ("Approach"), HOST scalars:
 *   *advantage = residual - *baseline, then
 *   *baseline  = mu * *baseline + (1 - mu) * residual,
 * so the advantage of a step never depends on its own draw (the estimator
 * stays unbiased).  residual = L(draw) - L(initial mask) of this step;
 * *baseline starts at 0.  mu in [0, 1], residual finite (E_RANGE otherwise);
 * E_NULL for a NULL pointer.  No device work. */
int maskpro_baseline(double residual, double mu, double *baseline, double *advantage);

#ifdef __cplusplus
}
#endif

#endif /* MASKPRO_H */
