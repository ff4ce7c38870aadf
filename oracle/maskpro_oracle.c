/*
 * maskpro_oracle.c -- plain CPU oracle of the linear-space N:M mask learner
 * MaskPro ("MaskPro: Linear-Space Probabilistic Learning for Strict
 * (N:M)-Sparsity on LLMs", read through its atlas.scime.ai summary page).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  The GPU library
 * never links, loads or calls it, and the two share no source, header, table
 * or constant generator.  It is built into the same shared object as
 * maskgs_oracle.c, whose Philox word, Gumbel variate, bf16 rounding and
 * magnitude top-N it reuses.
 *
 * What the summary page fixes ("Approach"): each block of M weights has one
 * categorical distribution over its M positions (M logits per block, so the
 * logits grow linearly with the weights); the N kept positions are drawn from
 * it without replacement; the logits learn by a policy gradient on the loss
 * residual against an initial mask, with a moving-average baseline.  Its
 * "Limitations" add that the logits start from an initial mask and a
 * magnitude C.  The readings taken where it is silent:
 *   - The draw is sequential: the first position from softmax(pi), each next
 *     one from softmax(pi) restricted to the positions not yet drawn.  It is
 *     realised with the Gumbel-top-k construction (the positions of the N
 *     largest pi_j + g_j in descending order are such an ordered draw;
 *     W. Kool, H. van Hoof, M. Welling, "Stochastic Beams and Where to Find
 *     Them", ICML 2019), g_j the Gumbel noise of maskgs_oracle.c with word
 *     index gb*M + j.  The key pi_j + g_j is one fp32 addition, so that the
 *     sample is fixed bit for bit; ties go to the lower position.
 *   - The policy's likelihood is that of the ordered draw:
 *       log p = sum_k [ pi_{j_k} - log sum_{l not in {j_1..j_{k-1}}} exp(pi_l) ].
 *   - The gradient estimate is A * d(log p)/d(pi), A = (L(m) - L(m0)) - b with
 *     b the moving average of the residuals of the earlier steps, updated
 *     after use: b <- mu*b + (1 - mu)*(L(m) - L(m0)), b = 0 at the start.
 *   - Initial logits: pi_j = C at the kept positions of the initial mask m0,
 *     0 elsewhere; m0 given as bits, or the magnitude top-N of |w|.
 * Everything after the sample is fp64 from the fp32 inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MP_NO_NOISE 1u /* keys = pi: the draw is the top-N of pi (test flag) */

uint32_t orc_philox_word(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n);
float orc_gumbel(uint32_t x);
uint16_t orc_bf16_from_double(double v);
int orc_magnitude_mask(int n, int m, int64_t rows, int64_t cols, const float *w, uint8_t *bits);

static int orc_mp_shape(int n, int m, int64_t rows, int64_t cols, int64_t *nblocks) {
    if (rows < 0 || cols < 0 || m < 1 || m > 8 || n < 1 || n > m || cols % m) return -1;
    *nblocks = rows * (cols / m);
    return 0;
}

/* Ordered draw of N of the M positions of global block gb ("Approach": N-way
 * sampling without replacement), by Gumbel-top-k: order[k] is the position of
 * the (k+1)-th largest key a_j = fp32(pi_j + g_j); a strict ">" scan, so ties
 * (and NaN keys) keep the lower position. */
static void orc_mp_draw(int n, int m, uint64_t seed, uint32_t step, uint32_t tensor_id,
                        uint64_t gb, uint32_t flags, const float *pib, int *order) {
    float a[8];
    int taken[8] = {0};
    for (int j = 0; j < m; ++j) {
        float g = 0.0f;
        if (!(flags & ORC_MP_NO_NOISE))
            g = orc_gumbel(orc_philox_word(seed, step, tensor_id, gb * (uint64_t)m + (uint64_t)j));
        a[j] = pib[j] + g;
    }
    for (int k = 0; k < n; ++k) {
        int best = -1;
        for (int j = 0; j < m; ++j)
            if (!taken[j] && (best < 0 || a[j] > a[best])) best = j;
        order[k] = best;
        taken[best] = 1;
    }
}

/* Forward: draw, then apply the hard mask to the frozen weights (out_j = w_j
 * at the N drawn positions, 0 elsewhere).  Outputs may be NULL:
 *   order_out [B*N] positions, draw order; bits: LSB-first stream, M bits per
 *   block; out_bf16 / out_f32 [B*M] masked weights. */
int orc_mp_fwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
               uint32_t tensor_id, uint64_t seed, uint32_t step, uint32_t flags,
               const float *w, const float *pi, uint8_t *order_out, uint8_t *bits,
               uint16_t *out_bf16, float *out_f32) {
    int64_t nb;
    if (orc_mp_shape(n, m, rows, cols, &nb)) return -1;
    if (nb == 0) return 0;
    /* pass 1, one block at a time (blocks are independent): the draw, its
     * order and the masked weights; the kept set of each block is kept for
     * pass 2 */
    uint8_t *keep_of = (uint8_t *)malloc((size_t)nb);
    if (!keep_of) return -3;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int order[8];
        orc_mp_draw(n, m, seed, step, tensor_id, block_offset + (uint64_t)b, flags, pi + b * m,
                    order);
        int keep[8] = {0};
        uint8_t kmask = 0;
        for (int k = 0; k < n; ++k) {
            keep[order[k]] = 1;
            kmask |= (uint8_t)(1u << order[k]);
            if (order_out) order_out[b * n + k] = (uint8_t)order[k];
        }
        keep_of[b] = kmask;
        for (int j = 0; j < m; ++j) {
            double u = keep[j] ? (double)w[b * m + j] : 0.0;
            if (out_bf16) out_bf16[b * m + j] = orc_bf16_from_double(u);
            if (out_f32) out_f32[b * m + j] = (float)u;
        }
    }
    /* pass 2, one byte of the LSB-first mask stream at a time (a byte holds
     * the bits of several blocks when m < 8) */
    if (bits) {
        const int64_t nbits = nb * m, nbytes = (nbits + 7) / 8;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < nbytes; ++i) {
            uint8_t v = 0;
            for (int64_t bit = 8 * i; bit < 8 * i + 8 && bit < nbits; ++bit)
                if (keep_of[bit / m] & (1u << (bit % m))) v |= (uint8_t)(1u << (bit - 8 * i));
            bits[i] = v;
        }
    }
    free(keep_of);
    return 0;
}

/* log-likelihood of the ordered draw of each block (reading above):
 * sum_k [ pi_{j_k} - log sum_{l not drawn before step k} exp(pi_l) ]. */
int orc_mp_logp(int n, int m, int64_t nblocks, const float *pi, const uint8_t *order,
                double *logp) {
    if (nblocks < 0 || m < 1 || m > 8 || n < 1 || n > m) return -1;
    for (int64_t b = 0; b < nblocks; ++b) {
        const float *p = pi + b * m;
        double mx = -INFINITY;
        for (int j = 0; j < m; ++j) mx = fmax(mx, (double)p[j]);
        int taken[8] = {0};
        double s = 0.0;
        for (int k = 0; k < n; ++k) {
            double z = 0.0;
            for (int l = 0; l < m; ++l)
                if (!taken[l]) z += exp((double)p[l] - mx);
            int jk = order[b * n + k];
            s += ((double)p[jk] - mx) - log(z);
            taken[jk] = 1;
        }
        logp[b] = s;
    }
    return 0;
}

/* Policy gradient ("Approach"): dpi = A * d(log p)/d(pi) for the ordered draw
 * of each block, where, with Z_k = sum of exp(pi_l) over the positions not
 * drawn before step k,
 *   d(log p)/d(pi_l) = sum_k [ 1{l = j_k} - 1{l not drawn before k} exp(pi_l)/Z_k ].
 * The draw is order_in ([B*N] positions) or, when order_in is NULL, drawn
 * again from (seed, step, tensor_id, block_offset, flags) as orc_mp_fwd does.
 * dpi_prev (nullable): the result is dpi_prev + A * gradient (accumulation). */
int orc_mp_grad(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
                uint32_t tensor_id, uint64_t seed, uint32_t step, uint32_t flags,
                const float *pi, const uint8_t *order_in, double advantage,
                const float *dpi_prev, double *dpi) {
    int64_t nb;
    if (orc_mp_shape(n, m, rows, cols, &nb)) return -1;
    /* blocks are independent: each writes only its own M gradients */
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        const float *p = pi + b * m;
        int order[8];
        if (order_in) {
            for (int k = 0; k < n; ++k) order[k] = order_in[b * n + k];
        } else {
            orc_mp_draw(n, m, seed, step, tensor_id, block_offset + (uint64_t)b, flags, p, order);
        }
        double mx = -INFINITY;
        for (int j = 0; j < m; ++j) mx = fmax(mx, (double)p[j]);
        double e[8], gr[8] = {0};
        for (int j = 0; j < m; ++j) e[j] = exp((double)p[j] - mx);
        int taken[8] = {0};
        for (int k = 0; k < n; ++k) {
            double z = 0.0;
            for (int l = 0; l < m; ++l)
                if (!taken[l]) z += e[l];
            for (int l = 0; l < m; ++l)
                if (!taken[l]) gr[l] -= e[l] / z;
            gr[order[k]] += 1.0;
            taken[order[k]] = 1;
        }
        for (int j = 0; j < m; ++j) {
            double v = advantage * gr[j];
            if (dpi_prev) v += (double)dpi_prev[b * m + j];
            dpi[b * m + j] = v;
        }
    }
    return 0;
}

/* Initial logits ("Limitations": a chosen initial mask and magnitude C):
 * pi_j = C at the kept positions of m0, 0 elsewhere.  m0 is the LSB-first bit
 * stream prior_bits, or the magnitude top-N mask of w when prior_bits is NULL. */
int orc_mp_init(int n, int m, int64_t rows, int64_t cols, const uint8_t *prior_bits,
                const float *w, float c, float *pi) {
    int64_t nb;
    if (orc_mp_shape(n, m, rows, cols, &nb)) return -1;
    uint8_t *own = NULL;
    const uint8_t *bits = prior_bits;
    if (!bits) {
        own = (uint8_t *)malloc((size_t)((nb * m + 7) / 8) + 1);
        if (!own) return -3;
        orc_magnitude_mask(n, m, rows, cols, w, own);
        bits = own;
    }
    for (int64_t i = 0; i < nb * m; ++i) pi[i] = (bits[i >> 3] & (1u << (i & 7))) ? c : 0.0f;
    free(own);
    return 0;
}

/* Moving-average baseline ("Approach"): for each step t in turn,
 * adv[t] = residual[t] - b, then b <- mu*b + (1 - mu)*residual[t].
 * b_inout holds b before the first step and after the last. */
int orc_mp_baseline(int64_t steps, const double *residual, double mu, double *b_inout,
                    double *adv) {
    if (steps < 0 || !(mu >= 0.0 && mu <= 1.0)) return -1;
    double b = *b_inout;
    for (int64_t t = 0; t < steps; ++t) {
        adv[t] = residual[t] - b;
        b = mu * b + (1.0 - mu) * residual[t];
    }
    *b_inout = b;
    return 0;
}
