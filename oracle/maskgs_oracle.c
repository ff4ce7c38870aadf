/*
 * maskgs_oracle.c -- plain CPU oracle of the differentiable N:M mask path of
 * MaskLLM ("MaskLLM: Learnable Semi-Structured Sparsity for Large Language
 * Models", arXiv 2409.17481, read through its paper-graph-ui summary page).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  The GPU library
 * never links, loads or calls it, and the two share no source, header, table
 * or constant generator.
 *
 * Precision.  Every step is carried out in fp64 in the order the summary page
 * gives, except the two steps that *define the sample*:
 *   - the Gumbel noise g (an fp32 value produced from a Philox word by the
 *     noise contract below), and
 *   - the perturbed, tempered logit a_i = fp32(fp32(kappa*z_i + g_i) * fp32(1/tau))
 *     (one fused multiply-add, then one multiply, both in fp32).
 * The logits are stored in fp32, and at tau = 0.05 the softmax amplifies a
 * one-ulp change of kappa*z+g twentyfold, far beyond any useful tolerance, so
 * the sample itself is fixed bit for bit in fp32 and everything downstream of
 * it (softmax, soft mask, masked weight, regulariser, gradient) is computed
 * here in fp64.  The flag ORC_EXACT_LOGITS replaces the fp32 logit step by
 * a_i = (kappa*z_i + g_i)/tau in fp64; it exists for finite-difference checks.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fused
 * multiply-adds other than the explicit fmaf() calls of the noise contract).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_NO_NOISE 1u        /* g = 0 for every candidate (test flag)          */
#define ORC_EXACT_LOGITS 2u    /* a_i in fp64 instead of the fp32 logit step     */
#define ORC_HARD_SAMPLE 4u     /* hard Gumbel-max sample, straight-through grad  */
#define ORC_MAX_K 70           /* C(8,4): the largest candidate set for M <= 8   */

/* ------------------------------------------------------------------------- */
/* Threads (used only by the CPU-baseline leg of the benchmark).             */
/* ------------------------------------------------------------------------- */
void orc_set_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Candidate set S.                                                          */
/* MaskLLM summary, section 3.2 "Big-Picture Architecture" (candidate mask   */
/* set S_{2:4}) and section 3.4, Eq. 7 (S has one candidate per row).        */
/* 2:4: the six patterns in the order the page lists them, first position of */
/* the pattern = bit 0.  Other N:M (M <= 8): every N-subset of the M         */
/* positions, in lexicographic order of the sorted kept positions.           */
/* ------------------------------------------------------------------------- */
static void orc_comb(int m, int n, int start, int left, uint8_t cur,
                     uint8_t *out, int *k, int cap) {
    if (left == 0) {
        if (*k < cap) out[*k] = cur;
        (*k)++;
        return;
    }
    for (int p = start; p <= m - left; ++p)
        orc_comb(m, n, p + 1, left - 1, (uint8_t)(cur | (1u << p)), out, k, cap);
}

/* Returns K = C(M,N) and writes min(K, cap) masks; -1 for an invalid pair. */
int orc_candidates(int n, int m, uint8_t *out, int cap) {
    if (m < 1 || m > 8 || n < 1 || n > m) return -1;
    if (n == 2 && m == 4) {
        /* [1,1,0,0] [1,0,1,0] [1,0,0,1] [0,1,0,1] [0,1,1,0] [0,0,1,1] */
        static const int rows[6][4] = {{1, 1, 0, 0}, {1, 0, 1, 0}, {1, 0, 0, 1},
                                       {0, 1, 0, 1}, {0, 1, 1, 0}, {0, 0, 1, 1}};
        for (int i = 0; i < 6 && i < cap; ++i) {
            uint8_t b = 0;
            for (int j = 0; j < 4; ++j)
                if (rows[i][j]) b |= (uint8_t)(1u << j);
            out[i] = b;
        }
        return 6;
    }
    int k = 0;
    orc_comb(m, n, 0, n, 0, out, &k, cap);
    return k;
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 counter-based generator, from J. K. Salmon, M. A. Moraes,   */
/* R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"     */
/* (SC'11): per round two 32x32->64 products of counter words 0 and 2 with   */
/* the multipliers 0xD2511F53 and 0xCD9E8D57, the high halves xor-ed with    */
/* the other two counter words and the round key, then a word permutation;   */
/* the two key words are bumped by the Weyl constants 0x9E3779B9 and         */
/* 0xBB67AE85 between rounds.                                                */
/* The MaskLLM pages only ask for independent U(0,1) noise per block and     */
/* candidate (section 3.4, Gumbel noise of Eq. 5 and Algorithm 1 step 1).    */
/* ------------------------------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Word layout of the noise stream: word index n = global_block*K + i (i =
 * candidate).  Call q = n / 4 uses counter (lo32(q), hi32(q), step,
 * tensor_id) and key (lo32(seed), hi32(seed)); the word is output n % 4. */
uint32_t orc_philox_word(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n) {
    uint64_t q = n >> 2;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), step, tensor_id};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[n & 3u];
}

void orc_philox_words(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                      int64_t count, uint32_t *words) {
    for (int64_t t = 0; t < count; ++t)
        words[t] = orc_philox_word(seed, step, tensor_id, n0 + (uint64_t)t);
}

/* ------------------------------------------------------------------------- */
/* Noise contract: uniform and Gumbel variates.                              */
/* Uniform: eps = (2*(x >> 9) + 1) * 2^-24, exact in fp32, strictly inside   */
/* (0, 1) as the Gumbel inverse CDF needs.                                    */
/* Gumbel (MaskLLM summary, section 3.4, Eq. 5): g = -ln(-ln eps), natural   */
/* logarithms, for each of the 2^23 values eps can take.  The pages fix no   */
/* precision; the value each side uses is defined in fp32 as the cubic        */
/* Taylor polynomial of -ln(-ln eps) about the centre of the segment that    */
/* holds eps, evaluated with three fused multiply-adds:                       */
/*   - k2 = 2*(x >> 9) + 1 (the odd integer eps * 2^24); side 0 when          */
/*     eps < 1/2 (v = k2), side 1 when eps > 1/2 (v = 2^24 - k2, i.e. the     */
/*     same integer for 1 - eps);                                             */
/*   - v lies in [2^b, 2^(b+1)); its binade splits into 32 segments of width  */
/*     2^(b-5), segment q = the five bits after the leading one of v;         */
/*   - d = v / 2^b - 1 - (q + 1/2)/32, the offset from the segment centre,     */
/*     exact in fp32, |d| <= 1/64;                                            */
/*   - g = ((c3*d + c2)*d + c1)*d + c0 with the Taylor coefficients c_n of    */
/*     -ln(-ln eps) in d about the centre, each evaluated in fp64 and rounded */
/*     once to fp32 (orc_gumbel_coef).                                        */
/* Over all 2^23 uniforms this stays within 1.25 ulp of max(|g|, 1) of the   */
/* exact value (pinned exhaustively by the tests).                            */
/* ------------------------------------------------------------------------- */
float orc_uniform(uint32_t x) {
    uint32_t k = x >> 9;
    return (float)(2u * k + 1u) * 0x1p-24f;
}

#define ORC_GS_BINADES 24
#define ORC_GS_SEGS 32

static float orc_gs[2][ORC_GS_BINADES][ORC_GS_SEGS][4];

/* Taylor coefficients c0..c3 of segment (side, b, q), as the step in d moves
 * eps by 2^(b-24) (side 0) or 1 - eps by 2^(b-24) (side 1).  With delta the
 * centre's eps (side 0) or 1 - eps (side 1):
 *   side 0: L = -ln(delta), g = -ln L, dg/d(delta) = 1/(delta L), and the
 *           n-th derivative in d is (2^(b-24)/delta)^n times
 *           1/L, (1/L^2 - 1/L), (2/L^3 - 3/L^2 + 2/L)          for n = 1, 2, 3;
 *   side 1: M = -ln(1 - delta), g = -ln M, and in d the derivatives are
 *           (2^(b-24)/(1 - delta))^n times
 *           -1/M, (1/M^2 - 1/M), (-2/M^3 + 3/M^2 - 2/M);
 * c_n = derivative / n!. */
static void orc_gumbel_coef_fill(int side, int b, int q, double co[4]) {
    double vc = ldexp(1.0 + (q + 0.5) / 32.0, b);
    double delta = vc * 0x1p-24;
    if (side == 0) {
        double L = -log(delta);
        double rho = ldexp(1.0, b) / vc;
        double iL = 1.0 / L;
        co[0] = -log(L);
        co[1] = rho * iL;
        co[2] = rho * rho * (iL * iL - iL) / 2.0;
        co[3] = rho * rho * rho * (2.0 * iL * iL * iL - 3.0 * iL * iL + 2.0 * iL) / 6.0;
    } else {
        double M = -log1p(-delta);
        double sig = ldexp(1.0, b - 24) / (1.0 - delta);
        double iM = 1.0 / M;
        co[0] = -log(M);
        co[1] = -sig * iM;
        co[2] = sig * sig * (iM * iM - iM) / 2.0;
        co[3] = sig * sig * sig * (-2.0 * iM * iM * iM + 3.0 * iM * iM - 2.0 * iM) / 6.0;
    }
}

__attribute__((constructor)) static void orc_gumbel_coef_init(void) {
    for (int side = 0; side < 2; ++side)
        for (int b = 0; b < ORC_GS_BINADES; ++b)
            for (int q = 0; q < ORC_GS_SEGS; ++q) {
                double co[4];
                orc_gumbel_coef_fill(side, b, q, co);
                for (int n = 0; n < 4; ++n) orc_gs[side][b][q][n] = (float)co[n];
            }
}

/* The fp32 coefficient table, [side][binade][segment][c0..c3] (1536 x 4). */
void orc_gumbel_coef(float *out) { memcpy(out, orc_gs, sizeof(orc_gs)); }

float orc_gumbel(uint32_t x) {
    uint32_t k2 = 2u * (x >> 9) + 1u;
    int side = k2 > (1u << 23);
    uint32_t v = side ? (1u << 24) - k2 : k2;
    int b = 0;
    while ((v >> (b + 1)) != 0) ++b;                   /* v in [2^b, 2^(b+1)) */
    uint32_t frac = v - (1u << b);                     /* v/2^b = 1 + frac/2^b */
    uint32_t q, r;                                     /* frac/2^b = q/32 + r/2^b */
    if (b >= 5) {
        q = frac >> (b - 5);
        r = frac - (q << (b - 5));
    } else {
        q = frac << (5 - b);
        r = 0;
    }
    float d = (float)r * ldexpf(1.0f, -b) - 0x1p-6f;   /* exact */
    const float *c = orc_gs[side][b][q];
    return fmaf(fmaf(fmaf(c[3], d, c[2]), d, c[1]), d, c[0]);
}

/* g for every one of the 2^23 distinct uniforms, indexed by x >> 9. */
void orc_gumbel_all(float *out) {
#pragma omp parallel for schedule(static)
    for (int32_t k = 0; k < (1 << 23); ++k) out[k] = orc_gumbel((uint32_t)k << 9);
}

/* ------------------------------------------------------------------------- */
/* Shared per-call description.                                              */
/* ------------------------------------------------------------------------- */
typedef struct {
    int n, m, k;
    int64_t rows, cols, nblocks;
    uint64_t block_offset;
    uint32_t tensor_id, step, flags;
    uint64_t seed;
    float kappa, tau;
    uint8_t cand[ORC_MAX_K];
} orc_ctx;

static int orc_setup(orc_ctx *c, int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
                     uint32_t tensor_id, uint64_t seed, uint32_t step, float kappa, float tau,
                     uint32_t flags) {
    if (rows < 0 || cols < 0 || m < 1 || cols % m != 0) return -1;
    c->k = orc_candidates(n, m, c->cand, ORC_MAX_K);
    if (c->k < 1 || c->k > ORC_MAX_K) return -1;
    c->n = n; c->m = m; c->rows = rows; c->cols = cols;
    c->nblocks = rows * (cols / m);
    c->block_offset = block_offset; c->tensor_id = tensor_id;
    c->seed = seed; c->step = step; c->kappa = kappa; c->tau = tau; c->flags = flags;
    return 0;
}

/* Soft index of one block (MaskLLM summary, section 3.4, Eq. 6 and
 * Algorithm 1 steps 1-2): y_i = exp(a_i) / sum_j exp(a_j), a_i = (pi_i*kappa +
 * g_i)/tau.  Local block b has global index block_offset + b. */
/* Perturbed, tempered logits of block b (Eq. 6 argument, Algorithm 1):
 * a_i = fp32(fp32(kappa*z_i + g_i) * fp32(1/tau)), or (kappa*z_i + g_i)/tau in
 * fp64 under ORC_EXACT_LOGITS. */
static void orc_logits(const orc_ctx *c, int64_t b, const float *zb, double *a) {
    uint64_t gb = c->block_offset + (uint64_t)b;
    float tau_inv = 1.0f / c->tau;
    for (int i = 0; i < c->k; ++i) {
        float g = 0.0f;
        if (!(c->flags & ORC_NO_NOISE))
            g = orc_gumbel(orc_philox_word(c->seed, c->step, c->tensor_id,
                                           gb * (uint64_t)c->k + (uint64_t)i));
        if (c->flags & ORC_EXACT_LOGITS)
            a[i] = ((double)c->kappa * (double)zb[i] + (double)g) / (double)c->tau;
        else
            a[i] = (double)(fmaf(c->kappa, zb[i], g) * tau_inv);
    }
}

/* Hard Gumbel-max sample of block b (section 3.4, Eq. 5: the argmax of the
 * perturbed logits is a draw from softmax(kappa*z)): the first index of the
 * largest a_i (strict ">" scan), written as the 0/1 mask S_k. */
static void orc_hard_sample(const orc_ctx *c, int64_t b, const float *zb, double *mk) {
    double a[ORC_MAX_K];
    orc_logits(c, b, zb, a);
    int best = 0;
    for (int i = 1; i < c->k; ++i)
        if (a[i] > a[best]) best = i;
    for (int j = 0; j < c->m; ++j) mk[j] = (c->cand[best] >> j) & 1u ? 1.0 : 0.0;
}

static void orc_soft_index(const orc_ctx *c, int64_t b, const float *zb, double *y) {
    double a[ORC_MAX_K] = {0.0};
    orc_logits(c, b, zb, a);
    double amax = a[0];
    for (int i = 1; i < c->k; ++i)
        if (a[i] > amax) amax = a[i];
    double s = 0.0;
    for (int i = 0; i < c->k; ++i) {
        y[i] = exp(a[i] - amax);
        s += y[i];
    }
    for (int i = 0; i < c->k; ++i) y[i] = y[i] / s;
}

/* Soft mask (section 3.4, Eq. 7): m_j = sum_i y_i * S_ij. */
static void orc_soft_mask(const orc_ctx *c, const double *y, double *mk) {
    for (int j = 0; j < c->m; ++j) {
        double s = 0.0;
        for (int i = 0; i < c->k; ++i)
            if (c->cand[i] & (1u << j)) s += y[i];
        mk[j] = s;
    }
}

/* bf16 round-to-nearest-even of an fp64 value (one rounding). */
uint16_t orc_bf16_from_double(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    if (v == 0.0) return (uint16_t)(signbit(v) ? 0x8000u : 0x0000u);
    int e;
    (void)frexp(v, &e);             /* |v| in [2^(e-1), 2^e)                 */
    if (e < -125) e = -125;         /* below 2^-126: subnormal spacing 2^-133 */
    double q = ldexp(1.0, e - 8);   /* spacing of 8-bit significands          */
    double r = nearbyint(v / q) * q;
    float rf;
    if (fabs(r) >= 0x1p128) rf = (float)(r > 0 ? INFINITY : -INFINITY);
    else rf = (float)r;             /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &rf, 4);
    return (uint16_t)(bits >> 16);
}

/* ------------------------------------------------------------------------- */
/* Forward: soft index, soft mask, masked weight and regulariser value.      */
/* Masked weight W (.) M~ (section 3.2, frozen backbone; Algorithm 1 step 3  */
/* forward).  Regulariser value R = sum_i ||W_i (.) M~_i||_2^2 of Eq. 8; the */
/* loss term is -lambda*R.                                                   */
/* w, z: fp32 (bf16 weights widened exactly).  Outputs may be NULL.          */
/* Returns 0, or -1 on an invalid shape.                                     */
/* ------------------------------------------------------------------------- */
int orc_fwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset, uint32_t tensor_id,
            uint64_t seed, uint32_t step, float kappa, float tau, uint32_t flags,
            const float *w, const float *z, double *y_out, double *m_out,
            uint16_t *out_bf16, float *out_f32, double *reg_out) {
    orc_ctx c;
    if (orc_setup(&c, n, m, rows, cols, block_offset, tensor_id, seed, step, kappa, tau, flags))
        return -1;
    double reg = 0.0;
#pragma omp parallel for schedule(static) reduction(+ : reg)
    for (int64_t b = 0; b < c.nblocks; ++b) {
        double y[ORC_MAX_K], mk[8];
        orc_soft_index(&c, b, z + b * c.k, y);
        orc_soft_mask(&c, y, mk);
        /* hard sample: the forward applies S_k (the soft index is still kept) */
        if (c.flags & ORC_HARD_SAMPLE) orc_hard_sample(&c, b, z + b * c.k, mk);
        for (int j = 0; j < c.m; ++j) {
            double u = (double)w[b * c.m + j] * mk[j];
            if (out_bf16) out_bf16[b * c.m + j] = orc_bf16_from_double(u);
            if (out_f32) out_f32[b * c.m + j] = (float)u;
            reg += u * u;
        }
        if (y_out)
            for (int i = 0; i < c.k; ++i) y_out[b * c.k + i] = y[i];
        if (m_out)
            for (int j = 0; j < c.m; ++j) m_out[b * c.m + j] = mk[j];
    }
    if (reg_out) *reg_out = reg;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward to the logits (section 3.2 information flow, section 3.4 Eq. 8,  */
/* Algorithm 1 backward step): the gradient of                               */
/*   L = L_LM(W (.) M~) - lambda * sum ||W (.) M~||^2                        */
/* with respect to pi, W frozen.  With G = dL_LM/d(W (.) M~):                */
/*   dL/dm_j  = G_j w_j - 2 lambda w_j^2 m_j                                 */
/*   dL/dy_i  = sum_j S_ij dL/dm_j            (Eq. 7 is linear in y)         */
/*   dL/dpi_i = (kappa/tau) y_i (dL/dy_i - sum_k y_k dL/dy_k)  (softmax)     */
/* dz_prev (nullable): the result is dz_prev + gradient (accumulation).      */
/* ------------------------------------------------------------------------- */
int orc_bwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset, uint32_t tensor_id,
            uint64_t seed, uint32_t step, float kappa, float tau, uint32_t flags,
            const float *w, const float *z, const float *gup, double lambda,
            const float *dz_prev, double *dz_out) {
    orc_ctx c;
    if (orc_setup(&c, n, m, rows, cols, block_offset, tensor_id, seed, step, kappa, tau, flags))
        return -1;
    double scale = (double)kappa / (double)tau;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < c.nblocks; ++b) {
        double y[ORC_MAX_K], mk[8], dm[8], dy[ORC_MAX_K];
        orc_soft_index(&c, b, z + b * c.k, y);
        orc_soft_mask(&c, y, mk);
        /* straight-through: the regulariser term is that of the mask the
         * forward applied (S_k); the Jacobian below is the soft index's */
        if (c.flags & ORC_HARD_SAMPLE) orc_hard_sample(&c, b, z + b * c.k, mk);
        for (int j = 0; j < c.m; ++j) {
            double wj = (double)w[b * c.m + j];
            dm[j] = (double)gup[b * c.m + j] * wj - 2.0 * lambda * wj * wj * mk[j];
        }
        double s = 0.0;
        for (int i = 0; i < c.k; ++i) {
            dy[i] = 0.0;
            for (int j = 0; j < c.m; ++j)
                if (c.cand[i] & (1u << j)) dy[i] += dm[j];
            s += y[i] * dy[i];
        }
        for (int i = 0; i < c.k; ++i) {
            double d = scale * y[i] * (dy[i] - s);
            if (dz_prev) d += (double)dz_prev[b * c.k + i];
            dz_out[b * c.k + i] = d;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Hard mask (section 3.2 inference flow; Algorithm 1 step 3): k = argmax pi */
/* (first index among equal maxima, fp32 compare), M* = S_k.                 */
/* bits:    S_k of block b at bits [b*M, b*M+M) of an LSB-first stream,      */
/*          zero padded (0.65 bits/parameter storage, section 1).            */
/* values:  for 2:4, the two kept weights of block b in ascending position   */
/*          (raw weight bytes, w_bytes per element).                         */
/* val_idx: for 2:4, nibble p0 | p1 << 2 of the kept positions; block 2i in  */
/*          the low nibble of byte i, block 2i+1 in the high nibble.         */
/* Any output may be NULL.  Returns -1 on an invalid shape, -2 if values or  */
/* val_idx are requested for a pattern other than 2:4.                        */
/* ------------------------------------------------------------------------- */
int orc_hard_extract(int n, int m, int64_t rows, int64_t cols, const float *z,
                     const void *w_raw, int w_bytes, uint8_t *idx, uint8_t *bits,
                     void *values, uint8_t *val_idx) {
    orc_ctx c;
    if (orc_setup(&c, n, m, rows, cols, 0, 0, 0, 0, 1.0f, 1.0f, 0)) return -1;
    if ((values || val_idx) && !(n == 2 && m == 4)) return -2;
    if (c.nblocks == 0) return 0;
    /* pass 1, one block at a time (blocks are independent): the argmax, and
     * the kept values of 2:4 blocks */
    uint8_t *best_of = idx ? idx : (uint8_t *)malloc((size_t)c.nblocks);
    if (!best_of) return -3;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < c.nblocks; ++b) {
        const float *zb = z + b * c.k;
        int best = 0;
        for (int i = 1; i < c.k; ++i)
            if (zb[i] > zb[best]) best = i;
        best_of[b] = (uint8_t)best;
        if (values) {
            uint8_t mask = c.cand[best];
            int pos[2], t = 0;
            for (int j = 0; j < 4; ++j)
                if (mask & (1u << j)) pos[t++] = j;
            for (int u = 0; u < 2; ++u)
                memcpy((char *)values + (b * 2 + u) * w_bytes,
                       (const char *)w_raw + (b * 4 + pos[u]) * w_bytes, (size_t)w_bytes);
        }
    }
    /* pass 2, one output byte at a time (a byte holds the bits or nibbles of
     * several blocks): the packed masks S_k and the 2:4 index nibbles */
    if (bits) {
        const int64_t nbytes = (c.nblocks * c.m + 7) / 8;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < nbytes; ++i) {
            uint8_t v = 0;
            for (int64_t bit = 8 * i; bit < 8 * i + 8 && bit < c.nblocks * c.m; ++bit) {
                const int64_t b = bit / c.m;
                if (c.cand[best_of[b]] & (1u << (bit % c.m))) v |= (uint8_t)(1u << (bit - 8 * i));
            }
            bits[i] = v;
        }
    }
    if (val_idx) {
        const int64_t nbytes = (c.nblocks + 1) / 2;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < nbytes; ++i) {
            uint8_t v = 0;
            for (int64_t b = 2 * i; b < 2 * i + 2 && b < c.nblocks; ++b) {
                uint8_t mask = c.cand[best_of[b]];
                int pos[2], t = 0;
                for (int j = 0; j < 4; ++j)
                    if (mask & (1u << j)) pos[t++] = j;
                uint8_t nib = (uint8_t)(pos[0] | (pos[1] << 2));
                v |= (uint8_t)((b & 1) ? (nib << 4) : nib);
            }
            val_idx[i] = v;
        }
    }
    if (!idx) free(best_of);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Magnitude prior (section 2, magnitude pruning as a one-shot prior;        */
/* section 3.4 "Prior types"): in each block keep the N weights of largest   */
/* |w|; |w| is compared on the bit pattern with the sign cleared (so -0 ==   */
/* +0) and ties keep the lower position.  Writes the LSB-first bit stream.   */
/* ------------------------------------------------------------------------- */
int orc_magnitude_mask(int n, int m, int64_t rows, int64_t cols, const float *w, uint8_t *bits) {
    if (rows < 0 || cols < 0 || m < 1 || m > 8 || n < 1 || n > m || cols % m) return -1;
    int64_t nblocks = rows * (cols / m);
    memset(bits, 0, (size_t)((nblocks * m + 7) / 8));
    for (int64_t b = 0; b < nblocks; ++b) {
        uint32_t mag[8];
        int kept[8] = {0};
        for (int j = 0; j < m; ++j) {
            uint32_t u;
            memcpy(&u, &w[b * m + j], 4);
            mag[j] = u & 0x7FFFFFFFu;
        }
        for (int t = 0; t < n; ++t) {
            int best = -1;
            for (int j = 0; j < m; ++j)
                if (!kept[j] && (best < 0 || mag[j] > mag[best])) best = j;
            kept[best] = 1;
        }
        for (int j = 0; j < m; ++j)
            if (kept[j]) {
                int64_t bit = b * m + j;
                bits[bit >> 3] |= (uint8_t)(1u << (bit & 7));
            }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Mask prior (section 3.4 "Mask Prior and Transfer Learning", Eqs. 9-10).   */
/* Eq. 9:  sim_i = <M0, S_i> - mean_k <M0, S_k>  (mean over all K candidates)*/
/* Eq. 10 (mode 0): pi_i <- pi_i + alpha * sigma(pi) * sim_i, sigma the      */
/*          population standard deviation of the block's K logits as given. */
/* mode 1:  pi_k0 <- pi_k0 + alpha at the candidate k0 equal to M0; a block  */
/*          whose prior matches no candidate is left unchanged.              */
/* The prior M0 is the bit stream prior_bits, or the magnitude top-N mask of */
/* w when prior_bits is NULL.  z is updated in place, one rounding to fp32.  */
/* ------------------------------------------------------------------------- */
int orc_prior_init(int n, int m, int64_t rows, int64_t cols, float *z, const uint8_t *prior_bits,
                   const float *w, float alpha, int mode) {
    orc_ctx c;
    if (orc_setup(&c, n, m, rows, cols, 0, 0, 0, 0, 1.0f, 1.0f, 0)) return -1;
    if (mode != 0 && mode != 1) return -1;
    uint8_t *bits = (uint8_t *)prior_bits;
    uint8_t *own = NULL;
    if (!bits) {
        own = (uint8_t *)malloc((size_t)((c.nblocks * c.m + 7) / 8) + 1);
        if (!own) return -3;
        orc_magnitude_mask(n, m, rows, cols, w, own);
        bits = own;
    }
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < c.nblocks; ++b) {
        float *zb = z + b * c.k;
        uint32_t m0 = 0;
        for (int j = 0; j < c.m; ++j) {
            int64_t bit = b * c.m + j;
            if (bits[bit >> 3] & (1u << (bit & 7))) m0 |= 1u << j;
        }
        double dot[ORC_MAX_K], mean = 0.0;
        for (int i = 0; i < c.k; ++i) {
            int d = 0;
            for (int j = 0; j < c.m; ++j)
                if ((m0 & c.cand[i]) & (1u << j)) d++;
            dot[i] = (double)d;
            mean += dot[i];
        }
        mean /= (double)c.k;
        if (mode == 0) {
            double mu = 0.0, var = 0.0;
            for (int i = 0; i < c.k; ++i) mu += (double)zb[i];
            mu /= (double)c.k;
            for (int i = 0; i < c.k; ++i) var += ((double)zb[i] - mu) * ((double)zb[i] - mu);
            double sigma = sqrt(var / (double)c.k);
            double zn[ORC_MAX_K];
            for (int i = 0; i < c.k; ++i)
                zn[i] = (double)zb[i] + (double)alpha * sigma * (dot[i] - mean);
            for (int i = 0; i < c.k; ++i) zb[i] = (float)zn[i];
        } else {
            for (int i = 0; i < c.k; ++i)
                if (c.cand[i] == m0) {
                    zb[i] = (float)((double)zb[i] + (double)alpha);
                    break;
                }
        }
    }
    free(own);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* AdamW update of the logits (MaskLLM summary, section 3.4, Algorithm 1     */
/* "update logits", and the training details: AdamW with lr 5e-4 for LLaMA-2 */
/* and Nemotron, weight decay 0.1).  The pages fix neither the moment        */
/* coefficients, nor epsilon, nor how the decay enters; the reading here is  */
/* Adam (Kingma & Ba, ICLR 2015: moments, bias correction) with decoupled    */
/* weight decay (Loshchilov & Hutter, ICLR 2019) scaled by the learning rate:*/
/*   m  = b1 m + (1 - b1) g            v  = b2 v + (1 - b2) g^2              */
/*   mh = m / (1 - b1^t)               vh = v / (1 - b2^t)                   */
/*   z  = z - lr (mh / (sqrt(vh) + eps) + wd z)    (z on the right: before   */
/*                                                  this step)               */
/* t >= 1 is the number of updates including this one.  Every operation in   */
/* fp64 from the fp32 inputs; z, m and v are rounded to fp32 once.  g is the */
/* logit gradient as stored (fp32).                                          */
/* ------------------------------------------------------------------------- */
int orc_adamw(int64_t count, float *z, const float *g, float *m, float *v, double lr,
              double b1, double b2, double eps, double wd, uint32_t t) {
    if (count < 0 || t < 1) return -1;
    double bc1 = 1.0 - pow(b1, (double)t);
    double bc2 = 1.0 - pow(b2, (double)t);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double gi = (double)g[i];
        double mi = b1 * (double)m[i] + (1.0 - b1) * gi;
        double vi = b2 * (double)v[i] + (1.0 - b2) * gi * gi;
        double mh = mi / bc1;
        double vh = vi / bc2;
        double zi = (double)z[i];
        double zn = zi - lr * (mh / (sqrt(vh) + eps) + wd * zi);
        z[i] = (float)zn;
        m[i] = (float)mi;
        v[i] = (float)vi;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The perturbed, tempered logits a of every block ([B, K], the fp32 values  */
/* of the noise contract); their first argmax is the Gumbel-max sample of    */
/* the block's mask (section 3.4, Eq. 5).                                    */
/* ------------------------------------------------------------------------- */
int orc_sample_logits(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
                      uint32_t tensor_id, uint64_t seed, uint32_t step, float kappa, float tau,
                      uint32_t flags, const float *z, float *a_out) {
    orc_ctx c;
    if (orc_setup(&c, n, m, rows, cols, block_offset, tensor_id, seed, step, kappa, tau, flags))
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < c.nblocks; ++b) {
        double a[ORC_MAX_K];
        orc_logits(&c, b, z + b * c.k, a);
        for (int i = 0; i < c.k; ++i) a_out[b * c.k + i] = (float)a[i];
    }
    return 0;
}
