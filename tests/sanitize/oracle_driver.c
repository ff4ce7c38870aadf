/*
 * Host sanitizer driver for the CPU oracle (test infrastructure): every
 * oracle entry point on small shapes with ragged tails, odd block offsets,
 * ties, both N:M patterns, both weight widths and every optional output,
 * built with -fsanitize=address,undefined by tests/test_sanitize.py.  Exits 0
 * when every call returns 0 and the sanitizers report nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_set_threads(int t);
int orc_candidates(int n, int m, uint8_t *out, int cap);
void orc_philox_words(uint64_t seed, uint32_t step, uint32_t tensor_id, uint64_t n0,
                      int64_t count, uint32_t *words);
float orc_gumbel(uint32_t x);
int orc_fwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset, uint32_t tensor_id,
            uint64_t seed, uint32_t step, float kappa, float tau, uint32_t flags,
            const float *w, const float *z, double *y_out, double *m_out,
            uint16_t *out_bf16, float *out_f32, double *reg_out);
int orc_bwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset, uint32_t tensor_id,
            uint64_t seed, uint32_t step, float kappa, float tau, uint32_t flags,
            const float *w, const float *z, const float *gup, double lambda,
            const float *dz_prev, double *dz_out);
int orc_hard_extract(int n, int m, int64_t rows, int64_t cols, const float *z,
                     const void *w_raw, int w_bytes, uint8_t *idx, uint8_t *bits,
                     void *values, uint8_t *val_idx);
int orc_magnitude_mask(int n, int m, int64_t rows, int64_t cols, const float *w, uint8_t *bits);
int orc_prior_init(int n, int m, int64_t rows, int64_t cols, float *z, const uint8_t *prior_bits,
                   const float *w, float alpha, int mode);
int orc_adamw(int64_t count, float *z, const float *g, float *m, float *v, double lr,
              double b1, double b2, double eps, double wd, uint32_t t);
int orc_sample_logits(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
                      uint32_t tensor_id, uint64_t seed, uint32_t step, float kappa, float tau,
                      uint32_t flags, const float *z, float *a_out);
int orc_mp_fwd(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
               uint32_t tensor_id, uint64_t seed, uint32_t step, uint32_t flags,
               const float *w, const float *pi, uint8_t *order_out, uint8_t *bits,
               uint16_t *out_bf16, float *out_f32);
int orc_mp_logp(int n, int m, int64_t nblocks, const float *pi, const uint8_t *order,
                double *logp);
int orc_mp_grad(int n, int m, int64_t rows, int64_t cols, uint64_t block_offset,
                uint32_t tensor_id, uint64_t seed, uint32_t step, uint32_t flags,
                const float *pi, const uint8_t *order_in, double advantage,
                const float *dpi_prev, double *dpi);
int orc_mp_init(int n, int m, int64_t rows, int64_t cols, const uint8_t *prior_bits,
                const float *w, float c, float *pi);
int orc_mp_baseline(int64_t steps, const double *residual, double mu, double *b_inout,
                    double *adv);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float frand(void) { /* xorshift64*, uniform in [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    uint64_t r = rng_state * 0x2545F4914F6CDD1Dull;
    return (float)((double)(r >> 11) * 0x1p-52 - 1.0);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) exit(3);
    return p;
}

#define CHECK(call)                                                   \
    do {                                                              \
        int rc_ = (call);                                             \
        if (rc_ != 0) {                                               \
            fprintf(stderr, "%s:%d: %s -> %d\n", __FILE__, __LINE__, #call, rc_); \
            return 1;                                                 \
        }                                                             \
    } while (0)

static int one_shape(int n, int m, int64_t rows, int64_t cols, uint64_t off) {
    uint8_t cand[128];
    const int K = orc_candidates(n, m, cand, 128);
    if (K < 1) return 1;
    const int64_t B = rows * (cols / m), W = rows * cols;
    float *w = xmalloc(sizeof(float) * (size_t)W), *g = xmalloc(sizeof(float) * (size_t)W);
    float *z = xmalloc(sizeof(float) * (size_t)(B * K)), *zp = xmalloc(sizeof(float) * (size_t)(B * K));
    double *y = xmalloc(sizeof(double) * (size_t)(B * K)), *mk = xmalloc(sizeof(double) * (size_t)(B * m));
    double *dz = xmalloc(sizeof(double) * (size_t)(B * K));
    uint16_t *o16 = xmalloc(2 * (size_t)W);
    float *o32 = xmalloc(4 * (size_t)W), *a = xmalloc(4 * (size_t)(B * K));
    uint8_t *idx = xmalloc((size_t)B), *bits = xmalloc((size_t)((B * m + 7) / 8));
    uint16_t *vals = xmalloc(2 * (size_t)(B * n));
    uint8_t *vidx = xmalloc((size_t)((B + 1) / 2));
    for (int64_t i = 0; i < W; ++i) {
        w[i] = 0.02f * frand();
        g[i] = 1e-3f * frand();
    }
    for (int64_t i = 0; i < B * K; ++i) z[i] = frand();
    if (B > 1)
        for (int k = 0; k < K; ++k) z[K + k] = 0.5f; /* a block of ties */
    for (int64_t i = 0; i < W; i += 7) w[i] = 0.25f;  /* magnitude ties */
    double reg = 0.0;
    const uint32_t flags[3] = {0u, 1u, 4u};            /* noise, no noise, hard sample */
    for (int f = 0; f < 3; ++f) {
        CHECK(orc_fwd(n, m, rows, cols, off, 3, 0x123456789ull, 7, 100.0f, 0.05f, flags[f], w, z,
                      y, mk, o16, o32, &reg));
        CHECK(orc_bwd(n, m, rows, cols, off, 3, 0x123456789ull, 7, 100.0f, 0.05f, flags[f], w, z,
                      g, 1e-5, f == 1 ? z : NULL, dz));
        CHECK(orc_sample_logits(n, m, rows, cols, off, 3, 9, 2, 100.0f, 4.0f, flags[f], z, a));
    }
    for (int64_t i = 0; i < W; ++i) o16[i] = (uint16_t)(lrintf(w[i] * 1000.0f) & 0xFFFF);
    CHECK(orc_hard_extract(n, m, rows, cols, z, n == 2 && m == 4 ? (const void *)o16 : NULL, 2,
                           idx, bits, n == 2 && m == 4 ? (void *)vals : NULL,
                           n == 2 && m == 4 ? vidx : NULL));
    if (n == 2 && m == 4)
        CHECK(orc_hard_extract(n, m, rows, cols, z, w, 4, NULL, NULL, o32, vidx));
    CHECK(orc_magnitude_mask(n, m, rows, cols, w, bits));
    for (int mode = 0; mode < 2; ++mode) {
        memcpy(zp, z, sizeof(float) * (size_t)(B * K));
        CHECK(orc_prior_init(n, m, rows, cols, zp, bits, NULL, 3.0f, mode));
        CHECK(orc_prior_init(n, m, rows, cols, zp, NULL, w, 3.0f, mode));
    }
    {
        float *gz = xmalloc(4 * (size_t)(B * K)), *m1 = xmalloc(4 * (size_t)(B * K));
        float *m2 = xmalloc(4 * (size_t)(B * K));
        for (int64_t i = 0; i < B * K; ++i) {
            gz[i] = (float)dz[i];
            m1[i] = 0.0f;
            m2[i] = 0.0f;
        }
        for (uint32_t t = 1; t <= 3; ++t)
            CHECK(orc_adamw(B * K, zp, gz, m1, m2, 5e-4, 0.9, 0.999, 1e-8, 0.1, t));
        free(gz);
        free(m1);
        free(m2);
    }
    /* linear-space variant */
    {
        float *pi = xmalloc(4 * (size_t)(B * m));
        uint8_t *ord = xmalloc((size_t)(B * n));
        double *lp = xmalloc(8 * (size_t)B), *dpi = xmalloc(8 * (size_t)(B * m));
        CHECK(orc_mp_init(n, m, rows, cols, NULL, w, 3.0f, pi));
        CHECK(orc_mp_init(n, m, rows, cols, bits, NULL, 2.0f, pi));
        for (int64_t i = 0; i < B * m; ++i) pi[i] += frand();
        for (uint32_t f = 0; f < 2; ++f) {
            CHECK(orc_mp_fwd(n, m, rows, cols, off, 5, 77, 3, f, w, pi, ord, bits, o16, o32));
            CHECK(orc_mp_logp(n, m, B, pi, ord, lp));
            CHECK(orc_mp_grad(n, m, rows, cols, off, 5, 77, 3, f, pi, ord, 0.5, NULL, dpi));
            CHECK(orc_mp_grad(n, m, rows, cols, off, 5, 77, 3, f, pi, NULL, -0.5, pi, dpi));
        }
        free(pi);
        free(ord);
        free(lp);
        free(dpi);
    }
    free(w); free(g); free(z); free(zp); free(y); free(mk); free(dz); free(o16); free(o32);
    free(a); free(idx); free(bits); free(vals); free(vidx);
    return 0;
}

int main(void) {
    orc_set_threads(2);
    uint32_t words[37];
    orc_philox_words(UINT64_C(0xFFFFFFFFFFFFFFFF), 0xFFFFFFFFu, 9, UINT64_C(0xFFFFFFFFFFFFFFF0), 37,
                     words);
    volatile float gsum = 0.0f;
    for (int i = 0; i < 37; ++i) gsum += orc_gumbel(words[i]);
    (void)gsum;
    const int shapes[][4] = {{2, 4, 7, 12}, {2, 4, 1, 4}, {4, 8, 5, 24}, {4, 8, 1, 8}, {1, 4, 3, 8}};
    for (int s = 0; s < 5; ++s)
        for (uint64_t off = 0; off < 3; ++off)
            if (one_shape(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], off)) return 1;
    /* empty tensors */
    if (one_shape(2, 4, 0, 8, 0) || one_shape(4, 8, 3, 0, 1)) return 1;
    double res[5] = {0.3, -0.1, 0.2, 0.0, 0.4}, adv[5], b = 0.0;
    if (orc_mp_baseline(5, res, 0.9, &b, adv)) return 1;
    printf("oracle sanitizer driver ok\n");
    return 0;
}
