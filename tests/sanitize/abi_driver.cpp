// Host sanitizer driver for the C-ABI layer (test infrastructure): every entry
// point of include/maskgs.h and include/maskpro.h with valid arguments (fake,
// 16-byte aligned device addresses: the launchers are stubs) and with each
// kind of invalid argument; checks the returned status codes.  Exits 0 when
// all of them are as documented and the sanitizers report nothing.
#include <cmath>
#include <cstdio>
#include <cstdint>

#include "maskgs.h"
#include "maskpro.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int got_ = (call);                                                        \
        if (got_ != (want)) {                                                           \
            std::fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #call, got_, \
                         (want));                                                       \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

int main() {
    void *A = reinterpret_cast<void *>(uintptr_t{1} << 20);
    void *U = reinterpret_cast<void *>((uintptr_t{1} << 20) + 4);  // misaligned
    float *Af = static_cast<float *>(A);
    double *Ad = static_cast<double *>(A);
    uint8_t *Ab = static_cast<uint8_t *>(A);
    const maskgs_tensor_desc d24{2, 4, 8, 16, 3, 1}, d48{4, 8, 8, 16, 1, 2};
    const maskgs_tensor_desc bad_nm{3, 8, 8, 16, 0, 0}, bad_cols{2, 4, 8, 18, 0, 0};
    const maskgs_tensor_desc empty{4, 8, 0, 16, 0, 0}, huge{2, 4, INT64_C(1) << 40, 1 << 20, 0, 0};
    maskgs_sample_params p{7, 3, 100.0f, 4.0f, 0u}, pbad{7, 3, 100.0f, 0.0f, 0u};
    maskgs_sample_params phs{7, 3, 100.0f, 4.0f, MASKGS_HARD_SAMPLE};
    maskgs_sample_params pnan{7, 3, std::nanf(""), 4.0f, 0u};
    const maskgs_adamw_params opt{5e-4f, 0.9f, 0.999f, 1e-8f, 0.1f, 1u};
    const maskgs_adamw_params opt_bad{5e-4f, 1.0f, 0.999f, 1e-8f, 0.1f, 1u};
    const maskpro_draw_params dp{9, 2, 0u};

    uint8_t masks[70];
    int32_t k = 0;
    EXPECT(maskgs_candidates(2, 4, masks, 70, &k), MASKGS_OK);
    EXPECT(maskgs_candidates(4, 8, masks, 70, &k), MASKGS_OK);
    EXPECT(maskgs_candidates(4, 8, masks, 69, &k), MASKGS_E_CAPACITY);
    EXPECT(maskgs_candidates(3, 8, masks, 70, &k), MASKGS_E_UNSUPPORTED);
    for (int s = -1; s < 12; ++s)
        if (!maskgs_status_str(s)) ++failures;
    EXPECT(maskgs_abi_version(), MASKGS_ABI_VERSION);

    for (const maskgs_tensor_desc *d : {&d24, &d48}) {
        EXPECT(maskgs_fwd(d, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr), MASKGS_OK);
        EXPECT(maskgs_fwd(d, &pbad, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
               MASKGS_E_RANGE);
        EXPECT(maskgs_fwd(d, &pnan, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
               MASKGS_E_RANGE);
        EXPECT(maskgs_fwd(d, &p, A, MASKGS_BF16, static_cast<float *>(U), A, MASKGS_BF16, Af, Ad,
                          nullptr),
               MASKGS_E_ALIGN);
        EXPECT(maskgs_fwd(d, &p, nullptr, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
               MASKGS_E_NULL);
        EXPECT(maskgs_fwd(d, &p, A, static_cast<maskgs_dtype>(7), Af, A, MASKGS_BF16, Af, Ad,
                          nullptr),
               MASKGS_E_DTYPE);
        EXPECT(maskgs_fwd_hard(d, &p, A, MASKGS_F32, Af, A, MASKGS_F32, nullptr, nullptr, Ab, Ab,
                               nullptr, nullptr, nullptr),
               MASKGS_OK);
        EXPECT(maskgs_bwd(d, &p, A, MASKGS_BF16, Af, nullptr, A, MASKGS_BF16, 1e-5f, Af, 0,
                          nullptr),
               MASKGS_OK);
        EXPECT(maskgs_bwd(d, &p, A, MASKGS_BF16, nullptr, Af, A, MASKGS_F32, 1e-5f, Af, 1,
                          nullptr),
               MASKGS_OK);
        EXPECT(maskgs_bwd(d, &phs, A, MASKGS_BF16, Af, Af, A, MASKGS_BF16, 1e-5f, Af, 0,
                          nullptr),
               MASKGS_E_UNSUPPORTED);
        EXPECT(maskgs_bwd(d, &p, A, MASKGS_BF16, Af, nullptr, A, MASKGS_BF16, -1.0f, Af, 0,
                          nullptr),
               MASKGS_E_RANGE);
        EXPECT(maskgs_bwd_adamw(d, &p, A, MASKGS_BF16, Af, nullptr, A, MASKGS_BF16, 1e-5f, Af, Af,
                                &opt, nullptr),
               MASKGS_OK);
        EXPECT(maskgs_bwd_adamw(d, &p, A, MASKGS_BF16, Af, nullptr, A, MASKGS_BF16, 1e-5f, Af, Af,
                                &opt_bad, nullptr),
               MASKGS_E_RANGE);
        EXPECT(maskgs_reg_reduce(d, &p, A, MASKGS_BF16, Af, nullptr, Ad, nullptr), MASKGS_OK);
        EXPECT(maskgs_hard_extract(d, Af, nullptr, MASKGS_BF16, Ab, Ab, nullptr, nullptr, nullptr),
               MASKGS_OK);
        EXPECT(maskgs_prior_init(d, Af, nullptr, A, MASKGS_BF16, 3.0f, 0, nullptr), MASKGS_OK);
        EXPECT(maskgs_prior_init(d, Af, Ab, nullptr, MASKGS_BF16, 3.0f, 2, nullptr),
               MASKGS_E_RANGE);
        EXPECT(maskgs_mask_stats(d, Af, 100.0f, &p, Ab, A, MASKGS_BF16, Af,
                                 static_cast<maskgs_stats *>(A), nullptr),
               MASKGS_OK);
        EXPECT(maskpro_fwd(d, &dp, A, MASKGS_BF16, Af, A, MASKGS_BF16, Ab, A, nullptr), MASKGS_OK);
        EXPECT(maskpro_fwd(d, &dp, nullptr, MASKGS_BF16, Af, A, MASKGS_BF16, Ab, A, nullptr),
               MASKGS_E_NULL);
        EXPECT(maskpro_bwd(d, &dp, Af, A, 0.5f, Af, 0, nullptr), MASKGS_OK);
        EXPECT(maskpro_bwd(d, &dp, Af, nullptr, std::nanf(""), Af, 0, nullptr), MASKGS_E_RANGE);
        EXPECT(maskpro_init(d, nullptr, A, MASKGS_F32, 3.0f, Af, nullptr), MASKGS_OK);
    }
    EXPECT(maskgs_hard_extract(&d48, Af, A, MASKGS_BF16, nullptr, nullptr, A, nullptr, nullptr),
           MASKGS_E_UNSUPPORTED);
    EXPECT(maskgs_fwd(&bad_nm, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
           MASKGS_E_UNSUPPORTED);
    EXPECT(maskgs_fwd(&bad_cols, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
           MASKGS_E_SHAPE);
    EXPECT(maskgs_fwd(&huge, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
           MASKGS_E_SHAPE);
    // (cols/m) * 80 past int64: 2^62 columns wrap the product to 0, and
    // 3689348814741910324 columns wrap it to 16; both are shape errors
    for (const int64_t wide_cols : {INT64_C(1) << 62, INT64_C(3689348814741910324)})
        for (const int64_t r : {INT64_C(0), INT64_C(1)}) {
            const maskgs_tensor_desc wide{2, 4, r, wide_cols, 0, 0};
            EXPECT(maskgs_fwd(&wide, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
                   MASKGS_E_SHAPE);
            EXPECT(maskpro_fwd(&wide, &dp, A, MASKGS_BF16, Af, A, MASKGS_BF16, Ab, Ab, nullptr),
                   MASKGS_E_SHAPE);
        }
    EXPECT(maskgs_fwd(&empty, &p, nullptr, MASKGS_BF16, nullptr, nullptr, MASKGS_BF16, nullptr,
                      nullptr, nullptr),
           MASKGS_OK);
    EXPECT(maskgs_fwd(nullptr, &p, A, MASKGS_BF16, Af, A, MASKGS_BF16, Af, Ad, nullptr),
           MASKGS_E_NULL);
    EXPECT(maskgs_debug_philox(1, 2, 3, 4, 100, static_cast<uint32_t *>(A), nullptr), MASKGS_OK);
    EXPECT(maskgs_debug_gumbel(static_cast<uint32_t *>(A), 100, Af, nullptr), MASKGS_OK);
    double b = 0.0, adv = 0.0;
    EXPECT(maskpro_baseline(0.25, 0.9, &b, &adv), MASKGS_OK);
    EXPECT(maskpro_baseline(0.25, 1.5, &b, &adv), MASKGS_E_RANGE);

    const int want_launches = 2 * 12 + 2;  // 12 valid calls per pattern, 2 debug hooks
    if (g_launches != want_launches) {
        std::fprintf(stderr, "launches %d, want %d\n", g_launches, want_launches);
        ++failures;
    }
    if (failures) return 1;
    std::printf("abi sanitizer driver ok\n");
    return 0;
}
