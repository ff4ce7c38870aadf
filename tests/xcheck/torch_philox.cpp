// Cross-check harness: prints Philox4x32-10 output words computed by PyTorch's
// own engine (ATen/core/PhiloxRNGEngine.h, called through its public API).
// stdin: lines "seed subsequence offset" (decimal); stdout: 4 hex words per line.
// The engine's counter is (offset_lo, offset_hi, subsequence_lo, subsequence_hi)
// with offset counted in 128-bit outputs, its key (seed_lo, seed_hi).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>

int main() {
    unsigned long long seed, subseq, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
        at::Philox4_32 eng(seed, subseq, offset);
        for (int i = 0; i < 4; ++i) std::printf("%08x%c", eng(), i == 3 ? '\n' : ' ');
    }
    return 0;
}
