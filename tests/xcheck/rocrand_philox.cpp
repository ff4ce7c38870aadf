// Cross-check harness: prints Philox4x32-10 output words computed by rocRAND
// (rocrand/rocrand_philox4x32_10.h, called through its public device/host API).
// stdin: lines "seed subsequence offset" (decimal, offset in 32-bit words, a
// multiple of 4); stdout: 4 hex words per line.  rocRAND's counter is
// (offset/4 lo, hi, subsequence lo, hi) and its key (seed lo, seed hi).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, subseq, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
        rocrand_state_philox4x32_10 s;
        rocrand_init(seed, subseq, offset, &s);
        for (int i = 0; i < 4; ++i) std::printf("%08x%c", rocrand(&s), i == 3 ? '\n' : ' ');
    }
    return 0;
}
