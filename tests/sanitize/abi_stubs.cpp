// Launcher stubs for the host sanitizer build of the C-ABI layer (test
// infrastructure): the argument checks of maskgs_api.hip run for real, and a
// call that passes them records which launcher it reached instead of
// enqueueing a kernel.  Built by tests/test_sanitize.py.
#include <hip/hip_runtime.h>

#include "maskgs_launch.hpp"
#include "maskpro_launch.hpp"

int g_launches = 0;

namespace maskgs {
#define STUB(sig) hipError_t sig { ++g_launches; return hipSuccess; }
STUB(launch_fwd24(const FwdArgs &, maskgs_dtype, maskgs_dtype, hipStream_t))
STUB(launch_bwd24(const BwdArgs &, maskgs_dtype, maskgs_dtype, hipStream_t))
STUB(launch_reg24(const RegArgs &, maskgs_dtype, hipStream_t))
STUB(launch_hard24(const HardArgs &, maskgs_dtype, hipStream_t))
STUB(launch_prior24(const PriorArgs &, maskgs_dtype, hipStream_t))
STUB(launch_stats24(const StatsArgs &, bool, maskgs_dtype, hipStream_t))
STUB(launch_fwd48(const FwdArgs &, maskgs_dtype, maskgs_dtype, hipStream_t))
STUB(launch_bwd48(const BwdArgs &, maskgs_dtype, maskgs_dtype, hipStream_t))
STUB(launch_reg48(const RegArgs &, maskgs_dtype, hipStream_t))
STUB(launch_hard48(const HardArgs &, hipStream_t))
STUB(launch_prior48(const PriorArgs &, maskgs_dtype, hipStream_t))
STUB(launch_stats48(const StatsArgs &, bool, maskgs_dtype, hipStream_t))
STUB(launch_debug_philox(uint64_t, uint32_t, uint32_t, uint64_t, int64_t, uint32_t *, hipStream_t))
STUB(launch_debug_gumbel(const uint32_t *, int64_t, float *, hipStream_t))
STUB(launch_mp_fwd(const MpArgs &, int, maskgs_dtype, maskgs_dtype, hipStream_t))
STUB(launch_mp_bwd(const MpArgs &, int, hipStream_t))
STUB(launch_mp_init(const MpInitArgs &, int, maskgs_dtype, hipStream_t))
#undef STUB
}  // namespace maskgs
