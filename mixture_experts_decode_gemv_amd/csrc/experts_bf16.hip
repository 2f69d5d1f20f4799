// Instances of the GEMV expert passes for bf16 expert weights.
#include "experts_impl.h"

namespace moe {
template hipError_t launch_pass1<MOE_BF16>(int, int, hipStream_t, const Pass1Args &);
template hipError_t launch_pass2<MOE_BF16>(int, int, int, hipStream_t, const Pass2Args &);
template hipError_t launch_pass2c<MOE_BF16>(int, int, hipStream_t, const Pass2cArgs &);
}  // namespace moe
