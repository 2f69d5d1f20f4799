// Instances of the GEMV expert passes for q4_0 expert weights.
#include "experts_impl.h"

namespace moe {
template hipError_t launch_pass1<MOE_Q4_0>(int, int, hipStream_t, const Pass1Args &);
template hipError_t launch_pass2<MOE_Q4_0>(int, int, int, hipStream_t, const Pass2Args &);
template hipError_t launch_pass2c<MOE_Q4_0>(int, int, hipStream_t, const Pass2cArgs &);
}  // namespace moe
