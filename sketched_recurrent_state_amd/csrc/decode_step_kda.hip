// decode_step_kda.hip -- the single-launch serving step for one rule (see decode_step.hpp).
#include "decode_step.hpp"

namespace ssm {

template hipError_t launch_decode_step_rule<KDA>(
    const ssm_dims&, int, const int32_t*, const int32_t*, const int32_t*, int, const int32_t*,
    float*, void*, void*, const float*, const void*, const void*, const void*, const float*,
    const float*, void*, void*, float*, float*, float*, hipStream_t);

}  // namespace ssm
