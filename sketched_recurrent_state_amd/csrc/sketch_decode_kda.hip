// sketch_decode_kda.hip -- the sketch-read launcher for one rule (see sketch_decode.hpp).
#include "sketch_decode.hpp"

namespace ssm {

template hipError_t launch_sketch_decode_rule<KDA>(
    const ssm_dims&, const int32_t*, const void*, const float*, const void*, const void*,
    const void*, const float*, const float*, void*, void*, float*, float*, int, float*,
    hipStream_t, const Varlen*, bool);

}  // namespace ssm
