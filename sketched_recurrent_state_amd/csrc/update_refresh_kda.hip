// update_refresh_kda.hip -- the window-update launcher for one rule (see update_refresh.hpp).
#include "update_refresh.hpp"

namespace ssm {

template hipError_t launch_update_refresh_rule<KDA>(const ssm_dims&, const int32_t*, float*, void*,
                                                   const float*, const void*, const void*,
                                                   const float*, const float*, int, hipStream_t,
                                                   const Varlen*, float*);

}  // namespace ssm
