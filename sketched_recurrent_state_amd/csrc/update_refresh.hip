// update_refresh.hip -- the shared-memory size of the window update and the entry to
// its per-rule launchers (update_refresh.hpp, update_refresh_<rule>.hip).
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

template <int RULE>
hipError_t launch_update_refresh_rule(const ssm_dims& d, const int32_t* rank_offsets,
                                      float* state, void* sketch, const float* basis,
                                      const void* k_buf, const void* v_buf,
                                      const float* decay_buf, const float* beta_buf, int n,
                                      hipStream_t stream, const Varlen* varlen, float* read_map);

size_t update_refresh_lds_bytes(const ssm_dims& d, int n, int max_rank, bool ls) {
  size_t floats = 0;
  (void)dispatch(d.rule, SSM_IN_F32, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto) {
    floats = (size_t)window_lds_floats<decltype(R)::value, decltype(DK)::value,
                                       decltype(DV)::value>(n);
    return hipSuccess;
  });
  // least squares: the sketch rows [r][d_v], the waves' partial read maps [waves][r][d_k]
  // (one wave per 32 columns, one at d_v = 16) and the Gram matrix / Cholesky factor [r][r]
  // in fp64
  const size_t waves = d.d_v >= 32 ? (size_t)(d.d_v / 32) : 1;
  const size_t ls_floats = ls ? (size_t)max_rank * d.d_v + waves * max_rank * d.d_k +
                                    2 * (size_t)max_rank * max_rank
                              : 0;
  return (floats + (size_t)max_rank * d.d_k + ls_floats) * sizeof(float);
}

hipError_t launch_update_refresh(const ssm_dims& d, const int32_t* rank_offsets, float* state,
                                 void* sketch, const float* basis, const void* k_buf,
                                 const void* v_buf, const float* decay_buf, const float* beta_buf,
                                 int n, hipStream_t stream, const Varlen* varlen, float* read_map) {
  switch (d.rule) {
    case SSM_MAMBA2:
      return launch_update_refresh_rule<MAMBA2>(d, rank_offsets, state, sketch, basis, k_buf,
                                                v_buf, decay_buf, beta_buf, n, stream, varlen,
                                                read_map);
    case SSM_GDN:
      return launch_update_refresh_rule<GDN>(d, rank_offsets, state, sketch, basis, k_buf, v_buf,
                                             decay_buf, beta_buf, n, stream, varlen, read_map);
    case SSM_KDA:
      return launch_update_refresh_rule<KDA>(d, rank_offsets, state, sketch, basis, k_buf, v_buf,
                                             decay_buf, beta_buf, n, stream, varlen, read_map);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
