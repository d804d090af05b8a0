// read_walk.hpp -- the buffer walk shared by the per-step read kernels.
//
// Both reads walk the window buffer newest to oldest from u = q. With token i's
// transition M_i and write weight b_i (beta, or 1 for Mamba-2):
//   s_i = k_i . u,  intra += b_i s_i v_i,  u <- M_i^T u
// which leaves q~ = A^T q in u and R^T q in intra, where S_tau = A S_win + R
// (within a window only the queries change: agihunt.info summary of SketchSSM,
// "Mechanism details").
#pragma once

#include "common.hpp"

namespace ssm {

// Lane j's value of x within each aligned group of G consecutive lanes (G = 16 or 32;
// j uniform): one v_readlane per group of the wave, then a select by the lane's group.
template <int G>
__device__ __forceinline__ float group_bcast(float x, int j) {
  static_assert(G == 16 || G == 32, "group size");
  const int grp = (int)(__lane_id() / G);
  float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
#pragma unroll
  for (int g = 1; g < 64 / G; ++g) {
    const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), g * G + j));
    r = grp == g ? o : r;
  }
  return r;
}

// u <- M^T u for one token on E key elements held by this lane, given s = k . u.
//   Mamba-2: M^T u = a u;  GDN: a (u - beta s k);  KDA: alpha (.) (u - beta s k)
template <int RULE, int E>
__device__ __forceinline__ void carry_back(float* u, const float* kk, const float* a, float bs) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (RULE == MAMBA2) {
      u[e] = a[0] * u[e];
    } else if constexpr (RULE == GDN) {
      u[e] = a[0] * fmaf(-bs, kk[e], u[e]);
    } else {
      u[e] = a[e] * fmaf(-bs, kk[e], u[e]);
    }
  }
}

}  // namespace ssm
