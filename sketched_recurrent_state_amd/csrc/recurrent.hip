// recurrent.hip -- the per-token recurrent decode step: the standard decode
// of a linear-attention layer that SketchSSM's kernel speedups are measured
// against (readsearch.ai listing of arXiv 2609.33051, Abstract: speedups over
// the standard vLLM baseline; agihunt.info summary, "Background": every decode
// step reads the full recurrent state). Each step applies the current token to
// the full state, writes the state back and reads y = S^T q.
//
// Same state-tile layout and memory order as the windowed update: one
// workgroup per unit, d_v/32 waves (one for d_v = 16), 4 columns x d_k/RG rows
// per lane with row group rg owning the interleaved rows rg, rg + RG, ... (each
// load instruction of the workgroup covers RG whole rows of S), and the block
// index remapped so each XCD streams one contiguous run of units. The d_k
// reductions run over lane bits 3..5 (and 2 for d_v = 16).
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

template <int RULE, int DK, int DV, typename TIN>
__global__ void __launch_bounds__((TileLayout<DK, DV>::NT))
recurrent_step_kernel(float* __restrict__ state, const TIN* __restrict__ q,
                      const TIN* __restrict__ k_t, const TIN* __restrict__ v_t,
                      const float* __restrict__ d_t, const float* __restrict__ b_t,
                      float* __restrict__ y) {
  using TL = TileLayout<DK, DV>;
  constexpr int CG = TL::CG, RG = TL::RG, RPL = TL::RPL, NT = TL::NT;
  constexpr int J = (DK + NT - 1) / NT;  // d_k elements staged per thread
  constexpr int NA = (RULE == KDA) ? DK : 1;
  // one pad slot past d_k takes the clamped lanes' stores
  __shared__ __align__(16) float lk[DK + 4];
  __shared__ __align__(16) float lq[DK + 4];
  __shared__ __align__(16) float la[NA + 4];

  // XCD x = blockIdx.x % 8 receives blocks x, x + 8, ...: give it the contiguous
  // run of units [x * q8 + min(x, rem), ...) instead (a bijection on the grid).
  const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, rem = G & 7;
  const int unit = xcd * q8 + min(xcd, rem) + (blockIdx.x >> 3);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane % CG, rg = lane / CG;
  const int col = wave * (4 * CG) + cg * 4;
  const int row0 = rg * RPL;  // this lane's d_k / RG values in lk, lq, la (interleaved_pos)

  // the token's small inputs first: issued behind the 64 KB state stream they
  // would wait for all of it. Indices are clamped so every lane issues the same
  // loads (the wait for them before the LDS writes stays exact).
  float kx[J], qx[J], ax[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = min(tid + j * NT, DK - 1);
    Vec<TIN, 1>::load(k_t + (size_t)unit * DK + i, &kx[j]);
    Vec<TIN, 1>::load(q + (size_t)unit * DK + i, &qx[j]);
    if constexpr (RULE == KDA) ax[j] = d_t[(size_t)unit * DK + i];
  }
  float vv[4];
  Vec<TIN, 4>::load(v_t + (size_t)unit * DV + col, vv);
  const float4 v4 = make_float4(vv[0], vv[1], vv[2], vv[3]);
  float* Su = state + (size_t)unit * (DK * DV);
  float4 s[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m) s[m] = load_stream(Su + (size_t)(m * RG + rg) * DV + col);

  // k, q (and KDA's per-row gates) to LDS in the interleaved order while the
  // state is in flight; s[m] holds row m * RG + rg. The stores are unconditional
  // (clamped lanes write the pad slot) so the loads above stay where they are.
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = tid + j * NT;
    const int pos = (i < DK) ? interleaved_pos<DK, RG>(i) : DK;
    lk[pos] = kx[j];
    lq[pos] = qx[j];
    if constexpr (RULE == KDA) la[pos] = ax[j];
  }
  __syncthreads();
  float kr[RPL], qr[RPL];
  Vec<float, RPL>::load(lk + row0, kr);
  Vec<float, RPL>::load(lq + row0, qr);
  float ar[(RULE == KDA) ? RPL : 1];
  if constexpr (RULE == KDA) Vec<float, RPL>::load(la + row0, ar);

  // S <- M S + b k v^T
  if constexpr (RULE == MAMBA2) {
    const float a = d_t[unit];
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], v4, scale4(a, s[m]));
  } else if constexpr (RULE == GDN) {
    const float a = d_t[unit], b = b_t[unit];
    float4 p = f4(0.f);
#pragma unroll
    for (int m = 0; m < RPL; ++m) p = fma4(kr[m], s[m], p);
    p = tile_sum<CG>(p);  // S^T k
    const float4 w = scale4(b, sub4(v4, scale4(a, p)));
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, scale4(a, s[m]));
  } else {
    const float b = b_t[unit];
    float4 p = f4(0.f);
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
      s[m] = scale4(ar[m], s[m]);
      p = fma4(kr[m], s[m], p);
    }
    p = tile_sum<CG>(p);
    const float4 w = scale4(b, sub4(v4, p));
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, s[m]);
  }
#pragma unroll
  for (int m = 0; m < RPL; ++m) store_stream(Su + (size_t)(m * RG + rg) * DV + col, s[m]);

  // y = S^T q on the updated state
  float4 out = f4(0.f);
#pragma unroll
  for (int m = 0; m < RPL; ++m) out = fma4(qr[m], s[m], out);
  out = tile_sum<CG>(out);
  if (rg == 0) *reinterpret_cast<float4*>(y + (size_t)unit * DV + col) = out;
}

}  // namespace

hipError_t launch_recurrent_step(const ssm_dims& d, float* state, const void* q, const void* k_t,
                                 const void* v_t, const float* decay_t, const float* beta_t,
                                 float* y, hipStream_t stream) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  return dispatch(d.rule, d.in_dtype, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = decltype(R)::value, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    hipLaunchKernelGGL((recurrent_step_kernel<kR, kDK, kDV, TIN>), dim3(units),
                       dim3(TileLayout<kDK, kDV>::NT), 0,
                       stream, state, static_cast<const TIN*>(q), static_cast<const TIN*>(k_t),
                       static_cast<const TIN*>(v_t), decay_t, beta_t, y);
    return hipGetLastError();
  });
}

}  // namespace ssm
