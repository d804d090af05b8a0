// decode.hip -- the exact read of the window-start state (the comparison path
// that still reads all of S), y = S_win^T q~ + intra after the buffer walk of
// read_walk.hpp, and the entry to the per-rule sketch-read launchers.
#include "common.hpp"
#include "launch.hpp"
#include "read_walk.hpp"

namespace ssm {

template <int RULE>
hipError_t launch_sketch_decode_rule(const ssm_dims& d, const int32_t* rank_offsets,
                                     const void* sketch, const float* basis, const void* q,
                                     const void* k_t, const void* v_t, const float* decay_t,
                                     const float* beta_t, void* k_buf, void* v_buf,
                                     float* decay_buf, float* beta_buf, int tau, float* y,
                                     hipStream_t stream, const Varlen* varlen, bool per_unit_map);

template <int RULE>
hipError_t launch_decode_step_rule(const ssm_dims& d, int num_slots, const int32_t* slot,
                                   const int32_t* tau, const int32_t* parity, int n_update,
                                   const int32_t* update_rows, float* state, void* sketch0,
                                   void* sketch1, const float* basis, const void* q,
                                   const void* k_t, const void* v_t, const float* decay_t,
                                   const float* beta_t, void* k_buf, void* v_buf,
                                   float* decay_buf, float* beta_buf, float* y,
                                   hipStream_t stream);

namespace {

// ---------------------------------------------------------------------------
// exact read of the window-start state: the state tile layout, one workgroup
// per unit. The query and the window are fetched first (the walk needs them
// first, and small reads issued behind a 64 KB state stream wait for all of
// it); the state loads follow and land while every wave walks the buffer on
// its own (no synchronisation after the staging barrier).
// ---------------------------------------------------------------------------
template <int RULE, int DK, int DV, typename TIN>
__global__ void __launch_bounds__((TileLayout<DK, DV>::NT))
full_read_kernel(const float* __restrict__ state, const TIN* __restrict__ q,
                 const TIN* __restrict__ k_t, const TIN* __restrict__ v_t,
                 const float* __restrict__ d_t, const float* __restrict__ b_t,
                 TIN* __restrict__ kbuf, TIN* __restrict__ vbuf, float* __restrict__ dbuf,
                 float* __restrict__ bbuf, float* __restrict__ y, int window, int tau) {
  using TL = TileLayout<DK, DV>;
  constexpr int CG = TL::CG, RPL = TL::RPL, NT = TL::NT;
  constexpr int DSTR = (RULE == KDA) ? DK : 1;
  constexpr int EA = (RULE == KDA) ? RPL : 1;

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);

  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane % CG, rg = lane / CG;
  const int col = wave * (4 * CG) + cg * 4;
  const int row0 = rg * RPL;
  const size_t slot0 = (size_t)unit * window;
  const bool fused = (k_t != nullptr);

  float u[RPL];
  Vec<TIN, RPL>::load(q + (size_t)unit * DK + row0, u);

  UnitWindow<TIN> uw{kbuf + slot0 * DK, vbuf + slot0 * DV, dbuf + slot0 * DSTR,
                     (RULE == MAMBA2) ? nullptr : bbuf + slot0,
                     fused ? k_t + (size_t)unit * DK : nullptr,
                     fused ? v_t + (size_t)unit * DV : nullptr,
                     fused ? d_t + (size_t)unit * DSTR : nullptr,
                     (fused && RULE != MAMBA2) ? b_t + unit : nullptr};
  WindowStage<RULE, DK, DV, TIN, NT> stage;
  stage.issue(uw, tau, tid);
  const float* Su = state + (size_t)unit * (DK * DV);
  float4 s[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
    s[m] = load_stream(Su + (size_t)(row0 + m) * DV + col);
  stage.commit(lds, uw, tau, tid);
  __syncthreads();
  const float* lk = lds;
  const float* lv = lk + tau * DK;
  const float* ld = lv + tau * DV;
  const float* lb = ld + pad4(tau * DSTR);

  float4 acc = f4(0.f);
#pragma unroll 1  // the walk holds cross-lane (convergent) reductions
  for (int i = tau - 1; i >= 0; --i) {
    float kk[RPL], a[EA];
    Vec<float, RPL>::load(lk + i * DK + row0, kk);
    const float4 vv = *reinterpret_cast<const float4*>(lv + i * DV + col);
    if constexpr (RULE == KDA) {
      Vec<float, RPL>::load(ld + i * DK + row0, a);
    } else {
      a[0] = ld[i];
    }
    const float b = (RULE == MAMBA2) ? 1.f : lb[i];
    float sd = 0.f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) sd = fmaf(kk[m], u[m], sd);
    sd = tile_sum<CG>(sd);
    const float bs = b * sd;
    acc = fma4(bs, vv, acc);
    carry_back<RULE, RPL>(u, kk, a, bs);
  }

  float4 out = f4(0.f);
#pragma unroll
  for (int m = 0; m < RPL; ++m) out = fma4(u[m], s[m], out);
  out = add4(tile_sum<CG>(out), acc);
  if (rg == 0) *reinterpret_cast<float4*>(y + (size_t)unit * DV + col) = out;
}

}  // namespace

hipError_t launch_sketch_decode(const ssm_dims& d, const int32_t* rank_offsets,
                                const void* sketch, const float* basis, const void* q,
                                const void* k_t, const void* v_t, const float* decay_t,
                                const float* beta_t, void* k_buf, void* v_buf, float* decay_buf,
                                float* beta_buf, int tau, float* y, hipStream_t stream,
                                const Varlen* varlen, bool per_unit_map) {
  switch (d.rule) {
    case SSM_MAMBA2:
      return launch_sketch_decode_rule<MAMBA2>(d, rank_offsets, sketch, basis, q, k_t, v_t,
                                               decay_t, beta_t, k_buf, v_buf, decay_buf,
                                               beta_buf, tau, y, stream, varlen, per_unit_map);
    case SSM_GDN:
      return launch_sketch_decode_rule<GDN>(d, rank_offsets, sketch, basis, q, k_t, v_t, decay_t,
                                            beta_t, k_buf, v_buf, decay_buf, beta_buf, tau, y,
                                            stream, varlen, per_unit_map);
    case SSM_KDA:
      return launch_sketch_decode_rule<KDA>(d, rank_offsets, sketch, basis, q, k_t, v_t, decay_t,
                                            beta_t, k_buf, v_buf, decay_buf, beta_buf, tau, y,
                                            stream, varlen, per_unit_map);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(const ssm_dims& d, int num_slots, const int32_t* slot,
                              const int32_t* tau, const int32_t* parity, int n_update,
                              const int32_t* update_rows, float* state, void* sketch0,
                              void* sketch1, const float* basis, const void* q, const void* k_t,
                              const void* v_t, const float* decay_t, const float* beta_t,
                              void* k_buf, void* v_buf, float* decay_buf, float* beta_buf,
                              float* y, hipStream_t stream) {
  switch (d.rule) {
    case SSM_MAMBA2:
      return launch_decode_step_rule<MAMBA2>(d, num_slots, slot, tau, parity, n_update,
                                             update_rows, state, sketch0, sketch1, basis, q, k_t,
                                             v_t, decay_t, beta_t, k_buf, v_buf, decay_buf,
                                             beta_buf, y, stream);
    case SSM_GDN:
      return launch_decode_step_rule<GDN>(d, num_slots, slot, tau, parity, n_update, update_rows,
                                          state, sketch0, sketch1, basis, q, k_t, v_t, decay_t,
                                          beta_t, k_buf, v_buf, decay_buf, beta_buf, y, stream);
    case SSM_KDA:
      return launch_decode_step_rule<KDA>(d, num_slots, slot, tau, parity, n_update, update_rows,
                                          state, sketch0, sketch1, basis, q, k_t, v_t, decay_t,
                                          beta_t, k_buf, v_buf, decay_buf, beta_buf, y, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_full_read_decode(const ssm_dims& d, const float* state, const void* q,
                                   const void* k_t, const void* v_t, const float* decay_t,
                                   const float* beta_t, void* k_buf, void* v_buf,
                                   float* decay_buf, float* beta_buf, int tau, float* y,
                                   hipStream_t stream) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  return dispatch(d.rule, d.in_dtype, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = decltype(R)::value, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    const size_t lds = (size_t)window_lds_floats<kR, kDK, kDV>(tau) * sizeof(float);
    hipLaunchKernelGGL((full_read_kernel<kR, kDK, kDV, TIN>), dim3(units),
                       dim3(TileLayout<kDK, kDV>::NT), lds,
                       stream, state, static_cast<const TIN*>(q), static_cast<const TIN*>(k_t),
                       static_cast<const TIN*>(v_t), decay_t, beta_t, static_cast<TIN*>(k_buf),
                       static_cast<TIN*>(v_buf), decay_buf, beta_buf, y, d.window, tau);
    return hipGetLastError();
  });
}

}  // namespace ssm
