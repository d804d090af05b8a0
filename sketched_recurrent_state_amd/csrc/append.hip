// append.hip -- token buffering: copy the current token of every unit into
// one slot of the window buffer (the buffering of keys and values between
// state writes that SketchSSM keeps from ReplaySSM; readsearch.ai listing of
// arXiv 2609.33051, Abstract). 16 lanes per unit, 16-byte copies where the
// row allows it.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

template <int RULE, int DK, int DV, typename TIN>
__global__ void __launch_bounds__(256)
append_kernel(const TIN* __restrict__ k_t, const TIN* __restrict__ v_t,
              const float* __restrict__ d_t, const float* __restrict__ b_t,
              TIN* __restrict__ kbuf, TIN* __restrict__ vbuf, float* __restrict__ dbuf,
              float* __restrict__ bbuf, int units, int window, int slot) {
  constexpr int G = 16;
  constexpr int EK = DK / G, EV = DV / G;
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int unit = gid / G, sub = gid % G;
  if (unit >= units) return;
  const size_t dst = (size_t)unit * window + slot;
  Vec<TIN, EK>::copy(k_t + (size_t)unit * DK + sub * EK, kbuf + dst * DK + sub * EK);
  Vec<TIN, EV>::copy(v_t + (size_t)unit * DV + sub * EV, vbuf + dst * DV + sub * EV);
  if constexpr (RULE == KDA) {
    Vec<float, EK>::copy(d_t + (size_t)unit * DK + sub * EK, dbuf + dst * DK + sub * EK);
  } else {
    if (sub == 0) dbuf[dst] = d_t[unit];
  }
  if constexpr (RULE != MAMBA2) {
    if (sub == 1) bbuf[dst] = b_t[unit];
  }
}

}  // namespace

hipError_t launch_buffer_append(const ssm_dims& d, const void* k_t, const void* v_t,
                                const float* decay_t, const float* beta_t, void* k_buf,
                                void* v_buf, float* decay_buf, float* beta_buf, int slot,
                                hipStream_t stream) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  const unsigned blocks = (units * 16u + 255u) / 256u;
  return dispatch(d.rule, d.in_dtype, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = decltype(R)::value, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    hipLaunchKernelGGL((append_kernel<kR, kDK, kDV, TIN>), dim3(blocks), dim3(256), 0, stream,
                       static_cast<const TIN*>(k_t), static_cast<const TIN*>(v_t), decay_t,
                       beta_t, static_cast<TIN*>(k_buf), static_cast<TIN*>(v_buf), decay_buf,
                       beta_buf, (int)units, d.window, slot);
    return hipGetLastError();
  });
}

}  // namespace ssm
