// launch.hpp -- internal interface between the C ABI (abi.hip) and the kernel
// translation units. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"
#include "sketchssm.h"

namespace ssm {

inline RankTable make_rank_table(const int32_t* rank_offsets, int heads) {
  RankTable t;
  t.heads = heads;
  for (int h = 0; h <= heads; ++h) t.off[h] = rank_offsets[h];
  // heads by rank, largest first, ties by index (a stable insertion sort; heads <= 256)
  for (int h = 0; h < heads; ++h) {
    const int r = t.off[h + 1] - t.off[h];
    int i = h;
    while (i > 0 && t.off[t.order[i - 1] + 1] - t.off[t.order[i - 1]] < r) {
      t.order[i] = t.order[i - 1];
      --i;
    }
    t.order[i] = (uint8_t)h;
  }
  return t;
}

template <typename T>
struct type_tag {
  using type = T;
};

// Calls f(d_k, d_v, type_tag<input type>) with compile-time constants for every
// supported combination; returns hipErrorInvalidValue for anything else.
template <typename F>
hipError_t dispatch_shape(int in_dtype, int dk, int dv, F&& f) {
  auto with_dv = [&](auto DK, auto T) -> hipError_t {
    switch (dv) {
      case 16: return f(DK, std::integral_constant<int, 16>{}, T);
      case 32: return f(DK, std::integral_constant<int, 32>{}, T);
      case 64: return f(DK, std::integral_constant<int, 64>{}, T);
      case 128: return f(DK, std::integral_constant<int, 128>{}, T);
    }
    return hipErrorInvalidValue;
  };
  auto with_dk = [&](auto T) -> hipError_t {
    switch (dk) {
      case 16: return with_dv(std::integral_constant<int, 16>{}, T);
      case 32: return with_dv(std::integral_constant<int, 32>{}, T);
      case 64: return with_dv(std::integral_constant<int, 64>{}, T);
      case 128: return with_dv(std::integral_constant<int, 128>{}, T);
    }
    return hipErrorInvalidValue;
  };
  if (in_dtype == SSM_IN_BF16) return with_dk(type_tag<uint16_t>{});
  if (in_dtype == SSM_IN_F32) return with_dk(type_tag<float>{});
  return hipErrorInvalidValue;
}

// Calls f(rule, d_k, d_v, type_tag<input type>) with compile-time constants for
// every supported combination; returns hipErrorInvalidValue for anything else.
template <typename F>
hipError_t dispatch(int rule, int in_dtype, int dk, int dv, F&& f) {
  auto with_dv = [&](auto R, auto DK, auto T) -> hipError_t {
    switch (dv) {
      case 16: return f(R, DK, std::integral_constant<int, 16>{}, T);
      case 32: return f(R, DK, std::integral_constant<int, 32>{}, T);
      case 64: return f(R, DK, std::integral_constant<int, 64>{}, T);
      case 128: return f(R, DK, std::integral_constant<int, 128>{}, T);
    }
    return hipErrorInvalidValue;
  };
  auto with_dk = [&](auto R, auto T) -> hipError_t {
    switch (dk) {
      case 16: return with_dv(R, std::integral_constant<int, 16>{}, T);
      case 32: return with_dv(R, std::integral_constant<int, 32>{}, T);
      case 64: return with_dv(R, std::integral_constant<int, 64>{}, T);
      case 128: return with_dv(R, std::integral_constant<int, 128>{}, T);
    }
    return hipErrorInvalidValue;
  };
  auto with_t = [&](auto R) -> hipError_t {
    if (in_dtype == SSM_IN_BF16) return with_dk(R, type_tag<uint16_t>{});
    if (in_dtype == SSM_IN_F32) return with_dk(R, type_tag<float>{});
    return hipErrorInvalidValue;
  };
  switch (rule) {
    case SSM_MAMBA2: return with_t(std::integral_constant<int, SSM_MAMBA2>{});
    case SSM_GDN: return with_t(std::integral_constant<int, SSM_GDN>{});
    case SSM_KDA: return with_t(std::integral_constant<int, SSM_KDA>{});
  }
  return hipErrorInvalidValue;
}

// Calls f(type_tag<sketch element type>) for d.sketch_dtype (fp32 or bf16 bits).
template <typename F>
hipError_t with_sketch_type(const ssm_dims& d, F&& f) {
  if (d.sketch_dtype == SSM_SKETCH_BF16) return f(type_tag<uint16_t>{});
  return f(type_tag<float>{});
}

// Per-head ranks: rank_offsets is a host array of heads + 1 prefix offsets (checked by the
// caller), or nullptr for the uniform rank d.rank.
inline int max_rank_of(const int32_t* rank_offsets, int heads) {
  int m = 0;
  for (int h = 0; h < heads; ++h) {
    const int r = rank_offsets[h + 1] - rank_offsets[h];
    m = r > m ? r : m;
  }
  return m;
}

// Bytes of dynamic LDS the update kernel needs for n staged tokens and a basis of max_rank rows
// (ls: plus the least-squares refresh's work space).
size_t update_refresh_lds_bytes(const ssm_dims& d, int n_tokens, int max_rank, bool ls);

// varlen != nullptr: per-row slots and token counts (n_tokens is then ignored).
// read_map != nullptr: the least-squares refresh (fp32 sketch, uniform rank, no varlen).
hipError_t launch_update_refresh(const ssm_dims& d, const int32_t* rank_offsets, float* state,
                                 void* sketch, const float* basis, const void* k_buf,
                                 const void* v_buf, const float* decay_buf, const float* beta_buf,
                                 int n_tokens, hipStream_t stream,
                                 const Varlen* varlen = nullptr, float* read_map = nullptr);

// per_unit_map: `basis` is a per-unit read map [N][H][r][d_k] (least-squares
// coefficients) instead of the per-head basis.
hipError_t launch_sketch_decode(const ssm_dims& d, const int32_t* rank_offsets,
                                const void* sketch, const float* basis,
                                const void* q, const void* k_t, const void* v_t,
                                const float* decay_t, const float* beta_t, void* k_buf,
                                void* v_buf, float* decay_buf, float* beta_buf, int tau, float* y,
                                hipStream_t stream, const Varlen* varlen = nullptr,
                                bool per_unit_map = false);

// The single-launch serving step (decode_step.hpp): the read of every batch row at its own
// window position with the fused append, and the window update of the n_update listed rows,
// with a double-buffered sketch chosen per row by parity.
hipError_t launch_decode_step(const ssm_dims& d, int num_slots, const int32_t* slot,
                              const int32_t* tau, const int32_t* parity, int n_update,
                              const int32_t* update_rows, float* state, void* sketch0,
                              void* sketch1, const float* basis, const void* q, const void* k_t,
                              const void* v_t, const float* decay_t, const float* beta_t,
                              void* k_buf, void* v_buf, float* decay_buf, float* beta_buf,
                              float* y, hipStream_t stream);

hipError_t launch_full_read_decode(const ssm_dims& d, const float* state, const void* q,
                                   const void* k_t, const void* v_t, const float* decay_t,
                                   const float* beta_t, void* k_buf, void* v_buf,
                                   float* decay_buf, float* beta_buf, int tau, float* y,
                                   hipStream_t stream);

hipError_t launch_buffer_append(const ssm_dims& d, const void* k_t, const void* v_t,
                                const float* decay_t, const float* beta_t, void* k_buf,
                                void* v_buf, float* decay_buf, float* beta_buf, int slot,
                                hipStream_t stream);

hipError_t launch_recurrent_step(const ssm_dims& d, float* state, const void* q, const void* k_t,
                                 const void* v_t, const float* decay_t, const float* beta_t,
                                 float* y, hipStream_t stream);

hipError_t launch_fit_basis(const ssm_dims& d, const void* samples, int n_samples, float* basis,
                            hipStream_t stream);

hipError_t launch_stream_probe(float* buf, long long n_tiles, int shape, hipStream_t stream);

}  // namespace ssm
