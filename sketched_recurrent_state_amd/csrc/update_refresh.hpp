// update_refresh.hpp -- the window update + refresh launched on its own: one
// workgroup per (sequence, head) unit runs the body of update_body.hpp. The
// launcher is instantiated once per rule, each in its own translation unit
// (update_refresh_<rule>.hip), so the instantiations compile in parallel.
// Workgroups are dealt to the 8 XCDs in turn; the block index is remapped so
// each XCD streams one contiguous run of units (with the interleaved rows of
// the body, about 5% faster than contiguous rows per lane in the natural block
// order).
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "update_body.hpp"

namespace ssm {

namespace {

template <int RULE, int DK, int DV, typename TIN, typename TSK, bool LS, typename RT, typename RM,
          bool MMA>
__global__ void __launch_bounds__((TileLayout<DK, DV>::NT), 4)
update_refresh_kernel(float* __restrict__ state, TSK* __restrict__ sketch,
                      float* __restrict__ rmap,
                      const float* __restrict__ basis, const TIN* __restrict__ kbuf,
                      const TIN* __restrict__ vbuf, const float* __restrict__ dbuf,
                      const float* __restrict__ bbuf, int heads, int window, const RT rt,
                      const RM rm) {
  // XCD x = blockIdx.x % 8 receives blocks x, x + 8, ...: give it the contiguous
  // run of units [x * q8 + min(x, rem), ...) instead (a bijection on the grid).
  const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, rem = G & 7;
  const int b = xcd * q8 + min(xcd, rem) + (blockIdx.x >> 3);
  int seq = 0, n = 0;  // the batch row's persistent slot and its number of buffered tokens
  if (!rm.row(b / heads, seq, n)) return;  // whole workgroup: a skipped row
  update_refresh_unit<RULE, DK, DV, TIN, TSK, LS, RT, MMA>(state, sketch, rmap, basis, kbuf, vbuf,
                                                      dbuf, bbuf, heads, window, rt, b % heads,
                                                      seq, n, CurrentToken<TIN>{});
}

}  // namespace

template <int RULE>
hipError_t launch_update_refresh_rule(const ssm_dims& d, const int32_t* rank_offsets,
                                      float* state, void* sketch, const float* basis,
                                      const void* k_buf, const void* v_buf,
                                      const float* decay_buf, const float* beta_buf, int n,
                                      hipStream_t stream, const Varlen* varlen, float* read_map) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  int max_rank = 0;
  if (sketch != nullptr) max_rank = rank_offsets ? max_rank_of(rank_offsets, d.heads) : d.rank;
  // a variable-length call can stage up to W tokens per row
  const size_t lds = update_refresh_lds_bytes(d, varlen ? d.window : n, max_rank, read_map != nullptr);
  return dispatch_shape(d.in_dtype, d.d_k, d.d_v, [&](auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = RULE, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    constexpr unsigned NT = TileLayout<kDK, kDV>::NT;
    if (read_map != nullptr) {  // least squares: fp32 sketch, uniform rank, lockstep
      hipLaunchKernelGGL(
          (update_refresh_kernel<kR, kDK, kDV, TIN, float, true, UniformRank, Lockstep, false>),
          dim3(units), dim3(NT), lds, stream, state, static_cast<float*>(sketch), read_map,
          basis, static_cast<const TIN*>(k_buf), static_cast<const TIN*>(v_buf), decay_buf,
          beta_buf, d.heads, d.window, UniformRank{d.rank, d.heads}, Lockstep{n});
      return hipGetLastError();
    }
    return with_sketch_type(d, [&](auto SK) {
      using TSK = typename decltype(SK)::type;
      auto launch = [&](auto rt, auto rm, auto mma) {
        hipLaunchKernelGGL((update_refresh_kernel<kR, kDK, kDV, TIN, TSK, false, decltype(rt),
                                                  decltype(rm), decltype(mma)::value>),
                           dim3(units), dim3(NT), lds, stream, state, static_cast<TSK*>(sketch),
                           nullptr, basis, static_cast<const TIN*>(k_buf),
                           static_cast<const TIN*>(v_buf), decay_buf, beta_buf, d.heads,
                           d.window, rt, rm);
        return hipGetLastError();
      };
      // The refresh on the matrix cores (d_k >= 64, d_v >= 32) where its vector time would
      // show: above rank 8 in every launch, and from rank 8 in the variable-length update,
      // whose calls in a serving step update a fraction of the units in one round of
      // workgroups, so every unit's arithmetic is on the critical path (the single-launch
      // serving step takes the same choice, so the two give the same bits)
      const int mma_from = varlen != nullptr ? 8 : 9;
      auto go = [&](auto rt, auto rm) {
        if constexpr (kDK >= 64 && kDV >= 32) {
          if (sketch != nullptr && max_rank >= mma_from) return launch(rt, rm, std::true_type{});
        }
        return launch(rt, rm, std::false_type{});
      };
      if (varlen != nullptr) return go(UniformRank{d.rank, d.heads}, *varlen);
      if (rank_offsets == nullptr) return go(UniformRank{d.rank, d.heads}, Lockstep{n});
      return go(make_rank_table(rank_offsets, d.heads), Lockstep{n});
    });
  });
}

}  // namespace ssm
