// decode_step.hpp -- one serving decode step over a slot pool in a single launch:
// every batch row reads its output from the sketch at its own window position
// (the current token appended on the way), and the rows whose window fills with
// this token also apply the window to the state and refresh the sketch. The
// SketchSSM pages write the full state once per window and read the sketch on
// every step (readsearch.ai listing of arXiv 2609.33051, Abstract); when the
// sequences of a batch sit at different window positions, a step holds both.
//
// One launch instead of a read launch and an update launch: the update blocks
// of a step are a fraction (1/W in a staggered batch) of a full update and fit
// in one round of workgroups, so alone they load, compute and store together
// with nothing to overlap; beside the read blocks the two kinds overlap.
//
// The sketch is double-buffered per row. A row at tau = W reads its window's
// sketch while its own update writes the next one: the read takes
// sketch[parity[row]], the update writes sketch[1 - parity[row]], and the
// caller flips parity for the row's next window. The update takes the window's
// newest token from the step's inputs (the read block of the same row writes it
// into the buffer in the same launch, with the same bits).
#pragma once

#include "sketch_decode.hpp"
#include "update_body.hpp"

namespace ssm {

namespace {

template <typename TIN, typename TSK>
struct DecodeStepArgs {
  float* state;
  TSK* sketch0;
  TSK* sketch1;
  const float* basis;
  const TIN* q;
  const TIN* k_t;
  const TIN* v_t;
  const float* d_t;
  const float* b_t;
  TIN* kbuf;
  TIN* vbuf;
  float* dbuf;
  float* bbuf;
  float* y;
  const int32_t* slot;         // [batch] or null (identity)
  const int32_t* tau;          // [batch]
  const int32_t* parity;       // [batch]
  const int32_t* update_rows;  // [n_update] batch rows
  int batch, heads, window, rank, num_slots, read_blocks, update_blocks;
};

// Block roles. While both kinds remain, blocks come in groups of 16: 8 read blocks,
// then 8 update blocks, so every XCD (blocks are dealt to the 8 XCDs in turn) gets
// both kinds and each read block keeps the XCD of its head; then the rest of the
// larger kind.
__device__ __forceinline__ bool block_role(int b, int nr, int nu, int& idx) {
  const int m8 = min(nr, nu) & ~7;
  if (b < 2 * m8) {
    idx = (b >> 4) * 8 + (b & 7);
    return (b & 15) < 8;
  }
  const int r = b - 2 * m8;
  const bool read = r < nr - m8;
  idx = m8 + (read ? r : r - (nr - m8));
  return read;
}

template <int RULE, int DK, int DV, typename TIN, typename TSK, int WMAX, bool MMA>
__global__ void __launch_bounds__(256, 4)
decode_step_varlen_kernel(const DecodeStepArgs<TIN, TSK> a) {
  constexpr int DSTR = (RULE == KDA) ? DK : 1;
  int idx = 0;
  const UniformRank rt{a.rank, a.heads};
  if (block_role(blockIdx.x, a.read_blocks, a.update_blocks, idx)) {
    sketch_read_block<RULE, DK, DV, TIN, TSK, WMAX, false, UniformRank, Varlen>(
        idx, a.sketch0, a.basis, a.q, a.k_t, a.v_t, a.d_t, a.b_t, a.kbuf, a.vbuf, a.dbuf, a.bbuf,
        a.y, a.batch, a.heads, a.window, rt, Varlen{a.slot, a.tau, a.num_slots, 1, a.window},
        a.sketch1, a.parity);
    return;
  }
  if (threadIdx.x >= TileLayout<DK, DV>::NT) return;  // an update's threads (whole waves)
  // update block idx runs on XCD idx % 8 (see block_role): give each XCD a contiguous run
  // of update units, as the window update's own launch does (a bijection on [0, nu))
  const int nu = a.update_blocks, x = idx & 7, q8 = nu >> 3, rem = nu & 7;
  const int uidx = x * q8 + min(x, rem) + (idx >> 3);
  const int head = uidx % a.heads;
  const int r = a.update_rows[uidx / a.heads];
  if (r < 0 || r >= a.batch) return;
  const int s = a.slot ? a.slot[r] : r;
  if (s < 0 || s >= a.num_slots || a.tau[r] != a.window) return;  // not a full window
  const size_t u = (size_t)r * a.heads + head;  // per-step arrays are indexed by batch row
  CurrentToken<TIN> cur;
  cur.k = a.k_t + u * DK;
  cur.v = a.v_t + u * DV;
  cur.d = a.d_t + u * DSTR;
  cur.b = (RULE == MAMBA2) ? nullptr : a.b_t + u;
  TSK* next = a.parity[r] != 0 ? a.sketch0 : a.sketch1;  // the buffer the next window reads
  update_refresh_unit<RULE, DK, DV, TIN, TSK, false, UniformRank, MMA>(
      a.state, next, nullptr, a.basis, a.kbuf, a.vbuf, a.dbuf, a.bbuf, a.heads, a.window, rt,
      head, s, a.window, cur);
}

}  // namespace

template <int RULE>
hipError_t launch_decode_step_rule(const ssm_dims& d, int num_slots, const int32_t* slot,
                                   const int32_t* tau, const int32_t* parity, int n_update,
                                   const int32_t* update_rows, float* state, void* sketch0,
                                   void* sketch1, const float* basis, const void* q,
                                   const void* k_t, const void* v_t, const float* decay_t,
                                   const float* beta_t, void* k_buf, void* v_buf,
                                   float* decay_buf, float* beta_buf, float* y,
                                   hipStream_t stream) {
  const size_t upd_lds = update_refresh_lds_bytes(d, d.window, d.rank, false);
  return dispatch_shape(d.in_dtype, d.d_k, d.d_v, [&](auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    constexpr unsigned UPB = 256u / sketch_group<kDK, kDV>();
    const int read_blocks = d.heads * (int)((d.batch + UPB - 1) / UPB);
    const int update_blocks = n_update * d.heads;
    const size_t rd_lds = (size_t)d.rank * kDK * sizeof(float);
    const size_t lds = upd_lds > rd_lds ? upd_lds : rd_lds;
    return with_sketch_type(d, [&](auto SK) {
      using TSK = typename decltype(SK)::type;
      const DecodeStepArgs<TIN, TSK> a{
          state, static_cast<TSK*>(sketch0), static_cast<TSK*>(sketch1), basis,
          static_cast<const TIN*>(q), static_cast<const TIN*>(k_t), static_cast<const TIN*>(v_t),
          decay_t, beta_t, static_cast<TIN*>(k_buf), static_cast<TIN*>(v_buf), decay_buf,
          beta_buf, y, slot, tau, parity, update_rows, d.batch, d.heads, d.window, d.rank,
          num_slots, read_blocks, update_blocks};
      auto launch = [&](auto wmax, auto mma) {
        constexpr int kW = decltype(wmax)::value;
        hipLaunchKernelGGL(
            (decode_step_varlen_kernel<RULE, kDK, kDV, TIN, TSK, kW, decltype(mma)::value>),
            dim3(read_blocks + update_blocks), dim3(256), lds, stream, a);
        return hipGetLastError();
      };
      // the refresh on the matrix cores from rank 8 (d_k >= 64, d_v >= 32), as in the
      // variable-length update: a step's update blocks fit in one round of workgroups, so
      // their arithmetic is not hidden behind other workgroups' streams
      auto go = [&](auto wmax) {
        if constexpr (kDK >= 64 && kDV >= 32) {
          if (d.rank >= 8) return launch(wmax, std::true_type{});
        }
        return launch(wmax, std::false_type{});
      };
      if (d.window <= 4) return go(std::integral_constant<int, 4>{});
      if (d.window <= 8) return go(std::integral_constant<int, 8>{});
      return go(std::integral_constant<int, 16>{});
    });
  });
}

}  // namespace ssm
