// sketch_decode.hpp -- the sketch read, every decode step of SketchSSM:
//   c = B q~,  y = Sk^T c + intra   (readsearch.ai listing of arXiv 2609.33051,
//   Abstract: each step combines the stored basis outputs with query-dependent
//   coefficients), after the buffer walk of read_walk.hpp.
// The launcher is instantiated once per rule, each in its own translation unit
// (sketch_decode_<rule>.hip), so the instantiations compile in parallel.
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "read_walk.hpp"

namespace ssm {

namespace {

// ---------------------------------------------------------------------------
// sketch read: G consecutive lanes per unit (G = 32, or 16 when d_k or d_v is 16).
// A workgroup serves 256/G sequences of ONE head, so the head's basis is
// staged once in LDS for all of them.
//
// Issue order. Every global load of the step is issued before any arithmetic,
// in the order the step consumes them: the head's basis (its first chunk goes
// to LDS right away), the scalar gates, the query, the buffered tokens newest
// first (slot j holds token tau-1-j: the walk starts at slot 0), then the first
// eight sketch rows.
// The number of loads does not depend on tau or the rank: a slot past tau, or a
// sketch row past the rank, loads a clamped address (token 0, row rank-1) and its
// result is discarded with a select, never with a branch. With a fixed count,
// each use waits only for its own load (the memory counter is in order), so the
// walk runs while the older tokens and the sketch rows are still arriving; and
// no load sits in a conditional block that the compiler could sink it into.
// A group whose batch row is inactive loads row 0 / slot 0 and stores nothing.
// WMAX >= W bounds the token slots. Scalar gates stay one per lane (lane j of a
// unit holds slot j's) and are broadcast when the walk reaches that slot.
// ---------------------------------------------------------------------------
template <int DK, int DV>
constexpr int sketch_group() { return (DK >= 32 && DV >= 32) ? 32 : 16; }

// MAP: `basis` is a per-unit read map [N][H][r][d_k] (least-squares coefficients,
// row m giving c_m = row . q~), read from memory like the sketch rows, instead of
// the head's basis in LDS.
//
// Block `blk` of a read launch: heads * ceil(batch / (256 / G)) blocks of 256 threads.
// sketch_alt / parity (both null, or both set): a double-buffered sketch, the row's
// current one being sketch_alt where parity[row] is non-zero, else sketch.
template <int RULE, int DK, int DV, typename TIN, typename TSK, int WMAX, bool MAP, typename RT,
          typename RM>
__device__ __forceinline__ void sketch_read_block(
    int blk, const TSK* __restrict__ sketch, const float* __restrict__ basis,
    const TIN* __restrict__ q, const TIN* __restrict__ k_t, const TIN* __restrict__ v_t,
    const float* __restrict__ d_t, const float* __restrict__ b_t, TIN* kbuf, TIN* vbuf,
    float* dbuf, float* bbuf, float* __restrict__ y, int batch, int heads, int window,
    const RT& rt, const RM& rm, const TSK* __restrict__ sketch_alt,
    const int32_t* __restrict__ parity) {
  constexpr int G = sketch_group<DK, DV>();
  static_assert(WMAX <= G, "one gate per lane");
  constexpr int UPB = 256 / G;                // sequences per workgroup
  constexpr int EK = DK / G, EV = DV / G;
  constexpr int RCH = 8;                      // sketch rows fetched ahead of the walk

  extern __shared__ float4 lds4[];
  float* lB = reinterpret_cast<float*>(lds4);  // [rank][DK]

  // Blocks are dealt to the 8 XCDs in turn. With one rank for all heads, block blk
  // serves head blk % heads, so each head stays on one XCD (its basis in one L2).
  // With per-head ranks the heads move different byte counts, and a rank pattern
  // that repeats with a period dividing 8 would load some XCDs far more than
  // others (ranks 2, 4, 8, 18 cycled over 32 heads put every rank-18 head on two
  // XCDs); there consecutive blocks take one head's consecutive row blocks, so
  // every head is spread over all XCDs, and the heads come largest rank first
  // (rt.order): the blocks resident together in one round then share a rank, and
  // each compute unit takes one block of each round. In head order, ranks 2, 4, 8,
  // 18 cycled over 32 heads gave every unit four blocks of one rank, and the units
  // holding rank 18 set the launch's time (14.9 against 13.2 us at N = 256).
  constexpr bool kSpread = std::is_same<RT, RankTable>::value;
  const int nrb = (batch + UPB - 1) / UPB;    // row blocks per head
  int head = blk % heads;
  if constexpr (kSpread) head = rt.order[blk / nrb];
  const int rblk = kSpread ? blk % nrb : blk / heads;
  const int rank = rt.rank(head);
  const int row = rblk * UPB + threadIdx.x / G;  // batch row
  const int sub = threadIdx.x % G;
  const int tid = threadIdx.x;
  int seq = 0, tau = 0;                       // the row's persistent slot and window position
  const bool active = row < batch && rm.row(row, seq, tau);  // whole G-lane groups
  // an inactive group reads row 0 / slot 0 (valid memory) and writes nothing
  const int ntok = active ? tau : 1;
  const size_t unit = (size_t)(active ? row : 0) * heads + head;    // per-step arrays
  const int aseq = active ? seq : 0;
  const size_t punit = (size_t)aseq * heads + head;   // state, sketch, buffer
  const size_t slot0 = punit * window;
  const bool fused = (k_t != nullptr);

  // ---- issue every load, in the order they are consumed ----
  const float* Bh = basis + (size_t)rt.offset(head) * DK;
  float4 b4 = f4(0.f);
  if constexpr (!MAP) b4 = *reinterpret_cast<const float4*>(Bh + min(tid * 4, rank * DK - 4));
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order (the scheduler regroups loads)
  Packed<TIN, EK> qr, kr[WMAX];
  Packed<TIN, EV> vr[WMAX];
  float ak[(RULE == KDA) ? WMAX : 1][EK];     // KDA: per-channel gates of each slot
  float a_lane = 1.f, b_lane = 1.f;           // scalar gates of slot `sub`
  float sk[RCH][EV];
  float ym[MAP ? RCH : 1][EK];                // MAP: the first read-map rows
  const float* Yu = basis + (MAP ? punit * (size_t)rank * DK + sub * EK : 0);
  const TSK* skb = (parity != nullptr && active && parity[row] != 0) ? sketch_alt : sketch;
  const TSK* Sku = skb + ((size_t)aseq * rt.total() + rt.offset(head)) * DV + sub * EV;
  {
    const int js = min(sub, WMAX - 1);
    const size_t slot = slot0 + max(ntok - 1 - js, 0);
    const bool cur = fused && js == 0;
    if constexpr (RULE != KDA) a_lane = cur ? d_t[unit] : dbuf[slot];
    if constexpr (RULE != MAMBA2) b_lane = cur ? b_t[unit] : bbuf[slot];
  }
  __builtin_amdgcn_sched_barrier(0);
  qr.load(q + unit * DK + sub * EK);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < WMAX; ++j) {
    const size_t slot = slot0 + max(ntok - 1 - j, 0);
    const bool cur = fused && j == 0;         // slot 0 is the current token
    kr[j].load((cur ? k_t + unit * DK : kbuf + slot * DK) + sub * EK);
    vr[j].load((cur ? v_t + unit * DV : vbuf + slot * DV) + sub * EV);
    if constexpr (RULE == KDA)
      Vec<float, EK>::load((cur ? d_t + unit * DK : dbuf + slot * DK) + sub * EK, ak[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = 0; m < RCH; ++m) Vec<TSK, EV>::load(Sku + (size_t)min(m, rank - 1) * DV, sk[m]);
  if constexpr (MAP) {
#pragma unroll
    for (int m = 0; m < RCH; ++m) Vec<float, EK>::load(Yu + (size_t)min(m, rank - 1) * DK, ym[m]);
  }
  // the basis chunk to LDS (its load was the first issued; duplicate clamped chunks write
  // the same values)
  if constexpr (!MAP) *reinterpret_cast<float4*>(lB + min(tid * 4, rank * DK - 4)) = b4;

  // ---- fused append: the current token (slot 0) into buffer slot tau-1 ----
  if (active && fused) {
    const size_t slot = slot0 + tau - 1;
    kr[0].store(kbuf + slot * DK + sub * EK);
    vr[0].store(vbuf + slot * DV + sub * EV);
    if constexpr (RULE == KDA) Vec<float, EK>::store(dbuf + slot * DK + sub * EK, ak[0]);
    if (sub == 0) {
      if constexpr (RULE != KDA) dbuf[slot] = a_lane;
      if constexpr (RULE != MAMBA2) bbuf[slot] = b_lane;
    }
  }

  // ---- walk the window newest to oldest; slots past tau leave u and intra as they are ----
  float u[EK], acc[EV];
  qr.unpack(u);
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j = 0; j < WMAX; ++j) {
    float kk[EK], vv[EV], a[(RULE == KDA) ? EK : 1];
    kr[j].unpack(kk);
    vr[j].unpack(vv);
    if constexpr (RULE == KDA) {
#pragma unroll
      for (int e = 0; e < EK; ++e) a[e] = ak[j][e];
    } else {
      a[0] = group_bcast<G>(a_lane, j);
    }
    const float b = (RULE == MAMBA2) ? 1.f : group_bcast<G>(b_lane, j);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) s = fmaf(kk[e], u[e], s);
    s = group_allreduce<G>(s);
    const float bs = b * s;
    const bool live = j < ntok;
    float un[EK];
#pragma unroll
    for (int e = 0; e < EK; ++e) un[e] = u[e];
    carry_back<RULE, EK>(un, kk, a, bs);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = live ? fmaf(bs, vv[e], acc[e]) : acc[e];
#pragma unroll
    for (int e = 0; e < EK; ++e) u[e] = live ? un[e] : u[e];
  }
  if constexpr (!MAP) {
    // basis chunks past the first (rank * d_k > 4 * 256), then every wave's chunk is in LDS
    for (int e = (tid + 256) * 4; e < rank * DK; e += 256 * 4)
      *reinterpret_cast<float4*>(lB + e) = *reinterpret_cast<const float4*>(Bh + e);
    __syncthreads();
  }

  // ---- c_m = b_m . q~ ; y = intra + sum_m c_m Sk[m] ----
  // the first RCH rows (issued with the step's loads); rows past the rank are discarded
#pragma unroll
  for (int m = 0; m < RCH; ++m) {
    float bm[EK];
    if constexpr (MAP) {
#pragma unroll
      for (int e = 0; e < EK; ++e) bm[e] = ym[m][e];
    } else {
      Vec<float, EK>::load(lB + min(m, rank - 1) * DK + sub * EK, bm);
    }
    float c = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) c = fmaf(bm[e], u[e], c);
    c = group_allreduce<G>(c);
    const bool live = m < rank;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] = live ? fmaf(c, sk[m][e], acc[e]) : acc[e];
  }
  // further rows, RCH at a time, one more memory round trip each
  for (int m0 = RCH; m0 < rank; m0 += RCH) {
#pragma unroll
    for (int m = 0; m < RCH; ++m) {
      Vec<TSK, EV>::load(Sku + (size_t)min(m0 + m, rank - 1) * DV, sk[m]);
      if constexpr (MAP) Vec<float, EK>::load(Yu + (size_t)min(m0 + m, rank - 1) * DK, ym[m]);
    }
#pragma unroll
    for (int m = 0; m < RCH; ++m) {
      float bm[EK];
      if constexpr (MAP) {
#pragma unroll
        for (int e = 0; e < EK; ++e) bm[e] = ym[m][e];
      } else {
        Vec<float, EK>::load(lB + min(m0 + m, rank - 1) * DK + sub * EK, bm);
      }
      float c = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e) c = fmaf(bm[e], u[e], c);
      c = group_allreduce<G>(c);
      const bool live = m0 + m < rank;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[e] = live ? fmaf(c, sk[m][e], acc[e]) : acc[e];
    }
  }
  if (active) Vec<float, EV>::store(y + unit * DV + sub * EV, acc);
}

template <int RULE, int DK, int DV, typename TIN, typename TSK, int WMAX, bool MAP, typename RT,
          typename RM>
__global__ void __launch_bounds__(256)
sketch_decode_kernel(const TSK* __restrict__ sketch, const float* __restrict__ basis,
                     const TIN* __restrict__ q, const TIN* __restrict__ k_t,
                     const TIN* __restrict__ v_t, const float* __restrict__ d_t,
                     const float* __restrict__ b_t, TIN* __restrict__ kbuf,
                     TIN* __restrict__ vbuf, float* __restrict__ dbuf, float* __restrict__ bbuf,
                     float* __restrict__ y, int batch, int heads, int window, const RT rt,
                     const RM rm) {
  sketch_read_block<RULE, DK, DV, TIN, TSK, WMAX, MAP, RT, RM>(
      blockIdx.x, sketch, basis, q, k_t, v_t, d_t, b_t, kbuf, vbuf, dbuf, bbuf, y, batch, heads,
      window, rt, rm, nullptr, nullptr);
}

}  // namespace

template <int RULE>
hipError_t launch_sketch_decode_rule(const ssm_dims& d, const int32_t* rank_offsets,
                                const void* sketch, const float* basis, const void* q,
                                const void* k_t, const void* v_t, const float* decay_t,
                                const float* beta_t, void* k_buf, void* v_buf, float* decay_buf,
                                float* beta_buf, int tau, float* y, hipStream_t stream,
                                const Varlen* varlen, bool per_unit_map) {
  const int max_rank = rank_offsets ? max_rank_of(rank_offsets, d.heads) : d.rank;
  return dispatch_shape(d.in_dtype, d.d_k, d.d_v, [&](auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = RULE, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    constexpr unsigned UPB = 256u / sketch_group<kDK, kDV>();
    const unsigned blocks = (unsigned)d.heads * (((unsigned)d.batch + UPB - 1) / UPB);
    const size_t lds = (size_t)max_rank * kDK * sizeof(float);
    if (per_unit_map) {  // least squares: fp32 sketch, uniform rank, lockstep
      auto go_map = [&](auto wmax) {
        constexpr int kW = decltype(wmax)::value;
        hipLaunchKernelGGL(
            (sketch_decode_kernel<kR, kDK, kDV, TIN, float, kW, true, UniformRank, Lockstep>),
            dim3(blocks), dim3(256), 0, stream, static_cast<const float*>(sketch), basis,
            static_cast<const TIN*>(q), static_cast<const TIN*>(k_t),
            static_cast<const TIN*>(v_t), decay_t, beta_t, static_cast<TIN*>(k_buf),
            static_cast<TIN*>(v_buf), decay_buf, beta_buf, y, d.batch, d.heads, d.window,
            UniformRank{d.rank, d.heads}, Lockstep{tau});
        return hipGetLastError();
      };
      if (d.window <= 4) return go_map(std::integral_constant<int, 4>{});
      if (d.window <= 8) return go_map(std::integral_constant<int, 8>{});
      return go_map(std::integral_constant<int, 16>{});
    }
    return with_sketch_type(d, [&](auto SK) {
      using TSK = typename decltype(SK)::type;
      auto go = [&](auto wmax, auto rt, auto rm) {
        constexpr int kW = decltype(wmax)::value;
        hipLaunchKernelGGL(
            (sketch_decode_kernel<kR, kDK, kDV, TIN, TSK, kW, false, decltype(rt), decltype(rm)>),
            dim3(blocks), dim3(256), lds, stream, static_cast<const TSK*>(sketch), basis,
            static_cast<const TIN*>(q), static_cast<const TIN*>(k_t),
            static_cast<const TIN*>(v_t), decay_t, beta_t, static_cast<TIN*>(k_buf),
            static_cast<TIN*>(v_buf), decay_buf, beta_buf, y, d.batch, d.heads, d.window, rt,
            rm);
        return hipGetLastError();
      };
      auto with_rank = [&](auto wmax) {
        if (varlen != nullptr) return go(wmax, UniformRank{d.rank, d.heads}, *varlen);
        if (rank_offsets == nullptr)
          return go(wmax, UniformRank{d.rank, d.heads}, Lockstep{tau});
        return go(wmax, make_rank_table(rank_offsets, d.heads), Lockstep{tau});
      };
      if (d.window <= 4) return with_rank(std::integral_constant<int, 4>{});
      if (d.window <= 8) return with_rank(std::integral_constant<int, 8>{});
      return with_rank(std::integral_constant<int, 16>{});
    });
  });
}

}  // namespace ssm
