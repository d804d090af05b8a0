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
// sketch read: G consecutive lanes per unit (G = 32, or 16 when d_k = 16).
// A workgroup serves 256/G sequences of ONE head, so the head's basis is
// staged once in LDS for all of them. Every global load of the step (query,
// the tau buffered tokens, the first eight sketch rows, the basis) is issued
// before any arithmetic: a step pays one memory latency instead of one per
// token and one per basis vector. WMAX >= W bounds the unrolled token slots.
// Scalar gates stay one per lane (lane i of a unit holds token i's) and are
// broadcast when the walk reaches that token.
// ---------------------------------------------------------------------------
template <int DK>
constexpr int sketch_group() { return DK >= 32 ? 32 : 16; }

// MAP: `basis` is a per-unit read map [N][H][r][d_k] (least-squares coefficients,
// row m giving c_m = row . q~), read from memory like the sketch rows, instead of
// the head's basis in LDS.
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
  constexpr int G = sketch_group<DK>();
  static_assert(WMAX <= G, "one gate per lane");
  constexpr int UPB = 256 / G;                // sequences per workgroup
  constexpr int EK = DK / G, EV = DV / G;
  constexpr int RCH = 8;                      // sketch rows fetched ahead of the walk

  extern __shared__ float4 lds4[];
  float* lB = reinterpret_cast<float*>(lds4);  // [rank][DK]

  const int head = blockIdx.x % heads;
  const int rank = rt.rank(head);
  const int row = (blockIdx.x / heads) * UPB + threadIdx.x / G;  // batch row
  const int sub = threadIdx.x % G;
  int seq = 0, tau = 0;                       // the row's persistent slot and window position
  const bool active = row < batch && rm.row(row, seq, tau);  // whole G-lane groups
  const size_t unit = (size_t)row * heads + head;            // per-step arrays
  const size_t punit = (size_t)seq * heads + head;           // state, sketch, buffer
  const size_t slot0 = punit * window;
  const bool fused = (k_t != nullptr);

  // ---- issue every load ----
  Packed<TIN, EK> qr, kr[WMAX];
  Packed<TIN, EV> vr[WMAX];
  float ak[(RULE == KDA) ? WMAX : 1][EK];     // KDA: per-channel gates of each token
  float a_lane = 1.f, b_lane = 1.f;           // scalar gates of token `sub`
  float sk[RCH][EV];
  float ym[MAP ? RCH : 1][EK];                // MAP: the first read-map rows
  const float* Yu = basis + (MAP ? punit * (size_t)rank * DK + sub * EK : 0);
  const TSK* Sku = sketch + ((size_t)seq * rt.total() + rt.offset(head)) * DV + sub * EV;
  if (active) {
    qr.load(q + unit * DK + sub * EK);
#pragma unroll
    for (int i = 0; i < WMAX; ++i) {
      if (i < tau) {
        const bool cur = fused && (i == tau - 1);
        const size_t slot = slot0 + i;
        kr[i].load((cur ? k_t + unit * DK : kbuf + slot * DK) + sub * EK);
        vr[i].load((cur ? v_t + unit * DV : vbuf + slot * DV) + sub * EV);
        if constexpr (RULE == KDA)
          Vec<float, EK>::load((cur ? d_t + unit * DK : dbuf + slot * DK) + sub * EK, ak[i]);
      }
    }
    if (sub < tau) {
      const bool cur = fused && (sub == tau - 1);
      if constexpr (RULE != KDA) a_lane = cur ? d_t[unit] : dbuf[slot0 + sub];
      if constexpr (RULE != MAMBA2) b_lane = cur ? b_t[unit] : bbuf[slot0 + sub];
    }
#pragma unroll
    for (int m = 0; m < RCH; ++m)
      if (m < rank) Vec<TSK, EV>::load(Sku + (size_t)m * DV, sk[m]);
    if constexpr (MAP) {
#pragma unroll
      for (int m = 0; m < RCH; ++m)
        if (m < rank) Vec<float, EK>::load(Yu + (size_t)m * DK, ym[m]);
    }
  }
  if constexpr (!MAP) {
    const float* Bh = basis + (size_t)rt.offset(head) * DK;
    for (int e = threadIdx.x * 4; e < rank * DK; e += 256 * 4)
      *reinterpret_cast<float4*>(lB + e) = *reinterpret_cast<const float4*>(Bh + e);
  }

  float u[EK], acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;
  if (active) {
    // ---- fused append: the current token into slot tau-1 ----
    if (fused) {
      const size_t slot = slot0 + tau - 1;
#pragma unroll
      for (int i = 0; i < WMAX; ++i) {
        if (i == tau - 1) {
          kr[i].store(kbuf + slot * DK + sub * EK);
          vr[i].store(vbuf + slot * DV + sub * EV);
          if constexpr (RULE == KDA) Vec<float, EK>::store(dbuf + slot * DK + sub * EK, ak[i]);
        }
      }
      if (sub == tau - 1) {
        if constexpr (RULE != KDA) dbuf[slot] = a_lane;
        if constexpr (RULE != MAMBA2) bbuf[slot] = b_lane;
      }
    }

    // ---- walk the window newest to oldest ----
    qr.unpack(u);
#pragma unroll
    for (int i = WMAX - 1; i >= 0; --i) {
      if (i < tau) {
        float kk[EK], vv[EV], a[(RULE == KDA) ? EK : 1];
        kr[i].unpack(kk);
        vr[i].unpack(vv);
        if constexpr (RULE == KDA) {
#pragma unroll
          for (int e = 0; e < EK; ++e) a[e] = ak[i][e];
        } else {
          a[0] = __shfl(a_lane, i, G);
        }
        const float b = (RULE == MAMBA2) ? 1.f : __shfl(b_lane, i, G);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) s = fmaf(kk[e], u[e], s);
        s = group_allreduce<G>(s);
        const float bs = b * s;
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[e] = fmaf(bs, vv[e], acc[e]);
        carry_back<RULE, EK>(u, kk, a, bs);
      }
    }
  }
  if constexpr (!MAP) __syncthreads();  // the basis is in LDS
  if (!active) return;

  // ---- c_m = b_m . q~ ; y = intra + sum_m c_m Sk[m] ----
  for (int m0 = 0; m0 < rank; m0 += RCH) {
    if (m0 > 0) {
#pragma unroll
      for (int m = 0; m < RCH; ++m) {
        if (m0 + m < rank) {
          Vec<TSK, EV>::load(Sku + (size_t)(m0 + m) * DV, sk[m]);
          if constexpr (MAP) Vec<float, EK>::load(Yu + (size_t)(m0 + m) * DK, ym[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < RCH; ++m) {
      if (m0 + m < rank) {
        float bm[EK];
        if constexpr (MAP) {
#pragma unroll
          for (int e = 0; e < EK; ++e) bm[e] = ym[m][e];
        } else {
          Vec<float, EK>::load(lB + (m0 + m) * DK + sub * EK, bm);
        }
        float c = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) c = fmaf(bm[e], u[e], c);
        c = group_allreduce<G>(c);
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[e] = fmaf(c, sk[m][e], acc[e]);
      }
    }
  }
  Vec<float, EV>::store(y + unit * DV + sub * EV, acc);
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
    constexpr unsigned UPB = 256u / sketch_group<kDK>();
    const unsigned blocks = (unsigned)d.heads * (((unsigned)d.batch + UPB - 1) / UPB);
    const size_t lds = (size_t)max_rank * kDK * sizeof(float);
    if (per_unit_map) {  // least squares: fp32 sketch, uniform rank, lockstep (checked)
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
