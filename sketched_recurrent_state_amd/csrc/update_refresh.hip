// update_refresh.hip -- the once-per-window state write fused with the sketch
// refresh (SketchSSM pages: readsearch.ai listing of arXiv 2609.33051,
// Abstract, one full-state read per update stores the basis outputs;
// agihunt.info summary, "Error control", the full state is updated once per
// window and the sketch is refreshed in the same kernel).
//
// One workgroup per (sequence, head) unit, d_v/32 independent waves. Every
// rule acts on the d_k side of S only (decay, projection and the rank-1 write
// k w^T), so each column of S evolves on its own: the waves split d_v and never
// synchronise after the initial staging barrier. Each lane keeps its 4 x d_k/8
// piece of S in VGPRs for the whole window: S is read from HBM once and
// written once. The window's keys, values and gates (and the head's basis) are
// staged in LDS as fp32 so every wave reads them without touching HBM again.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

template <int RULE, int DK>
struct Layout {
  static constexpr int DSTR = (RULE == KDA) ? DK : 1;  // gate floats per token
};

__host__ __device__ inline int pad4(int x) { return (x + 3) & ~3; }

template <int RULE, int DK, int DV, typename TIN>
__global__ void __launch_bounds__(2 * DV)
update_refresh_kernel(float* __restrict__ state, float* __restrict__ sketch,
                      const float* __restrict__ basis, const TIN* __restrict__ kbuf,
                      const TIN* __restrict__ vbuf, const float* __restrict__ dbuf,
                      const float* __restrict__ bbuf, int heads, int window, int rank, int n) {
  constexpr int RPL = DK / 8;          // rows of S per lane
  constexpr int NT = 2 * DV;           // threads per unit: d_v/32 waves
  constexpr int DSTR = Layout<RULE, DK>::DSTR;
  constexpr int VIN = 16 / sizeof(TIN);  // input elements per 16-byte load

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);

  const int unit = blockIdx.x;
  const int head = unit % heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane & 7, rg = lane >> 3;
  const int col = wave * 32 + cg * 4;
  const int row0 = rg * RPL;

  // 1. issue the loads of this lane's state piece (the only HBM read of S)
  float* Su = state + (size_t)unit * (DK * DV);
  float4 s[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
    s[m] = *reinterpret_cast<const float4*>(Su + (size_t)(row0 + m) * DV + col);

  // 2. stage the window (and the basis) in LDS as fp32
  float* lk = lds;                          // [n][DK]
  float* lv = lk + n * DK;                  // [n][DV]
  float* ld = lv + n * DV;                  // [n][DSTR]
  float* lb = ld + pad4(n * DSTR);          // [n]      (delta rules)
  float* lB = lb + ((RULE == MAMBA2) ? 0 : pad4(n));  // [rank][DK]
  const size_t slot0 = (size_t)unit * window;
  {
    const TIN* ku = kbuf + slot0 * DK;
    for (int e = tid * VIN; e < n * DK; e += NT * VIN) {
      float x[VIN];
      Vec<TIN, VIN>::load(ku + e, x);
      Vec<float, VIN>::store(lk + e, x);
    }
    const TIN* vu = vbuf + slot0 * DV;
    for (int e = tid * VIN; e < n * DV; e += NT * VIN) {
      float x[VIN];
      Vec<TIN, VIN>::load(vu + e, x);
      Vec<float, VIN>::store(lv + e, x);
    }
    const float* du = dbuf + slot0 * DSTR;
    for (int e = tid; e < n * DSTR; e += NT) ld[e] = du[e];
    if constexpr (RULE != MAMBA2) {
      for (int e = tid; e < n; e += NT) lb[e] = bbuf[slot0 + e];
    }
    if (sketch != nullptr) {
      const float* Bh = basis + (size_t)head * rank * DK;
      for (int e = tid * 4; e < rank * DK; e += NT * 4)
        *reinterpret_cast<float4*>(lB + e) = *reinterpret_cast<const float4*>(Bh + e);
    }
  }
  __syncthreads();

  // 3. the window's tokens, in order: S <- M_t S + b_t k_t v_t^T on the
  //    register-resident piece; the k^T S reduction over d_k crosses the 8
  //    lanes that share this lane's columns.
  for (int t = 0; t < n; ++t) {
    float kr[RPL];
    Vec<float, RPL>::load(lk + t * DK + row0, kr);
    const float4 vv = *reinterpret_cast<const float4*>(lv + t * DV + col);
    if constexpr (RULE == MAMBA2) {
      const float a = ld[t];
#pragma unroll
      for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], vv, scale4(a, s[m]));
    } else if constexpr (RULE == GDN) {
      const float a = ld[t], b = lb[t];
      float4 p = f4(0.f);
#pragma unroll
      for (int m = 0; m < RPL; ++m) p = fma4(kr[m], s[m], p);
      p = tile_allreduce(p);  // p = S^T k for this lane's 4 columns
      const float4 w = scale4(b, sub4(vv, scale4(a, p)));
#pragma unroll
      for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, scale4(a, s[m]));
    } else {
      const float b = lb[t];
      float ar[RPL];
      Vec<float, RPL>::load(ld + t * DK + row0, ar);
      float4 p = f4(0.f);
#pragma unroll
      for (int m = 0; m < RPL; ++m) {
        s[m] = scale4(ar[m], s[m]);  // Diag(alpha) S
        p = fma4(kr[m], s[m], p);
      }
      p = tile_allreduce(p);
      const float4 w = scale4(b, sub4(vv, p));
#pragma unroll
      for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, s[m]);
    }
  }

  // 4. write the state back (the only HBM write of S)
  if (n > 0) {
#pragma unroll
    for (int m = 0; m < RPL; ++m)
      *reinterpret_cast<float4*>(Su + (size_t)(row0 + m) * DV + col) = s[m];
  }

  // 5. sketch refresh from the register-resident state: Sk[m] = S^T b_m.
  //    Eight basis rows at a time; the d_k reduction is a reduce-scatter over
  //    the 8 row groups, after which lane group rg holds basis row m0 + rg.
  if (sketch != nullptr) {
    float* Sku = sketch + (size_t)unit * rank * DV;
    const bool b3 = (lane >> 3) & 1;
    for (int m0 = 0; m0 < rank; m0 += 8) {
      float4 P[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        P[e] = f4(0.f);
        if (m0 + e < rank) {
          float bm[RPL];
          Vec<float, RPL>::load(lB + (m0 + e) * DK + row0, bm);
#pragma unroll
          for (int m = 0; m < RPL; ++m) P[e] = fma4(bm[m], s[m], P[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // lane bit 5: keep rows e (low half) / e + 4 (high half)
        halve32(P[e].x, P[e + 4].x);
        halve32(P[e].y, P[e + 4].y);
        halve32(P[e].z, P[e + 4].z);
        halve32(P[e].w, P[e + 4].w);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {  // lane bit 4
        halve16(P[e].x, P[e + 2].x);
        halve16(P[e].y, P[e + 2].y);
        halve16(P[e].z, P[e + 2].z);
        halve16(P[e].w, P[e + 2].w);
      }
      float4 res;  // lane bit 3
      res.x = halve8(P[0].x, P[1].x, b3);
      res.y = halve8(P[0].y, P[1].y, b3);
      res.z = halve8(P[0].z, P[1].z, b3);
      res.w = halve8(P[0].w, P[1].w, b3);
      const int m = m0 + rg;
      if (m < rank) *reinterpret_cast<float4*>(Sku + (size_t)m * DV + col) = res;
    }
  }
}

}  // namespace

size_t update_refresh_lds_bytes(const ssm_dims& d, int n, bool refresh) {
  const int dstr = (d.rule == SSM_KDA) ? d.d_k : 1;
  size_t floats = (size_t)n * d.d_k + (size_t)n * d.d_v + pad4(n * dstr) +
                  ((d.rule == SSM_MAMBA2) ? 0 : pad4(n)) + (refresh ? (size_t)d.rank * d.d_k : 0);
  return floats * sizeof(float);
}

hipError_t launch_update_refresh(const ssm_dims& d, float* state, float* sketch,
                                 const float* basis, const void* k_buf, const void* v_buf,
                                 const float* decay_buf, const float* beta_buf, int n,
                                 hipStream_t stream) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  const size_t lds = update_refresh_lds_bytes(d, n, sketch != nullptr);
  return dispatch(d.rule, d.in_dtype, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = decltype(R)::value, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    hipLaunchKernelGGL((update_refresh_kernel<kR, kDK, kDV, TIN>), dim3(units), dim3(2 * kDV),
                       lds, stream, state, sketch, basis, static_cast<const TIN*>(k_buf),
                       static_cast<const TIN*>(v_buf), decay_buf, beta_buf, d.heads, d.window,
                       d.rank, n);
    return hipGetLastError();
  });
}

}  // namespace ssm
