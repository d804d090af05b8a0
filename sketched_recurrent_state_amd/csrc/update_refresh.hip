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
//
// Memory order: lane group rg owns the interleaved rows rg, rg + 8, ... so each
// load instruction of the workgroup covers 8 whole rows of S (contiguous), and
// consecutive units go to the same XCD (workgroups are dealt to the 8 XCDs in
// turn; the block index is remapped so each XCD streams one contiguous run of
// units). Together these move S about 5% faster than contiguous rows per lane
// with the natural block order.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

// Rank decisions of the least-squares refresh: a sketch row whose part orthogonal
// to the rows before it is below this fraction of the largest row norm adds nothing.
constexpr float kLsRelTol = 1e-5f;

// LS = false: stores Sk = B S (row m = S^T b_m). LS = true (least-squares
// coefficients): stores instead Q, orthonormal rows spanning the rows of Sk, in
// `sketch`, and the read map Y = Q S^T [r][d_k] in `rmap`; a read then gives
// Q^T (Y q~), the projection of S^T q~ on the span of the sketch rows.
template <int RULE, int DK, int DV, typename TIN, typename TSK, bool LS, typename RT, typename RM>
__global__ void __launch_bounds__(2 * DV, 4)
update_refresh_kernel(float* __restrict__ state, TSK* __restrict__ sketch,
                      float* __restrict__ rmap,
                      const float* __restrict__ basis, const TIN* __restrict__ kbuf,
                      const TIN* __restrict__ vbuf, const float* __restrict__ dbuf,
                      const float* __restrict__ bbuf, int heads, int window, const RT rt,
                      const RM rm) {
  constexpr int RPL = DK / 8;          // rows of S per lane
  constexpr int NT = 2 * DV;           // threads per unit: d_v/32 waves
  constexpr int DSTR = (RULE == KDA) ? DK : 1;

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);

  // XCD x = blockIdx.x % 8 receives blocks x, x + 8, ...: give it the contiguous
  // run of units [x * q8 + min(x, rem), ...) instead (a bijection on the grid).
  const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, rem = G & 7;
  const int b = xcd * q8 + min(xcd, rem) + (blockIdx.x >> 3);
  const int head = b % heads;
  int seq = 0, n = 0;  // the batch row's persistent slot and its number of buffered tokens
  if (!rm.row(b / heads, seq, n)) return;  // whole workgroup: a skipped row
  const size_t unit = (size_t)seq * heads + head;
  const int rank = rt.rank(head);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane & 7, rg = lane >> 3;
  const int col = wave * 32 + cg * 4;
  // s[m] holds row m * 8 + rg of S; the LDS copies of keys, gates and basis
  // keep this lane's d_k / 8 values at [row0, row0 + RPL) (interleaved_pos).
  const int row0 = rg * RPL;

  // 1. issue the staging reads: the window's tokens and the head's basis (each
  //    thread's first chunk of every array, one memory round trip in all)
  const size_t slot0 = (size_t)unit * window;
  UnitWindow<TIN> uw{const_cast<TIN*>(kbuf) + slot0 * DK, const_cast<TIN*>(vbuf) + slot0 * DV,
                     const_cast<float*>(dbuf) + slot0 * DSTR,
                     (RULE == MAMBA2) ? nullptr : const_cast<float*>(bbuf) + slot0,
                     nullptr, nullptr, nullptr, nullptr};
  WindowStage<RULE, DK, DV, TIN, NT, true> stage;
  if (n > 0) stage.issue(uw, n, tid);
  const float* Bh = basis + (size_t)rt.offset(head) * DK;
  float4 b4 = f4(0.f);
  if (sketch != nullptr) b4 = *reinterpret_cast<const float4*>(Bh + min(tid * 4, rank * DK - 4));
  // 2. then the loads of this lane's state piece (the only HBM read of S). In
  //    this order the small staging reads are served first; issued behind the
  //    unit's 64 KB stream they would wait for it, and for every other
  //    workgroup's: then all workgroups start computing at once and HBM idles
  //    meanwhile (about 10% of the kernel's time at 128 x 128).
  float* Su = state + (size_t)unit * (DK * DV);
  float4 s[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m)
    s[m] = load_stream(Su + (size_t)(m * 8 + rg) * DV + col);
  // 3. the staged data to LDS as fp32 while the state is in flight
  if (n > 0) stage.commit(lds, uw, n, tid);
  const float* lk = lds;
  const float* lv = lk + n * DK;
  const float* ld = lv + n * DV;
  const float* lb = ld + pad4(n * DSTR);
  float* lB = lds + window_lds_floats<RULE, DK, DV>(n);  // [rank][DK]
  if (sketch != nullptr) {
    auto put = [&](float4 x4, int e) {
      float* row = lB + (e - e % DK);
      const int i0 = e % DK;
      row[interleaved_pos<DK>(i0)] = x4.x;
      row[interleaved_pos<DK>(i0 + 1)] = x4.y;
      row[interleaved_pos<DK>(i0 + 2)] = x4.z;
      row[interleaved_pos<DK>(i0 + 3)] = x4.w;
    };
    if (tid * 4 < rank * DK) put(b4, tid * 4);
    for (int e = (tid + NT) * 4; e < rank * DK; e += NT * 4)
      put(*reinterpret_cast<const float4*>(Bh + e), e);
  }
  __syncthreads();

  // 4. the window's tokens, in order: S <- M_t S + b_t k_t v_t^T on the
  //    register-resident piece; the k^T S reduction over d_k crosses the 8
  //    lanes that share this lane's columns. Mamba-2 and GDN carry a scaled
  //    copy of the piece so the per-token decay costs nothing (below); KDA
  //    decays rows by different gates and updates S directly.
  // 5. write the state back (the only HBM write of S), then
  // 6. refresh the sketch from the register-resident state: Sk[m] = S^T b_m.
  //    Eight basis rows at a time; the d_k reduction is a reduce-scatter over
  //    the 8 row groups, after which lane group rg holds basis row m0 + rg.
  // Least-squares refresh, after the rows of Sk are in LDS (lQ). The rows are made
  // orthonormal as Gram-Schmidt would, through the Cholesky factor of their Gram
  // matrix (Sk = L Q with Q orthonormal rows, L lower triangular, G = Sk Sk^T = L L^T):
  //   a. G in fp64 (products of fp32 values are exact there), four lanes per entry;
  //   b. wave 0 factors G = L L^T column by column, lane i owning row i; a row whose
  //      pivot, its squared residual against the rows before it, is below
  //      kLsRelTol^2 of the largest squared row norm is dropped (zero column of L);
  //   c. step b also forms L^-1 (fp64, in place of L, the inverse pivots on the
  //      diagonal; a dropped row is zero), then Q = L^-1 Sk in place, one column of
  //      the sketch per thread, each row from the exact fp32 sketch;
  //   d. every wave forms Y = Q S^T over its 32 columns: per row of S a dot product
  //      of 4 columns, summed over the 8 lanes of the row group (lane bits 0..2) as a
  //      reduce-scatter over four rows of Q at a time;
  //   e. the waves' partial Y are added in a fixed order and stored with Q.
  float* lQ = lB + rank * DK;  // [rank][DV] (LS only)
  float* lP = lQ + rank * DV;  // [DV / 32][rank][DK] per-wave partial Y (LS only)
  double* lG = reinterpret_cast<double*>(lP + (DV / 32) * rank * DK);  // [rank][rank] (LS only)
  auto ls_epilogue = [&](float* Qu) {
    __syncthreads();
    for (int e0 = 0; e0 < rank * rank; e0 += NT / 4) {  // a. Gram matrix, lower triangle
      const int e = e0 + tid / 4, part = tid & 3;
      double g = 0.0;
      if (e < rank * rank) {
        const float* ri = lQ + (e / rank) * DV;
        const float* rj = lQ + (e % rank) * DV;
        // the rows all start on the same LDS bank: each entry walks the columns from its own
        // offset, so the lanes of a wave read different banks
        const int rot = 8 * (e % rank) + 32 * ((e / rank) & 1);
        for (int c = part; c < DV; c += 4) {
          const int cc = (c + rot) & (DV - 1);
          g = fma((double)ri[cc], (double)rj[cc], g);
        }
      }
      g += __shfl_xor(g, 1);
      g += __shfl_xor(g, 2);
      if (e < rank * rank && part == 0 && e % rank <= e / rank) lG[e] = g;
    }
    __syncthreads();
    if (wave == 0) {  // b. Cholesky, left-looking
      double maxd = 0.0;
      for (int i = 0; i < rank; ++i) maxd = fmax(maxd, lG[i * rank + i]);
      const double thr = (double)kLsRelTol * (double)kLsRelTol * maxd;
      const int i = lane;
      if (rank <= 8) {
        // In registers: lane i holds row i of G, then of L; row k of L comes from lane k
        // by readlane, so the factorisation makes no LDS round trip (entries above the
        // diagonal are scratch). Only L^-1 goes back to LDS.
        double g[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) g[p] = lG[min(i, rank - 1) * rank + min(p, rank - 1)];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k < rank) {
            double d = g[k];  // in lane k: its pivot, G[k][k] less its row of L so far
#pragma unroll
            for (int p = 0; p < k; ++p) d = fma(-g[p], g[p], d);
            d = readlane_f64(d, k);
            const double lkk = d > thr ? sqrt(d) : 0.0;
            const double inv = lkk > 0.0 ? 1.0 / lkk : 0.0;
            double x = g[k];
#pragma unroll
            for (int p = 0; p < k; ++p) x = fma(-g[p], readlane_f64(g[p], k), x);
            g[k] = (i == k) ? inv : x * inv;  // the diagonal keeps the inverse pivot
          }
        }
        // L^-1 by columns, lane j taking column j: entry r > j is -inv_r times the sum over
        // j <= k < r of L[r][k] L^-1[k][j] (the entries above the diagonal are zero)
        double w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if (r < rank) {
            const double inv_r = readlane_f64(g[r], r);
            double x = 0.0;
#pragma unroll
            for (int k = 0; k < r; ++k) x = fma(readlane_f64(g[k], r), w[k], x);
            w[r] = (i == r) ? inv_r : (i < r ? -inv_r * x : 0.0);
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r)
          if (i < rank && r < rank && r >= i) lG[r * rank + i] = w[r];  // L^-1[r][i]
      } else {  // larger ranks: through LDS
        for (int k = 0; k < rank; ++k) {
          // every lane reads row k (and its own row) before lanes i >= k write column k
          double dk = lG[k * rank + k];
          for (int p = 0; p < k; ++p) dk = fma(-lG[k * rank + p], lG[k * rank + p], dk);
          const double lkk = dk > thr ? sqrt(dk) : 0.0;
          double x = 0.0;
          if (i > k && i < rank && lkk > 0.0) {
            x = lG[i * rank + k];
            for (int p = 0; p < k; ++p) x = fma(-lG[i * rank + p], lG[k * rank + p], x);
            x /= lkk;
          }
          if (i > k && i < rank) lG[i * rank + k] = x;
          if (i == k) lG[k * rank + k] = lkk > 0.0 ? 1.0 / lkk : 0.0;  // kept: the inverse pivot
        }
        // L^-1 by columns into the upper triangle (L^-1[r][j] at row j, column r), lane j
        // taking column j; L^-1[k][j] for k >= j is then lG[j][k], the diagonal included.
        // Once done (L is no longer read), each lane moves its column below the diagonal.
        if (i < rank) {
          for (int r = i + 1; r < rank; ++r) {
            double x = 0.0;
            for (int k = i; k < r; ++k) x = fma(lG[r * rank + k], lG[i * rank + k], x);
            lG[i * rank + r] = -lG[r * rank + r] * x;
          }
        }
        for (int r = i + 1; r < rank; ++r) lG[r * rank + i] = lG[i * rank + r];
      }
    }
    __syncthreads();
    // c. Q = L^-1 Sk, one column per thread, last row first so that row m still reads the
    //    sketch rows p <= m it needs (in place); each row is formed in fp64 from the exact
    //    sketch values, with no rounded row of Q feeding the next
    for (int c = tid; c < DV; c += NT) {
      for (int m = rank - 1; m >= 0; --m) {
        double x = 0.0;
        for (int p = 0; p <= m; ++p) x = fma(lG[m * rank + p], (double)lQ[p * DV + c], x);
        lQ[m * DV + c] = (float)x;  // zero for a dropped row
      }
    }
    __syncthreads();
    // Four rows of Q at a time, summed over the 8 lanes of the row group as a
    // reduce-scatter: slot sl of lane cg holds Q row m0 + (sl ^ f) with f = lane bits 2, 1
    // of cg, so the lane that row_half_mirror pairs it with (cg ^ 7) holds the same row in
    // slot sl ^ 3, and quad_perm 2301's partner (cg ^ 2) in slot sl ^ 1. Four adds leave
    // row m0 + f summed over all 8 lanes (twelve as four separate all-reduces).
    const int f = ((cg >> 1) & 1) | ((cg >> 2) << 1);
    for (int m0 = 0; m0 < rank; m0 += 4) {
      float4 qv[4];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int m = m0 + (sl ^ f);
        const float4 x = *reinterpret_cast<const float4*>(lQ + min(m, rank - 1) * DV + col);
        qv[sl] = m < rank ? x : f4(0.f);
      }
#pragma unroll
      for (int mm = 0; mm < RPL; ++mm) {
        float a[4];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          a[sl] = qv[sl].x * s[mm].x;
          a[sl] = fmaf(qv[sl].y, s[mm].y, a[sl]);
          a[sl] = fmaf(qv[sl].z, s[mm].z, a[sl]);
          a[sl] = fmaf(qv[sl].w, s[mm].w, a[sl]);
        }
        a[0] += dpp<DPP_HALF_MIRROR>(a[3]);  // lanes cg, cg ^ 7
        a[1] += dpp<DPP_HALF_MIRROR>(a[2]);
        a[0] += dpp<DPP_QUAD_2301>(a[1]);    // and cg ^ 2, cg ^ 5
        a[0] += dpp<DPP_QUAD_1032>(a[0]);    // and the other four (cg ^ 1 shares f)
        // row m0 + f of Q against row mm * 8 + rg of S, over this wave's 32 columns
        if (!(cg & 1) && m0 + f < rank) lP[(wave * rank + m0 + f) * DK + mm * 8 + rg] = a[0];
      }
    }
    __syncthreads();
    float* Yu = rmap + unit * (size_t)rank * DK;
    for (int e = tid; e < rank * DK; e += NT) {
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < DV / 32; ++w) y += lP[w * rank * DK + e];
      Yu[e] = y;
    }
    for (int e = tid; e < rank * DV; e += NT) Qu[e] = lQ[e];
  };

  auto finish = [&]() {
    if (n > 0) {
#pragma unroll
      for (int m = 0; m < RPL; ++m)
        store_stream(Su + (size_t)(m * 8 + rg) * DV + col, s[m]);
    }
    if (sketch == nullptr) return;
    TSK* Sku = sketch + ((size_t)seq * rt.total() + rt.offset(head)) * DV;
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
      if constexpr (LS) {
        if (m < rank) *reinterpret_cast<float4*>(lQ + m * DV + col) = res;
      } else {
        if (m < rank) store4(Sku + (size_t)m * DV + col, res);  // fp32, or bf16 rounded to nearest
      }
    }
    if constexpr (LS) ls_epilogue(Sku);
  };

  if constexpr (RULE == KDA) {
#pragma unroll 1
    for (int t = 0; t < n; ++t) {
      float kr[RPL], ar[RPL];
      Vec<float, RPL>::load(lk + t * DK + row0, kr);
      Vec<float, RPL>::load(ld + t * DK + row0, ar);
      const float4 vv = *reinterpret_cast<const float4*>(lv + t * DV + col);
      const float b = lb[t];
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
    finish();
  } else {
    // Mamba-2 and GDN decay the whole state by one scalar a_t per token. With
    // rho_t = a_{t+1} ... a_{n-1} (the decay still to come after token t), the
    // tile carries X_t = rho_t S_t instead of S_t:
    //   X_{-1} = rho_{-1} S_win,   X_t = X_{t-1} + k_t (rho_t w_t)^T,   X_{n-1} = S,
    // with rho_t w_t = rho_t v_t (Mamba-2) or b_t (rho_t v_t - X_{t-1}^T k_t)
    // (GDN, since rho_t a_t = rho_{t-1}). Each token then costs one FMA per
    // element for the write (plus one for the GDN reduction); the decay is a
    // single scaling of the tile per window. No division: rho is a product of
    // gates, a zero gate simply clears what came before it.
    // Lane L holds rho_{L-1} = a_L ... a_{n-1} (lanes >= n hold 1).
    float rho = 1.f;
    for (int j = lane; j < n; ++j) rho *= ld[j];
    const float rho_start = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), 0));
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = scale4(rho_start, s[m]);
#pragma unroll 1
    for (int t = 0; t < n; ++t) {
      float kr[RPL];
      Vec<float, RPL>::load(lk + t * DK + row0, kr);
      const float4 vv = *reinterpret_cast<const float4*>(lv + t * DV + col);
      const float rho_t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rho), t + 1));
      float4 w = scale4(rho_t, vv);
      if constexpr (RULE == GDN) {
        float4 p = f4(0.f);
#pragma unroll
        for (int m = 0; m < RPL; ++m) p = fma4(kr[m], s[m], p);
        p = tile_allreduce(p);  // X_{t-1}^T k for this lane's 4 columns
        w = scale4(lb[t], sub4(w, p));
      }
#pragma unroll
      for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, s[m]);
    }
    finish();
  }
}

}  // namespace

size_t update_refresh_lds_bytes(const ssm_dims& d, int n, int max_rank, bool ls) {
  size_t floats = 0;
  (void)dispatch(d.rule, SSM_IN_F32, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto) {
    floats = (size_t)window_lds_floats<decltype(R)::value, decltype(DK)::value,
                                       decltype(DV)::value>(n);
    return hipSuccess;
  });
  // least squares: the sketch rows [r][d_v], the waves' partial read maps [d_v/32][r][d_k]
  // and the Gram matrix / Cholesky factor [r][r] in fp64
  const size_t ls_floats = ls ? (size_t)max_rank * d.d_v + (size_t)(d.d_v / 32) * max_rank * d.d_k +
                                    2 * (size_t)max_rank * max_rank
                              : 0;
  return (floats + (size_t)max_rank * d.d_k + ls_floats) * sizeof(float);
}

hipError_t launch_update_refresh(const ssm_dims& d, const int32_t* rank_offsets, float* state,
                                 void* sketch, const float* basis, const void* k_buf,
                                 const void* v_buf, const float* decay_buf, const float* beta_buf,
                                 int n, hipStream_t stream, const Varlen* varlen, float* read_map) {
  const unsigned units = (unsigned)d.batch * (unsigned)d.heads;
  int max_rank = 0;
  if (sketch != nullptr) max_rank = rank_offsets ? max_rank_of(rank_offsets, d.heads) : d.rank;
  // a variable-length call can stage up to W tokens per row
  const size_t lds = update_refresh_lds_bytes(d, varlen ? d.window : n, max_rank, read_map != nullptr);
  return dispatch(d.rule, d.in_dtype, d.d_k, d.d_v, [&](auto R, auto DK, auto DV, auto T) {
    using TIN = typename decltype(T)::type;
    constexpr int kR = decltype(R)::value, kDK = decltype(DK)::value, kDV = decltype(DV)::value;
    if (read_map != nullptr) {  // least squares: fp32 sketch, uniform rank, lockstep (checked)
      hipLaunchKernelGGL(
          (update_refresh_kernel<kR, kDK, kDV, TIN, float, true, UniformRank, Lockstep>),
          dim3(units), dim3(2 * kDV), lds, stream, state, static_cast<float*>(sketch), read_map,
          basis, static_cast<const TIN*>(k_buf), static_cast<const TIN*>(v_buf), decay_buf,
          beta_buf, d.heads, d.window, UniformRank{d.rank, d.heads}, Lockstep{n});
      return hipGetLastError();
    }
    return with_sketch_type(d, [&](auto SK) {
      using TSK = typename decltype(SK)::type;
      auto go = [&](auto rt, auto rm) {
        hipLaunchKernelGGL(
            (update_refresh_kernel<kR, kDK, kDV, TIN, TSK, false, decltype(rt), decltype(rm)>),
            dim3(units), dim3(2 * kDV), lds, stream, state, static_cast<TSK*>(sketch), nullptr,
            basis, static_cast<const TIN*>(k_buf), static_cast<const TIN*>(v_buf), decay_buf,
            beta_buf, d.heads, d.window, rt, rm);
        return hipGetLastError();
      };
      if (varlen != nullptr) return go(UniformRank{d.rank, d.heads}, *varlen);
      if (rank_offsets == nullptr) return go(UniformRank{d.rank, d.heads}, Lockstep{n});
      return go(make_rank_table(rank_offsets, d.heads), Lockstep{n});
    });
  });
}

}  // namespace ssm
