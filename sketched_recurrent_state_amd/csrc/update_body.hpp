// update_body.hpp -- the once-per-window state write fused with the sketch
// refresh, as the work of one workgroup (SketchSSM pages: readsearch.ai listing
// of arXiv 2609.33051, Abstract, one full-state read per update stores the
// basis outputs; agihunt.info summary, "Error control", the full state is
// updated once per window and the sketch is refreshed in the same kernel).
// Launched on its own by update_refresh.hip, and beside the sketch read in the
// serving step of decode_step.hpp.
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
// load instruction of the workgroup covers 8 whole rows of S (contiguous).
#pragma once

#include "common.hpp"

namespace ssm {

// Rank decisions of the least-squares refresh: a sketch row whose part orthogonal
// to the rows before it is below this fraction of the largest row norm adds nothing.
constexpr float kLsRelTol = 1e-5f;

// LS = false: stores Sk = B S (row m = S^T b_m). LS = true (least-squares
// coefficients): stores instead Q, orthonormal rows spanning the rows of Sk, in
// `sketch`, and the read map Y = Q S^T [r][d_k] in `rmap`; a read then gives
// Q^T (Y q~), the projection of S^T q~ on the span of the sketch rows.
// The current token of one unit when it is the newest token of the window being
// applied: it is then taken from here (and also written into its buffer slot) instead
// of from the window buffer. All null: every token comes from the buffer.
template <typename TIN>
struct CurrentToken {
  const TIN* k = nullptr;
  const TIN* v = nullptr;
  const float* d = nullptr;
  const float* b = nullptr;
};

// One unit's window update and refresh, the work of one workgroup of
// TileLayout<DK, DV>::NT threads: head `head` of slot `seq`, applying its first n
// buffered tokens.
// MMA: the refresh on the matrix cores (refresh_mfma below), chosen by the host for ranks
// above 8; else the fp32 VALU reduce-scatter.
template <int RULE, int DK, int DV, typename TIN, typename TSK, bool LS, typename RT,
          bool MMA = false>
__device__ __forceinline__ void update_refresh_unit(
    float* __restrict__ state, TSK* __restrict__ sketch, float* __restrict__ rmap,
    const float* __restrict__ basis, const TIN* kbuf, const TIN* vbuf, const float* dbuf,
    const float* bbuf, int heads, int window, const RT& rt, int head, int seq, int n,
    const CurrentToken<TIN>& cur) {
  using TL = TileLayout<DK, DV>;
  constexpr int CG = TL::CG, RG = TL::RG;  // column groups per wave, row groups
  constexpr int RPL = TL::RPL;             // rows of S per lane
  constexpr int NT = TL::NT;               // threads per unit: one wave per 4 CG columns
  constexpr int DSTR = (RULE == KDA) ? DK : 1;
  static_assert(!MMA || (!LS && CG == 8), "the matrix-core refresh: d_v >= 32, no least squares");

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);

  const size_t unit = (size_t)seq * heads + head;
  const int rank = rt.rank(head);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = lane % CG, rg = lane / CG;
  const int col = wave * (4 * CG) + cg * 4;
  // s[m] holds row m * RG + rg of S; the LDS copies of keys, gates and basis
  // keep this lane's d_k / RG values at [row0, row0 + RPL) (interleaved_pos).
  const int row0 = rg * RPL;

  // 1. issue the staging reads: the window's tokens and the head's basis (each
  //    thread's first chunk of every array, one memory round trip in all)
  const size_t slot0 = (size_t)unit * window;
  UnitWindow<TIN> uw{const_cast<TIN*>(kbuf) + slot0 * DK, const_cast<TIN*>(vbuf) + slot0 * DV,
                     const_cast<float*>(dbuf) + slot0 * DSTR,
                     (RULE == MAMBA2) ? nullptr : const_cast<float*>(bbuf) + slot0,
                     cur.k, cur.v, cur.d, cur.b};
  WindowStage<RULE, DK, DV, TIN, NT, true, RG> stage;
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
    s[m] = load_stream(Su + (size_t)(m * RG + rg) * DV + col);
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
      row[interleaved_pos<DK, RG>(i0)] = x4.x;
      row[interleaved_pos<DK, RG>(i0 + 1)] = x4.y;
      row[interleaved_pos<DK, RG>(i0 + 2)] = x4.z;
      row[interleaved_pos<DK, RG>(i0 + 3)] = x4.w;
    };
    if (tid * 4 < rank * DK) put(b4, tid * 4);
    for (int e = (tid + NT) * 4; e < rank * DK; e += NT * 4)
      put(*reinterpret_cast<const float4*>(Bh + e), e);
  }
  __syncthreads();

  // 4. the window's tokens, in order: S <- M_t S + b_t k_t v_t^T on the
  //    register-resident piece; the k^T S reduction over d_k crosses the RG
  //    lanes that share this lane's columns. Mamba-2 and GDN carry a scaled
  //    copy of the piece so the per-token decay costs nothing (below); KDA
  //    decays rows by different gates and updates S directly.
  // 5. write the state back (the only HBM write of S), then
  // 6. refresh the sketch from the register-resident state: Sk[m] = S^T b_m.
  //    Eight basis rows at a time; the d_k reduction is a reduce-scatter over
  //    lane bits 5, 4 and 3 (after a sum over bit 2 when RG = 16), after which the
  //    lanes with lane >> 3 = j hold basis row m0 + j.
  // Least-squares refresh, after the rows of Sk are in LDS (lQ). The rows are made
  // orthonormal as Gram-Schmidt would, through the Cholesky factor of their Gram
  // matrix (Sk = L Q with Q orthonormal rows, L lower triangular, G = Sk Sk^T = L L^T):
  //   a. the lower triangle of G in fp64 (products of fp32 values are exact there),
  //      four lanes per entry, each over d_v / 4 columns in 16-byte reads;
  //   b. one wave (it rotates with the unit, so no SIMD takes every unit's share)
  //      factors G = L L^T column by column, lane i owning row i; a row whose pivot,
  //      its squared residual against the rows before it, is below kLsRelTol^2 of the
  //      largest squared row norm is dropped (zero column of L). The inverse pivot is
  //      the reciprocal square root of the pivot (v_rsq_f64 and two Newton steps);
  //   c. step b also forms L^-1 (fp64, in place of L, the inverse pivots on the
  //      diagonal; a dropped row is zero), then Q = L^-1 Sk in place, one column of
  //      the sketch per thread (the threads rotate with the unit as in b), each row
  //      from the exact fp32 sketch;
  //   d. every wave forms Y = Q S^T over its 32 columns: per row of S a dot product
  //      of 4 columns, summed over the 8 lanes of the row group (lane bits 0..2) as a
  //      reduce-scatter over four rows of Q at a time;
  //   e. the waves' partial Y are added in a fixed order and stored with Q.
  constexpr int NW = TL::WAVES;  // waves of the unit: column blocks of 4 CG columns
  float* lQ = lB + rank * DK;  // [rank][DV] (LS only)
  float* lP = lQ + rank * DV;  // [NW][rank][DK] per-wave partial Y (LS only)
  double* lG = reinterpret_cast<double*>(lP + NW * rank * DK);  // [rank][rank] (LS only)
  const int ls_turn = (int)(unit % (NT / 64));  // the wave (and threads) of steps b and c
  auto ls_epilogue = [&](float* Qu) {
    __syncthreads();
    // a. Gram matrix, lower triangle: entry (i, j), j <= i, is number i (i + 1) / 2 + j
    const int ntri = rank * (rank + 1) / 2;
    for (int e0 = 0; e0 < ntri; e0 += NT / 4) {
      const int e = e0 + tid / 4, part = tid & 3;
      int i = 0, j = 0;
      double g0 = 0.0, g1 = 0.0;
      if (e < ntri) {
        i = (int)((__builtin_sqrtf(8.f * (float)e + 1.f) - 1.f) * 0.5f);
        if ((i + 1) * (i + 2) / 2 <= e) ++i;  // the float root rounded down past a square
        if (i * (i + 1) / 2 > e) --i;
        j = e - i * (i + 1) / 2;
        const float* ri = lQ + i * DV;
        const float* rj = lQ + j * DV;
        // the rows all start on the same LDS bank: the entries of a wave walk the columns
        // from different offsets, so their lanes read different banks
        const int rot = 16 * ((tid >> 2) & 7);
#pragma unroll
        for (int c = 0; c < DV; c += 16) {
          const int cc = (c + 4 * part + rot) & (DV - 1);
          const float4 a = *reinterpret_cast<const float4*>(ri + cc);
          const float4 b = *reinterpret_cast<const float4*>(rj + cc);
          g0 = fma((double)a.x, (double)b.x, g0);
          g1 = fma((double)a.y, (double)b.y, g1);
          g0 = fma((double)a.z, (double)b.z, g0);
          g1 = fma((double)a.w, (double)b.w, g1);
        }
      }
      double g = g0 + g1;
      g += __shfl_xor(g, 1);
      g += __shfl_xor(g, 2);
      if (e < ntri && part == 0) lG[i * rank + j] = g;
    }
    __syncthreads();
    if (wave == ls_turn) {  // b. Cholesky, left-looking
      double maxd = 0.0;
      for (int i = 0; i < rank; ++i) maxd = fmax(maxd, lG[i * rank + i]);
      const double thr = (double)kLsRelTol * (double)kLsRelTol * maxd;
      const int i = lane;
      if (rank <= 8) {
        // In registers: lane i holds row i of G, then of L; row k of L comes from lane k
        // by readlane, so the factorisation makes no LDS round trip (entries above the
        // diagonal are scratch, zero at the start). Only L^-1 goes back to LDS.
        double g[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
          g[p] = (i < rank && p <= i) ? lG[i * rank + p] : 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (k < rank) {
            double d = g[k];  // in lane k: its pivot, G[k][k] less its row of L so far
#pragma unroll
            for (int p = 0; p < k; ++p) d = fma(-g[p], g[p], d);
            d = readlane_f64(d, k);
            const double inv = d > thr ? rsqrt_f64(d) : 0.0;
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
          const double inv = dk > thr ? rsqrt_f64(dk) : 0.0;
          double x = 0.0;
          if (i > k && i < rank && inv > 0.0) {
            x = lG[i * rank + k];
            for (int p = 0; p < k; ++p) x = fma(-lG[i * rank + p], lG[k * rank + p], x);
            x *= inv;
          }
          if (i > k && i < rank) lG[i * rank + k] = x;
          if (i == k) lG[k * rank + k] = inv;  // kept: the inverse pivot
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
    // c. Q = L^-1 Sk in place, one column per thread: up to rank 8 the column is read into
    //    registers first; above, the rows go last first, so that row m still reads the
    //    sketch rows p <= m it needs. Each row is formed in fp64 from the exact sketch
    //    values, with no rounded row of Q feeding the next.
    const int c = (tid + DV * ls_turn) % NT;  // DV divides NT
    if (c < DV) {
      if (rank <= 8) {  // the column in registers first, then every row from it
        double x[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) x[p] = p < rank ? (double)lQ[p * DV + c] : 0.0;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < rank) {
            double q = 0.0;
#pragma unroll
            for (int p = 0; p <= m; ++p) q = fma(lG[m * rank + p], x[p], q);
            lQ[m * DV + c] = (float)q;  // zero for a dropped row
          }
        }
      } else {
        for (int m = rank - 1; m >= 0; --m) {
          double q = 0.0;
          for (int p = 0; p <= m; ++p) q = fma(lG[m * rank + p], (double)lQ[p * DV + c], q);
          lQ[m * DV + c] = (float)q;  // zero for a dropped row
        }
      }
    }
    __syncthreads();
    if constexpr (CG == 8) {
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
    } else {
      // d_v = 16 (4 lanes per row group): four rows of Q at a time, each summed over the row
      // group's lanes (lane bits 0, 1) by two quad permutations; lane cg keeps row m0 + cg
      for (int m0 = 0; m0 < rank; m0 += 4) {
        float4 qv[4];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int m = m0 + sl;
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
            a[sl] += dpp<DPP_QUAD_1032>(a[sl]);
            a[sl] += dpp<DPP_QUAD_2301>(a[sl]);
          }
          const float mine = cg == 0 ? a[0] : cg == 1 ? a[1] : cg == 2 ? a[2] : a[3];
          if (m0 + cg < rank) lP[(wave * rank + m0 + cg) * DK + mm * RG + rg] = mine;
        }
      }
    }
    __syncthreads();
    float* Yu = rmap + unit * (size_t)rank * DK;
    for (int e = tid; e < rank * DK; e += NT) {
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) y += lP[w * rank * DK + e];
      Yu[e] = y;
    }
    for (int e = tid; e < rank * DV; e += NT) Qu[e] = lQ[e];
  };

  // The refresh on the matrix cores (MMA, chosen by the host: above rank 8, where the fp32
  // VALU refresh, 2 r d_k d_v / NT FMAs per lane, outweighs the token loop: 17% off the GDN
  // update at r = 32, W = 16; and from rank 8 in launches whose update blocks fit in one
  // round of workgroups, where no other workgroup's stream hides the refresh. Not below
  // rank 8: at r = 4 it is 2% slower). Eight basis rows at a time, with
  // v_mfma_f32_16x16x32_bf16 (A[i][*] from lane i + 16g, B[*][j] from lane j + 16g,
  // element e of lane group g of A paired with element e of lane group g of B; D[i][j]
  // in lane j + 16 (i / 4), element i % 4) and fp32 accumulation. Each fp32 value is
  // split as x = hi + lo + d with hi = bf16(x), lo = bf16(x - hi) and |d| <= 2^-17 |x|;
  // a product is taken as hi*hi + hi*lo + lo*hi (three passes), so it is off by at
  // most about 2^-16 of |b| |s|, against the 1e-4 the sketch is held to.
  //  - B operand: lane l = j + 16g (j = cg + 8 (rg & 1), g = rg >> 1) passes its own
  //    state values of column c at rows 8m + rg for the 8 m of a block;
  //  - A operand: the same lane passes b_{m0 + cg} at the same rows.
  //  An element of D then pairs equal rows only on its diagonal 8 x 8 blocks (i, j < 8:
  //  the even row groups; i, j >= 8: the odd ones); the other two blocks are not used.
  //  Lane l < 32 with bit 3 clear adds lane l + 40's odd half (a permlane32 swap, then
  //  row_ror:8) and holds basis rows m0 + 4 (l >> 4) + e, e = 0..3, at the 4 columns of
  //  column group l & 7.
  auto refresh_mfma = [&](TSK* Sku) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    constexpr int MB = (RPL + 7) / 8;  // blocks of 8 rows of this lane (zero-padded)
    // two floats -> their hi parts packed (one v_cvt_pk_bf16_f32) and lo parts packed
    auto split2 = [](float a, float b, uint32_t& hp, uint32_t& lp) {
      hp = pack_bf16x2(a, b);
      lp = pack_bf16x2(a - bf16_lo(hp), b - bf16_hi(hp));
    };
    auto as8 = [](const uint32_t* w) {  // 4 packed words -> 8 bf16 (element 2i in the low half)
      return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    };
    bf16x8 sh[4][MB], sl[4][MB];      // [column][block]: hi and lo parts of the state
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb * 8 + 2 * i;
          const float4 x0 = m < RPL ? s[m] : f4(0.f);
          const float4 x1 = m + 1 < RPL ? s[m + 1] : f4(0.f);
          const float a = c == 0 ? x0.x : c == 1 ? x0.y : c == 2 ? x0.z : x0.w;
          const float b = c == 0 ? x1.x : c == 1 ? x1.y : c == 2 ? x1.z : x1.w;
          split2(a, b, hw[i], lw[i]);
        }
        sh[c][mb] = as8(hw);
        sl[c][mb] = as8(lw);
      }
    }
    const bool owner = lane < 32 && (lane & 8) == 0;
    const int ocol = wave * 32 + (lane & 7) * 4;
    for (int m0 = 0; m0 < rank; m0 += 8) {
      v4f acc[4] = {};
      const float* brow = lB + min(m0 + cg, rank - 1) * DK + row0;  // b_{m0 + cg}, this lane's rows
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float bx[8];
        if constexpr (RPL >= 8) {
          Vec<float, 8>::load(brow + mb * 8, bx);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) bx[i] = i < RPL ? brow[i] : 0.f;
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split2(bx[2 * i], bx[2 * i + 1], hw[i], lw[i]);
        const bf16x8 ah = as8(hw), al = as8(lw);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sh[c][mb], acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl[c][mb], acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh[c][mb], acc[c], 0, 0, 0);
        }
      }
      float out[4][4];  // [e][c]: basis row m0 + 4 (lane >> 4) + e, column ocol + c
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[c][e];
          const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                          false, false);  // [1]: lane l | 32
          out[e][c] = x + dpp<DPP_ROR8>(__uint_as_float(h[1]));
        }
      }
      if (owner) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + 4 * (lane >> 4) + e;
          if (m < rank)
            store4(Sku + (size_t)m * DV + ocol, make_float4(out[e][0], out[e][1], out[e][2],
                                                            out[e][3]));
        }
      }
    }
  };

  auto finish = [&]() {
    if (n > 0) {
#pragma unroll
      for (int m = 0; m < RPL; ++m)
        store_stream(Su + (size_t)(m * RG + rg) * DV + col, s[m]);
    }
    if (sketch == nullptr) return;
    TSK* Sku = sketch + ((size_t)seq * rt.total() + rt.offset(head)) * DV;
    if constexpr (MMA) {
      refresh_mfma(Sku);
      return;
    }
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
        if constexpr (CG == 4) {  // the two row groups that differ in lane bit 2
          P[e].x += xor4(P[e].x);
          P[e].y += xor4(P[e].y);
          P[e].z += xor4(P[e].z);
          P[e].w += xor4(P[e].w);
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
      const int m = m0 + (lane >> 3);
      const bool owner = CG == 8 || !(lane & 4);  // lanes l and l ^ 4 hold the same sums
      if constexpr (LS) {
        if (m < rank) *reinterpret_cast<float4*>(lQ + m * DV + col) = res;
      } else {
        if (m < rank && owner) store4(Sku + (size_t)m * DV + col, res);  // fp32, or bf16 rounded
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
      p = tile_sum<CG>(p);
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
        p = tile_sum<CG>(p);  // X_{t-1}^T k for this lane's 4 columns
        w = scale4(lb[t], sub4(w, p));
      }
#pragma unroll
      for (int m = 0; m < RPL; ++m) s[m] = fma4(kr[m], w, s[m]);
    }
    finish();
  }
}

}  // namespace ssm
