// update_chunk.hpp -- the once-per-window state write fused with the sketch
// refresh for the rules whose transition is a scalar decay times (I - beta k k^T)
// (Mamba-2, Gated DeltaNet), with the window's contractions on the matrix cores.
// It computes what update_body.hpp computes (SketchSSM pages: readsearch.ai
// listing of arXiv 2609.33051, Abstract, one full-state read per update stores
// the basis outputs; agihunt.info summary, "Error control", the full state is
// updated once per window and the sketch refreshed in the same kernel), for
// windows long enough that the vector version is bound by its FMA issue rate.
//
// The window in closed form. With rho_t the product of the gates after token t,
// the tile carries X_t = rho_t S_t (as in update_body.hpp):
//   X_{-1} = rho_{-1} S_win,  X_t = X_{t-1} + k_t u_t^T,
//   u_t = beta_t (rho_t v_t - X_{t-1}^T k_t)   (GDN),   u_t = rho_t v_t  (Mamba-2),
// and X_{t-1}^T k_t = X_{-1}^T k_t + sum_{s<t} (k_s . k_t) u_s. So, for the whole
// window at once:
//   1. P = [K; B] X_{-1}: every token's k^T X_{-1} and the basis outputs of
//      X_{-1}, one contraction over d_k (K = the window's keys as rows, B the
//      basis rows);
//   2. u_t = beta_t (rho_t v_t - P_t - sum_{s<t} G_ts u_s), G = K K^T: a
//      triangular recurrence shared by every column, solved once per unit as
//      U = T R (T below), R = rho v - P;
//   3. S = X_{-1} + K^T U, and Sk = B S = B X_{-1} + (B K^T) U.
// Steps 1 and 3, U = T R and the (B K^T) U term run on v_mfma_f32_32x32x2f32 (fp32
// products, fp32 accumulation), so the window costs about 7,000 matrix-core
// cycles per wave at W = 16 and a few hundred vector instructions, where the
// vector form issues two FMAs per state element per token.
//
// Layout. One workgroup per unit, one wave per 32 columns of S, each wave all
// d_k rows. The state stays in the accumulator layout of the 32 x 32 MFMA for
// the whole window: lane l (column l % 32 of the wave's block, half h = l / 32)
// holds, for every block of 32 rows, rows 8a + 4h + i (a, i < 4) in 16
// registers. That layout is at once the B operand of step 1 (contraction index
// k = h at register 4a + i) and the accumulator of step 3. Its memory accesses
// are one 4-byte element per lane and register, two whole 128-byte rows per
// load instruction: measured as fast as 16-byte accesses (5.86 TB/s in place).
//
// Limits: d_k and d_v multiples of 32, at most 16 tokens and 16 basis rows per
// unit (the 32 rows of the tile of step 1).
#pragma once

#include "common.hpp"
#include "update_body.hpp"

namespace ssm {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChunkTokens = 16;  // token rows of the tile of step 1
// Buffer resources (raw, stride 0): word 3 of the descriptor for 32-bit data on gfx950,
// and the cache-policy bit of a non-temporal access.
constexpr int kBufferRsrcFlags = 0x00020000;
constexpr int kAuxNonTemporal = 2;
constexpr int kChunkRank = 16;    // basis rows beside them

// LDS of one unit, in floats.
template <int DK, int DV>
struct ChunkLds {
  static constexpr int KS = DK + 4;                // row stride of [K; B] (rows on distinct banks)
  static constexpr int TS = 20;                    // row stride of T and of B K^T
  static constexpr int KP = 0;                     // [32][KS]: keys 0..15, basis rows 16..31
  static constexpr int V = KP + 32 * KS;           // [16][DV] values
  static constexpr int GATE = V + 16 * DV;         // [16] scalar gates
  static constexpr int BETA = GATE + 16;           // [16] beta (0 past the window)
  static constexpr int RHO = BETA + 16;            // [32]: rho_{-1}, rho_0, ..., rho_15
  static constexpr int G = RHO + 32;               // [16][16] k_t . k_s
  static constexpr int T = G + 256;                // [16][TS] the recurrence's solution matrix
  static constexpr int BK = T + 16 * TS;           // [16][TS] b_m . k_t
  static constexpr int SK = BK + 16 * TS;          // [16][DV] the new sketch, for coalesced stores
  static constexpr int FLOATS = SK + 16 * DV;
};

// The window's first n tokens -> LDS as fp32 (keys in rows 0..n-1 of [K; B],
// values, gates, beta), zeros for the token rows n..15. Two phases as in
// WindowStage: issue() starts every thread's first chunk of each array, commit()
// stores them and copies any further chunks. With a fused append the newest slot
// is read from the current token and also written into the buffer.
template <int RULE, int DK, int DV, typename TIN, int NT>
struct ChunkStage {
  using L = ChunkLds<DK, DV>;
  using WS = WindowStage<RULE, DK, DV, TIN, NT>;
  static constexpr int VIN = 16 / sizeof(TIN);
  Packed<TIN, VIN> k0, v0;
  float g0 = 0.f, b0 = 0.f;

  __device__ __forceinline__ void issue(const UnitWindow<TIN>& uw, int n, int tid) {
    const bool fused = uw.kt != nullptr;
    const int last = n - 1;
    k0.load(WS::template src<TIN>(uw.k, uw.kt, min(tid * VIN, n * DK - VIN), DK, last, fused));
    v0.load(WS::template src<TIN>(uw.v, uw.vt, min(tid * VIN, n * DV - VIN), DV, last, fused));
    g0 = *WS::template src<float>(uw.d, uw.dt, min(tid, last), 1, last, fused);
    if constexpr (RULE == GDN) b0 = *WS::template src<float>(uw.b, uw.bt, min(tid, last), 1, last, fused);
  }

  __device__ __forceinline__ void commit(float* lds, const UnitWindow<TIN>& uw, int n,
                                         int tid) const {
    const bool fused = uw.kt != nullptr;
    const int last = n - 1;
    auto put_k = [&](const Packed<TIN, VIN>& x, int e) {
      if (fused && e / DK == last) x.store(uw.k + e);
      float f[VIN];
      x.unpack(f);
      Vec<float, VIN>::store(lds + L::KP + (e / DK) * L::KS + e % DK, f);
    };
    auto put_v = [&](const Packed<TIN, VIN>& x, int e) {
      if (fused && e / DV == last) x.store(uw.v + e);
      float f[VIN];
      x.unpack(f);
      Vec<float, VIN>::store(lds + L::V + e, f);
    };
    if (tid * VIN < n * DK) put_k(k0, tid * VIN);
    if (tid * VIN < n * DV) put_v(v0, tid * VIN);
    if (tid < kChunkTokens) {
      if (tid < n && fused && tid == last) {
        uw.d[tid] = g0;
        if constexpr (RULE == GDN) uw.b[tid] = b0;
      }
      lds[L::GATE + tid] = tid < n ? g0 : 1.f;
      lds[L::BETA + tid] = (RULE == GDN && tid < n) ? b0 : 0.f;
    }
    for (int e = (tid + NT) * VIN; e < n * DK; e += NT * VIN) {
      Packed<TIN, VIN> x;
      x.load(WS::template src<TIN>(uw.k, uw.kt, e, DK, last, fused));
      put_k(x, e);
    }
    for (int e = (tid + NT) * VIN; e < n * DV; e += NT * VIN) {
      Packed<TIN, VIN> x;
      x.load(WS::template src<TIN>(uw.v, uw.vt, e, DV, last, fused));
      put_v(x, e);
    }
    for (int e = tid * 4; e < (kChunkTokens - n) * DK; e += NT * 4)  // token rows past the window
      *reinterpret_cast<float4*>(lds + L::KP + (n + e / DK) * L::KS + e % DK) = f4(0.f);
    for (int e = tid * 4; e < (kChunkTokens - n) * DV; e += NT * 4)
      *reinterpret_cast<float4*>(lds + L::V + n * DV + e) = f4(0.f);
  }
};

// Host-side LDS bytes of the chunked update.
template <int DK, int DV>
constexpr size_t chunk_lds_bytes() {
  return (size_t)ChunkLds<DK, DV>::FLOATS * sizeof(float);
}

// One unit's window update and refresh on the matrix cores: the work of one
// workgroup of 64 * d_v / 32 threads, head `head` of slot `seq`, applying its
// first n <= 16 buffered tokens; at most 16 basis rows.
template <int RULE, int DK, int DV, typename TIN, typename TSK, typename RT>
__device__ __forceinline__ void update_refresh_unit_chunk(
    float* __restrict__ state, TSK* __restrict__ sketch, const float* __restrict__ basis,
    const TIN* kbuf, const TIN* vbuf, const float* dbuf, const float* bbuf, int heads,
    int window, const RT& rt, int head, int seq, int n, const CurrentToken<TIN>& cur) {
  static_assert(RULE == MAMBA2 || RULE == GDN, "scalar-decay rules only");
  static_assert(DK % 32 == 0 && DV % 32 == 0, "tile shape");
  using L = ChunkLds<DK, DV>;
  constexpr int WAVES = DV / 32, NT = 64 * WAVES, RB = DK / 32;

  extern __shared__ float4 lds4[];
  float* lds = reinterpret_cast<float*>(lds4);

  const size_t unit = (size_t)seq * heads + head;
  const int rank = sketch != nullptr ? rt.rank(head) : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, cn = lane & 31;  // row half and column of the accumulator layout
  const int col = wave * 32 + cn;

  // 1. the staging reads (window and basis), then the state
  const size_t slot0 = unit * window;
  UnitWindow<TIN> uw{const_cast<TIN*>(kbuf) + slot0 * DK, const_cast<TIN*>(vbuf) + slot0 * DV,
                     const_cast<float*>(dbuf) + slot0,
                     (RULE == MAMBA2) ? nullptr : const_cast<float*>(bbuf) + slot0,
                     cur.k, cur.v, cur.d, cur.b};
  ChunkStage<RULE, DK, DV, TIN, NT> stage;
  if (n > 0) stage.issue(uw, n, tid);
  const float* Bh = basis + (size_t)rt.offset(head) * DK;
  float4 b4 = f4(0.f);
  if (rank > 0) b4 = *reinterpret_cast<const float4*>(Bh + min(tid * 4, rank * DK - 4));

  // The unit's tile through a buffer resource: the lane's byte offset in a VGPR, each
  // register's row offset a constant (scalar), so the 2 x 16 x d_k/32 accesses of a
  // lane need no per-access address registers. Non-temporal (the aux bit "nt"): S is
  // touched once per window.
  float* Su = state + unit * (DK * DV);
  const __amdgpu_buffer_rsrc_t srsrc =
      __builtin_amdgcn_make_buffer_rsrc(Su, 0, DK * DV * (int)sizeof(float), kBufferRsrcFlags);
  const int voff = (4 * h * DV + col) * (int)sizeof(float);
  auto row_off = [](int rb, int r) { return (32 * rb + 8 * (r >> 2) + (r & 3)) * DV * (int)sizeof(float); };
  // xs[rb][4a + i] = X[32 rb + 8a + 4h + i][col]
  v16f xs[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      xs[rb][r] = __builtin_bit_cast(  // the builtin returns the 32 bits as an integer
          float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, voff, row_off(rb, r), kAuxNonTemporal));
  }

  // 2. staged data to LDS: keys (rows 0..15 of [K; B]), values, gates, beta; the basis
  //    in rows 16..31 (zero past the rank)
  if (n > 0) {
    stage.commit(lds, uw, n, tid);
  } else {
    for (int e = tid * 4; e < kChunkTokens * DK; e += NT * 4)
      *reinterpret_cast<float4*>(lds + L::KP + (e / DK) * L::KS + e % DK) = f4(0.f);
    for (int e = tid * 4; e < kChunkTokens * DV; e += NT * 4)
      *reinterpret_cast<float4*>(lds + L::V + e) = f4(0.f);
    if (tid < kChunkTokens) {
      lds[L::GATE + tid] = 1.f;
      lds[L::BETA + tid] = 0.f;
    }
  }
  {
    float* lB = lds + L::KP + kChunkTokens * L::KS;
    auto put = [&](float4 x4, int e) {
      *reinterpret_cast<float4*>(lB + (e / DK) * L::KS + e % DK) = x4;
    };
    if (tid * 4 < rank * DK) put(b4, tid * 4);
    for (int e = (tid + NT) * 4; e < rank * DK; e += NT * 4)
      put(*reinterpret_cast<const float4*>(Bh + e), e);
    for (int e = rank * DK + tid * 4; e < kChunkRank * DK; e += NT * 4) put(f4(0.f), e);
  }
  __syncthreads();

  // 3. Before the state arrives: the window's Gram matrix G = K K^T and B K^T,
  //    v_mfma_f32_16x16x4f32 over d_k (contraction index k, lane bits 4 and 5, of
  //    instruction j is row 16 (j / 4) + 4k + j % 4); G by wave 0, B K^T by the last
  //    wave. Wave 0 then solves the window's triangular recurrence once for the whole
  //    unit: u = T r with T = (I + diag(beta) L)^-1 diag(beta), L the strictly lower
  //    part of G (lane j < 16 forms column j by forward substitution), and forms the
  //    gate products RHO[0] = rho_{-1}, RHO[t + 1] = rho_t (0 past the window).
  {
    const int m = lane & 15, q = lane >> 4;
    auto gram = [&](int arow, float* out, int ostride) {
      const float* pa = lds + L::KP + arow * L::KS + 4 * q;
      const float* pb = lds + L::KP + m * L::KS + 4 * q;
      v4f g = {};
#pragma unroll
      for (int c = 0; c < DK / 16; ++c) {
        const float4 a = *reinterpret_cast<const float4*>(pa + 16 * c);
        const float4 b = *reinterpret_cast<const float4*>(pb + 16 * c);
        g = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, g, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(4 * q + i) * ostride + m] = g[i];
    };
    if (wave == 0) {
      if (lane <= kChunkTokens) {
        float rho = 1.f;
        for (int j = lane; j < n; ++j) rho *= lds[L::GATE + j];
        lds[L::RHO + lane] = (lane == 0 || lane - 1 < n) ? rho : 0.f;
      }
      if (RULE == GDN && n > 0) {
        gram(m, lds + L::G, 16);
        // the same wave reads back what its other lanes wrote (a wave's LDS accesses
        // complete in order; the fence keeps the compiler from moving them)
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lane < kChunkTokens) {
          const float* G = lds + L::G;
          const float* beta = lds + L::BETA;
          float x[kChunkTokens];
#pragma unroll
          for (int t = 0; t < kChunkTokens; ++t) {
            float acc_t = t == lane ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < t; ++s2) acc_t = fmaf(-G[t * 16 + s2], x[s2], acc_t);
            x[t] = beta[t] * acc_t;
          }
#pragma unroll
          for (int t = 0; t < kChunkTokens; ++t) lds[L::T + t * L::TS + lane] = x[t];
        }
      }
    }
    if (wave == WAVES - 1 && rank > 0 && n > 0) gram(kChunkTokens + m, lds + L::BK, L::TS);
  }
  __syncthreads();

  // 4. X_{-1} = rho_{-1} S_win, then P = [K; B] X_{-1} (rows M = 8a + 4h + i of acc:
  //    tokens for M < 16, basis rows M - 16 above)
  const float rho_start = lds[L::RHO];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) xs[rb] *= rho_start;
  v16f acc = {};
  {
    const float* pa = lds + L::KP + cn * L::KS + 4 * h;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 av = *reinterpret_cast<const float4*>(pa + 32 * rb + 8 * a);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, xs[rb][4 * a + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, xs[rb][4 * a + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, xs[rb][4 * a + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, xs[rb][4 * a + 3], acc, 0, 0, 0);
      }
    }
  }

  // 5. U into acc rows 0..15 (register r < 8 holds token tk(r) = 8 (r / 4) + 4h + r % 4,
  //    the contraction index of the next two steps): r_t = rho_t v_t - P_t (GDN) or
  //    rho_t v_t (Mamba-2, where u = r); GDN then takes U = T R on the matrix cores,
  //    the A operand T[M][tk] in lanes M < 16 (zero rows above leave the basis rows).
  if (n > 0) {
    float rv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int t = 8 * (r >> 2) + 4 * h + (r & 3);
      const float vt = lds[L::V + t * DV + col] * lds[L::RHO + 1 + t];
      rv[r] = (RULE == GDN) ? vt - acc[r] : vt;
      acc[r] = (RULE == GDN) ? 0.f : vt;
    }
    if constexpr (RULE == GDN) {
      const bool trow = cn < kChunkTokens;
      const float* pt = lds + L::T + (trow ? cn : 0) * L::TS + 4 * h;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float4 tv = *reinterpret_cast<const float4*>(pt + 8 * a);
        if (!trow) tv = f4(0.f);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(tv.x, rv[4 * a + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(tv.y, rv[4 * a + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(tv.z, rv[4 * a + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(tv.w, rv[4 * a + 3], acc, 0, 0, 0);
      }
    }
  }

  // 6. the basis outputs of the new state: acc rows 16..31 += (B K^T) U. Formed in an
  //    accumulator of its own that starts at zero (zero A rows below 16), then added:
  //    every MFMA here accumulates in place, so none of its input registers is freed
  //    (and reloaded) while the matrix core may still read it.
  if (n > 0 && rank > 0) {
    const bool brow = cn >= kChunkTokens;
    const float* pb = lds + L::BK + (brow ? cn - kChunkTokens : 0) * L::TS + 4 * h;
    float4 bv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      bv[a] = *reinterpret_cast<const float4*>(pb + 8 * a);
      if (!brow) bv[a] = f4(0.f);
    }
    v16f sacc = {};
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[a].x, acc[4 * a + 0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[a].y, acc[4 * a + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[a].z, acc[4 * a + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[a].w, acc[4 * a + 3], sacc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 8; r < 16; ++r) acc[r] += sacc[r];
  }
  // the sketch rows of this wave's columns to LDS: register r >= 8 holds basis row
  // 8 (r / 4 - 2) + 4h + r % 4
  if (rank > 0) {
#pragma unroll
    for (int r = 8; r < 16; ++r) {
      const int m = 8 * ((r >> 2) - 2) + 4 * h + (r & 3);
      if (m < rank) lds[L::SK + m * DV + col] = acc[r];
    }
  }

  // 7. S = X_{-1} + K^T U (A operand: key tk(r) at this lane's row 32 rb + cn), then
  //    the state's only write
  if (n > 0) {
    const float* pk = lds + L::KP + 4 * h * L::KS + cn;
    const int na = n > 8 ? 2 : 1;  // token rows 8..15 are zero below 9 tokens
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        if (a < na) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xs[rb] = __builtin_amdgcn_mfma_f32_32x32x2f32(pk[(8 * a + i) * L::KS + 32 * rb],
                                                          acc[4 * a + i], xs[rb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, (float)xs[rb][r]), srsrc,
                                              voff, row_off(rb, r), kAuxNonTemporal);
    }
  }

  // 8. the sketch of this wave's 32 columns, back from LDS so that each lane stores 16
  //    contiguous bytes (lane l: row l / 8 + 8j, columns 4 (l % 8) ..): eight rows of
  //    128 bytes per store instruction. One lane's own registers hold four rows of one
  //    column; stored directly, those scattered 4-byte writes cost 57 us more on a
  //    32,768-unit update. The wave reads back only what its own lanes wrote (a
  //    wave's LDS accesses complete in order), so no workgroup barrier is needed.
  if (rank > 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    TSK* Sku = sketch + ((size_t)seq * rt.total() + rt.offset(head)) * DV;
    const int c4 = wave * 32 + (lane & 7) * 4;
    for (int m = lane >> 3; m < rank; m += 8)
      store4(Sku + (size_t)m * DV + c4, *reinterpret_cast<const float4*>(lds + L::SK + m * DV + c4));
  }
}

}  // namespace ssm
