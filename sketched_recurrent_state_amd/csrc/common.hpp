// common.hpp -- device helpers shared by the SketchSSM kernels (gfx950 only).
//
// Lane layouts used by the kernels:
//  * state tile ("tile", TileLayout): one workgroup per (sequence, head) unit,
//    one wave per 32-column block of the d_k x d_v state (one wave for d_v =
//    16). Lane l owns 4 adjacent columns (column group cg = l % CG, one 128-bit
//    load per row) of d_k/RG rows (row group rg = l / CG). CG = 8 for d_v >= 32:
//    8 lanes cover a 128-byte line, RG = 8; CG = 4 for d_v = 16: 4 lanes cover
//    the 64-byte row, RG = 16. Rows are contiguous per lane (rg*d_k/RG ...) in
//    the read kernels and interleaved (rg, rg + RG, ...) in the window update,
//    whose waves then cover RG whole rows of contiguous memory per load
//    instruction. A reduction over d_k is a sum over the RG lanes that share cg,
//    i.e. over lane bits 3, 4 and 5 (and 2 when CG = 4): DPP row_ror:8 for bit
//    3, the gfx950 permlane16/permlane32 swaps for bits 4 and 5, and for bit 2
//    a row_half_mirror followed by a quad_perm reversal (lane l ^ 4).
//  * group: G = 16 or 32 consecutive lanes per unit, each holding d_k/G key
//    elements and d_v/G value elements; reductions are DPP row operations plus,
//    for G = 32, one permlane16 swap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

enum Rule { MAMBA2 = 0, GDN = 1, KDA = 2 };

typedef uint16_t bf16_t;  // bf16 bit pattern

// ---------------------------------------------------------------------------
// input loads: E consecutive elements of T -> float
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 bits (a in the low half), rounded to nearest with
// ties to even: one gfx950 v_cvt_pk_bf16_f32 under the default rounding mode.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Four floats stored at p as fp32 (16 bytes) or bf16 (8 bytes).
__device__ __forceinline__ void store4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ void store4(uint16_t* p, float4 x) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
}

template <typename T, int E>
struct Vec;

template <int E>
struct Vec<float, E> {
  static __device__ __forceinline__ void load(const float* __restrict__ p, float* out) {
    if constexpr (E % 4 == 0) {
#pragma unroll
      for (int i = 0; i < E; i += 4) {
        float4 x = *reinterpret_cast<const float4*>(p + i);
        out[i] = x.x; out[i + 1] = x.y; out[i + 2] = x.z; out[i + 3] = x.w;
      }
    } else if constexpr (E == 2) {
      float2 x = *reinterpret_cast<const float2*>(p);
      out[0] = x.x; out[1] = x.y;
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) out[i] = p[i];
    }
  }
  static __device__ __forceinline__ void store(float* __restrict__ p, const float* in) {
    if constexpr (E % 4 == 0) {
#pragma unroll
      for (int i = 0; i < E; i += 4)
        *reinterpret_cast<float4*>(p + i) = make_float4(in[i], in[i + 1], in[i + 2], in[i + 3]);
    } else if constexpr (E == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(in[0], in[1]);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) p[i] = in[i];
    }
  }
  static __device__ __forceinline__ void copy(const float* __restrict__ src, float* __restrict__ dst) {
    if constexpr (E % 4 == 0) {
#pragma unroll
      for (int i = 0; i < E; i += 4)
        *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(src + i);
    } else if constexpr (E == 2) {
      *reinterpret_cast<float2*>(dst) = *reinterpret_cast<const float2*>(src);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) dst[i] = src[i];
    }
  }
};

template <int E>
struct Vec<bf16_t, E> {
  static __device__ __forceinline__ void load(const bf16_t* __restrict__ p, float* out) {
    if constexpr (E % 8 == 0) {
#pragma unroll
      for (int i = 0; i < E; i += 8) {
        uint4 x = *reinterpret_cast<const uint4*>(p + i);
        out[i + 0] = bf16_lo(x.x); out[i + 1] = bf16_hi(x.x);
        out[i + 2] = bf16_lo(x.y); out[i + 3] = bf16_hi(x.y);
        out[i + 4] = bf16_lo(x.z); out[i + 5] = bf16_hi(x.z);
        out[i + 6] = bf16_lo(x.w); out[i + 7] = bf16_hi(x.w);
      }
    } else if constexpr (E == 4) {
      uint2 x = *reinterpret_cast<const uint2*>(p);
      out[0] = bf16_lo(x.x); out[1] = bf16_hi(x.x);
      out[2] = bf16_lo(x.y); out[3] = bf16_hi(x.y);
    } else if constexpr (E == 2) {
      uint32_t x = *reinterpret_cast<const uint32_t*>(p);
      out[0] = bf16_lo(x); out[1] = bf16_hi(x);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) out[i] = __uint_as_float(uint32_t(p[i]) << 16);
    }
  }
  static __device__ __forceinline__ void copy(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst) {
    if constexpr (E % 8 == 0) {
#pragma unroll
      for (int i = 0; i < E; i += 8)
        *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
    } else if constexpr (E == 4) {
      *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
    } else if constexpr (E == 2) {
      *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) dst[i] = src[i];
    }
  }
};

// E elements of T held as raw 32-bit words (bf16 stays packed two per word)
// from the load until unpack(): halves the registers of in-flight bf16 data.
template <typename T, int E>
struct Packed {
  static constexpr int BYTES = E * (int)sizeof(T);
  static constexpr int NW = (BYTES + 3) / 4;
  uint32_t w[NW];

  __device__ __forceinline__ void load(const T* __restrict__ p) {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i) {
        uint4 x = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
      }
    } else if constexpr (BYTES == 8) {
      uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x; w[1] = x.y;
    } else if constexpr (BYTES == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      static_assert(BYTES == 2, "unsupported width");
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  }
  __device__ __forceinline__ void store(T* __restrict__ p) const {
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
      for (int i = 0; i < BYTES / 16; ++i)
        reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else if constexpr (BYTES == 8) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (BYTES == 4) {
      *reinterpret_cast<uint32_t*>(p) = w[0];
    } else {
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)w[0];
    }
  }
  __device__ __forceinline__ void unpack(float* out) const {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if constexpr (sizeof(T) == 4) {
        out[i] = __uint_as_float(w[i]);
      } else {
        out[i] = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// cross-lane primitives
// ---------------------------------------------------------------------------
// DPP controls (GCN/CDNA encoding)
constexpr int DPP_QUAD_1032 = 0xB1;  // quad_perm:[1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;  // quad_perm:[2,3,0,1]
constexpr int DPP_ROR4 = 0x124;      // row_ror:4
constexpr int DPP_ROR8 = 0x128;      // row_ror:8
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror: lane p <-> 7 - p in each 8 lanes
constexpr int DPP_QUAD_3210 = 0x1B;   // quad_perm:[3,2,1,0]

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// a + (the same register of lane l ^ 16): permlane16_swap exchanges odd rows of
// the first operand with even rows of the second; summing both results gives
// every lane the pair sum.
__device__ __forceinline__ float xsum16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// a + (the same register of lane l ^ 32), via permlane32_swap.
__device__ __forceinline__ float xsum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Halving exchange over lane bit 4: afterwards lanes with bit 4 clear hold
// lo + partner's lo, lanes with bit 4 set hold hi + partner's hi (in `lo`).
__device__ __forceinline__ void halve16(float& lo, float hi) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same over lane bit 5.
__device__ __forceinline__ void halve32(float& lo, float hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same over lane bit 3 (inside a 16-lane row): row_ror:8 reaches lane l ^ 8.
__device__ __forceinline__ float halve8(float lo, float hi, bool upper) {
  float keep = upper ? hi : lo;
  float send = upper ? lo : hi;
  return keep + dpp<DPP_ROR8>(send);
}

// Lane k's value of x, in every lane (two v_readlane_b32; k must be uniform).
__device__ __forceinline__ double readlane_f64(double x, int k) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, k);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), k);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / sqrt(d) for d > 0: the hardware estimate (v_rsq_f64) and two Newton steps
// y <- y (3 - d y^2) / 2, each of which doubles the correct bits.
__device__ __forceinline__ double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  const double h = 0.5 * d;
  y = y * fma(-h, y * y, 1.5);
  y = y * fma(-h, y * y, 1.5);
  return y;
}

// The value of lane l ^ 4: reversing each 8 lanes (p -> 7 - p) and then each 4
// (p -> 3 - p) maps position p to p ^ 4.
__device__ __forceinline__ float xor4(float x) {
  return dpp<DPP_QUAD_3210>(dpp<DPP_HALF_MIRROR>(x));
}

// The state tile for d_k x d_v (see the top of this file): column groups per wave,
// row groups, rows per lane, waves and threads per unit.
template <int DK, int DV>
struct TileLayout {
  static constexpr int CG = DV >= 32 ? 8 : 4;
  static constexpr int RG = 64 / CG;
  static constexpr int RPL = DK / RG;
  static constexpr int WAVES = DV / (4 * CG);
  static constexpr int NT = 64 * WAVES;
  static_assert(RPL >= 1 && WAVES >= 1, "tile shape");
};

// Sum over the 8 lanes that differ in bits 3..5 (the tile layout's d_k split).
__device__ __forceinline__ float tile_allreduce(float x) {
  x += dpp<DPP_ROR8>(x);
  x = xsum16(x);
  return xsum32(x);
}

// The same for four values: a reduce-scatter leaves each lane the sum of one of them
// (halvings over bits 5 and 4, then the pair over bit 3), and an all-gather returns
// all four. A swap's two results are, in every lane, the value of its lower and of
// its upper lane half, so the gathered columns come back in order without selects:
// ten cross-lane steps instead of four separate all-reduces.
__device__ __forceinline__ float4 tile_allreduce(float4 v) {
  float xz = v.x, yw = v.y;
  halve32(xz, v.z);           // bit 5 clear: x, set: z (summed over the bit-5 pair)
  halve32(yw, v.w);           // bit 5 clear: y, set: w
  halve16(xz, yw);            // bit 4 clear: x or z, set: y or w
  xz += dpp<DPP_ROR8>(xz);    // the bit-3 pair: this lane's value summed over all 8 lanes
  const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(xz), __float_as_uint(xz),
                                                  false, false);  // [0] x or z, [1] y or w
  const auto a = __builtin_amdgcn_permlane32_swap(h[0], h[0], false, false);  // [0] x, [1] z
  const auto b = __builtin_amdgcn_permlane32_swap(h[1], h[1], false, false);  // [0] y, [1] w
  return make_float4(__uint_as_float(a[0]), __uint_as_float(b[0]), __uint_as_float(a[1]),
                     __uint_as_float(b[1]));
}

// Sum over the lanes of a tile that share this lane's column group (all RG row
// groups): lane bits 3..5, and bit 2 first when a wave holds 4 column groups.
template <int CG>
__device__ __forceinline__ float tile_sum(float x) {
  if constexpr (CG == 4) x += xor4(x);
  return tile_allreduce(x);
}

template <int CG>
__device__ __forceinline__ float4 tile_sum(float4 v) {
  if constexpr (CG == 4) {
    v.x += xor4(v.x);
    v.y += xor4(v.y);
    v.z += xor4(v.z);
    v.w += xor4(v.w);
  }
  return tile_allreduce(v);
}

// Sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_allreduce(float x) {
  x += dpp<DPP_QUAD_1032>(x);
  x += dpp<DPP_QUAD_2301>(x);
  x += dpp<DPP_ROR4>(x);
  x += dpp<DPP_ROR8>(x);
  return x;
}

// Sum over an aligned group of G consecutive lanes (G = 16, 32 or 64).
template <int G>
__device__ __forceinline__ float group_allreduce(float x) {
  static_assert(G == 16 || G == 32 || G == 64, "group size");
  x = row_allreduce(x);
  if constexpr (G >= 32) x = xsum16(x);
  if constexpr (G >= 64) x = xsum32(x);
  return x;
}

// ---------------------------------------------------------------------------
// streaming (non-temporal) 128-bit accesses: for data touched once per window
// (the full state), so it does not push the sketch and the window buffer,
// which every step re-reads, out of the caches.
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float* p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(float* p, float4 x) {
  v4f v;
  v.x = x.x; v.y = x.y; v.z = x.z; v.w = x.w;
  __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

// ---------------------------------------------------------------------------
// float4 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 f4(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 sub4(float4 a, float4 b) {
  return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 scale4(float a, float4 b) {
  return make_float4(a * b.x, a * b.y, a * b.z, a * b.w);
}
// a * b + c, componentwise with scalar a
__device__ __forceinline__ float4 fma4(float a, float4 b, float4 c) {
  return make_float4(fmaf(a, b.x, c.x), fmaf(a, b.y, c.y), fmaf(a, b.z, c.z), fmaf(a, b.w, c.w));
}

// ---------------------------------------------------------------------------
// sketch rank per head. Basis rows of head h: [offset(h), offset(h) + rank(h));
// the sketch of sequence n holds total() rows, head h's at the same offsets.
// ---------------------------------------------------------------------------
struct UniformRank {  // every head has rank r
  int r, heads;
  __device__ __forceinline__ int rank(int) const { return r; }
  __device__ __forceinline__ int offset(int h) const { return h * r; }
  __device__ __forceinline__ int total() const { return heads * r; }
};

constexpr int kMaxRankedHeads = 256;

struct RankTable {  // per-head ranks: off[h + 1] - off[h], off[0] = 0 (checked on the host)
  int heads;
  int off[kMaxRankedHeads + 1];
  // The heads by rank, largest first (ties by index): the order in which the sketch read
  // deals its blocks out, so that each round of resident workgroups holds one rank class
  // and every compute unit receives a mix of ranks (heads of equal rank on one unit would
  // make it the slowest).
  uint8_t order[kMaxRankedHeads];
  __device__ __forceinline__ int rank(int h) const { return off[h + 1] - off[h]; }
  __device__ __forceinline__ int offset(int h) const { return off[h]; }
  __device__ __forceinline__ int total() const { return off[heads]; }
};

// ---------------------------------------------------------------------------
// batch rows -> persistent slots and window positions. Per-step arrays (q, the
// current token, y) are indexed by the batch row; the state, the sketch and the
// window buffer by the row's slot.
// ---------------------------------------------------------------------------
struct Lockstep {  // row n is slot n; every row holds `count` tokens (tau, or n_tokens)
  int count;
  __device__ __forceinline__ bool row(int n, int& slot, int& cnt) const {
    slot = n;
    cnt = count;
    return true;
  }
};

struct Varlen {  // per-row slot (identity if null) and token count; rows out of range are skipped
  const int32_t* slot;
  const int32_t* count;
  int num_slots, lo, hi;  // a row is served when lo <= count <= hi and 0 <= slot < num_slots
  __device__ __forceinline__ bool row(int n, int& s, int& cnt) const {
    s = slot ? slot[n] : n;
    cnt = count[n];
    return s >= 0 && s < num_slots && cnt >= lo && cnt <= hi;
  }
};

// ---------------------------------------------------------------------------
// window staging: the first n buffered tokens of one unit -> LDS as fp32
// ---------------------------------------------------------------------------
__host__ __device__ inline int pad4(int x) { return (x + 3) & ~3; }

// One unit's window buffer (slot 0 of each array) and, for a fused append, its
// current token (kt == nullptr: not fused, the buffers are only read).
template <typename TIN>
struct UnitWindow {
  TIN* k;
  TIN* v;
  float* d;
  float* b;
  const TIN* kt;
  const TIN* vt;
  const float* dt;
  const float* bt;
};

// LDS floats needed for n staged tokens: k [n][DK] | v [n][DV] | gates | beta.
template <int RULE, int DK, int DV>
__host__ __device__ inline int window_lds_floats(int n) {
  constexpr int DSTR = (RULE == KDA) ? DK : 1;
  return n * DK + n * DV + pad4(n * DSTR) + ((RULE == MAMBA2) ? 0 : pad4(n));
}

// Position in LDS of d_k index i for the interleaved row layout (row group g
// of RG owns rows g, g + RG, g + 2 RG, ...): group g's d_k / RG values are
// stored contiguously so each lane reads them with vector loads.
template <int DK, int RG = 8>
__host__ __device__ __forceinline__ int interleaved_pos(int i) {
  return (i % RG) * (DK / RG) + i / RG;
}

// Cooperative copy by the NT threads of a workgroup, in two phases so that a
// caller can issue other loads in between: issue() starts every thread's first
// chunk of each array (keys, values, gates, beta), so the whole window costs one
// memory round trip; commit() writes those chunks to LDS and copies any further
// ones (windows longer than one chunk per thread) directly. Loads are clamped
// into the window, so every lane issues the same instructions (the wait counts
// stay exact); only lanes in range store. With a fused append the newest slot
// (n - 1) is read from the current token and also written into the buffer. With
// PERM the d_k-indexed rows (keys, and KDA's per-row gates) are stored in
// interleaved_pos order (RG row groups). Requires n >= 1; the caller synchronises
// the workgroup before reading the LDS.
template <int RULE, int DK, int DV, typename TIN, int NT, bool PERM = false, int RG = 8>
struct WindowStage {
  static constexpr int DSTR = (RULE == KDA) ? DK : 1;
  static constexpr int VIN = 16 / sizeof(TIN);       // input elements per chunk
  static constexpr int VG = (RULE == KDA) ? 4 : 1;   // gate elements per chunk
  Packed<TIN, VIN> k0, v0;
  float g0[VG];
  float b0 = 0.f;

  // source of the chunk at element e of a [n][len] array: the buffer, or the
  // current token for the newest slot of a fused append
  template <typename T>
  static __device__ __forceinline__ const T* src(const T* buf, const T* cur, int e, int len,
                                                 int last, bool fused) {
    return (fused && e / len == last) ? cur + (e - last * len) : buf + e;
  }

  __device__ __forceinline__ void issue(const UnitWindow<TIN>& uw, int n, int tid) {
    const bool fused = uw.kt != nullptr;
    const int last = n - 1;
    k0.load(src<TIN>(uw.k, uw.kt, min(tid * VIN, n * DK - VIN), DK, last, fused));
    v0.load(src<TIN>(uw.v, uw.vt, min(tid * VIN, n * DV - VIN), DV, last, fused));
    Vec<float, VG>::load(src<float>(uw.d, uw.dt, min(tid * VG, n * DSTR - VG), DSTR, last, fused),
                         g0);
    if constexpr (RULE != MAMBA2) b0 = *src<float>(uw.b, uw.bt, min(tid, last), 1, last, fused);
  }

  __device__ __forceinline__ void commit(float* lds, const UnitWindow<TIN>& uw, int n,
                                         int tid) const {
    float* lk = lds;
    float* lv = lk + n * DK;
    float* ld = lv + n * DV;
    float* lb = ld + pad4(n * DSTR);
    const bool fused = uw.kt != nullptr;
    const int last = n - 1;
    auto put_k = [&](const Packed<TIN, VIN>& x, int e) {
      if (fused && e / DK == last) x.store(uw.k + e);
      float f[VIN];
      x.unpack(f);
      if constexpr (PERM) {
        const int t0 = e - e % DK, i0 = e % DK;
#pragma unroll
        for (int j = 0; j < VIN; ++j) lk[t0 + interleaved_pos<DK, RG>(i0 + j)] = f[j];
      } else {
        Vec<float, VIN>::store(lk + e, f);
      }
    };
    auto put_v = [&](const Packed<TIN, VIN>& x, int e) {
      if (fused && e / DV == last) x.store(uw.v + e);
      float f[VIN];
      x.unpack(f);
      Vec<float, VIN>::store(lv + e, f);
    };
    auto put_g = [&](const float* g, int e) {
      if (fused && e / DSTR == last) Vec<float, VG>::store(uw.d + e, g);
      if constexpr (PERM && RULE == KDA) {
        const int t0 = e - e % DK, i0 = e % DK;
#pragma unroll
        for (int j = 0; j < VG; ++j) ld[t0 + interleaved_pos<DK, RG>(i0 + j)] = g[j];
      } else {
        Vec<float, VG>::store(ld + e, g);
      }
    };
    auto put_b = [&](float x, int e) {
      if (fused && e == last) uw.b[e] = x;
      lb[e] = x;
    };
    // the chunks issue() fetched
    if (tid * VIN < n * DK) put_k(k0, tid * VIN);
    if (tid * VIN < n * DV) put_v(v0, tid * VIN);
    if (tid * VG < n * DSTR) put_g(g0, tid * VG);
    if constexpr (RULE != MAMBA2) {
      if (tid < n) put_b(b0, tid);
    }
    // the rest, for windows longer than one chunk per thread
    for (int e = (tid + NT) * VIN; e < n * DK; e += NT * VIN) {
      Packed<TIN, VIN> x;
      x.load(src<TIN>(uw.k, uw.kt, e, DK, last, fused));
      put_k(x, e);
    }
    for (int e = (tid + NT) * VIN; e < n * DV; e += NT * VIN) {
      Packed<TIN, VIN> x;
      x.load(src<TIN>(uw.v, uw.vt, e, DV, last, fused));
      put_v(x, e);
    }
    for (int e = (tid + NT) * VG; e < n * DSTR; e += NT * VG) {
      float g[VG];
      Vec<float, VG>::load(src<float>(uw.d, uw.dt, e, DSTR, last, fused), g);
      put_g(g, e);
    }
    if constexpr (RULE != MAMBA2) {
      for (int e = tid + NT; e < n; e += NT) put_b(*src<float>(uw.b, uw.bt, e, 1, last, fused), e);
    }
  }
};

}  // namespace ssm
