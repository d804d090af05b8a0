// fit_basis.hip -- the offline basis fit on the device: per head, the rank
// leading eigenvectors of the uncentred second moment of sampled queries,
// orthonormal, in decreasing order of eigenvalue. The SketchSSM pages fix the
// query basis offline (readsearch.ai listing of arXiv 2609.33051, Abstract;
// agihunt.info summary, "Mechanism details"); the top PCA directions of sampled
// queries, made orthonormal, are the recipe of the Mamba-2 workload.
//
// One workgroup per head, everything in LDS (up to 160 KB per workgroup on
// gfx950; 130 KB at d_k = 128):
//  1. M = X^T X / S on the matrix cores. The samples are staged transposed in
//     LDS, d_k / 2 at a time, and each wave accumulates its 16 x 16 tiles of M
//     with v_mfma_f32_16x16x4_f32 (A[i][k] from lane i + 16k, B[k][j] from lane
//     j + 16k, D[i][j] in lane j + 16 (i / 4), element i % 4). A tile's A and B
//     operands are both columns of the staged block, rows of M and its columns.
//  2. Cyclic Jacobi on M, V accumulating the rotations. A sweep visits every
//     pair (p, q) once, in d_k - 1 rounds of d_k / 2 disjoint pairs (the circle
//     schedule: index d_k - 1 stays, the others rotate). The rotations of one
//     round commute, so they are applied together: rows p, q of M, then columns
//     p, q of M and of V. A rotation is skipped when |m_pq| is negligible next to
//     sqrt(|m_pp m_qq|) (or to the largest diagonal entry, for null directions);
//     a sweep without rotations ends the iteration.
//  3. The rank largest diagonal entries pick columns of V. Two-pass Gram-Schmidt
//     makes them orthonormal in fp32, and each is signed so that its entry of
//     largest magnitude (the first on a tie) is positive.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

constexpr int kFitMaxSweeps = 40;
constexpr float kFitEps = 1.1920929e-7f;  // 2^-23

template <int DK>
constexpr int fit_ld() {
  return DK + 1;  // padded row stride: row and column walks both spread over the banks
}

// LDS floats: M [DK][LD] | V [DK][LD] | cos, sin [DK / 2] | flags [4] | chosen [32]
template <int DK>
constexpr size_t fit_lds_floats() {
  return 2 * (size_t)DK * fit_ld<DK>() + DK + 4 + 32;
}

// pair j of round r in the circle schedule, returned with p < q
template <int DK>
__device__ __forceinline__ void round_pair(int r, int j, int& p, int& q) {
  constexpr int M1 = DK - 1;
  const int a = (j == 0) ? r : (r + j) % M1;
  const int b = (j == 0) ? M1 : (r - j + M1) % M1;
  p = min(a, b);
  q = max(a, b);
}

template <int DK, typename TIN>
__global__ void __launch_bounds__(256)
fit_basis_kernel(const TIN* __restrict__ samples, int n_samples, int rank,
                 float* __restrict__ basis) {
  constexpr int LD = fit_ld<DK>();
  constexpr int NP = DK / 2;              // pairs per round
  constexpr int SB = DK / 2;              // samples per staged block
  constexpr int SLD = SB + 1;
  constexpr int NTL = DK / 16;            // 16 x 16 tiles per side of M
  constexpr int TPW = (NTL * NTL + 3) / 4;  // tiles per wave
  constexpr int VIN = 16 / sizeof(TIN);
  constexpr int EPL = (DK + 63) / 64;     // vector entries per lane in step 3

  extern __shared__ float4 lds4[];
  float* M = reinterpret_cast<float*>(lds4);
  float* V = M + DK * LD;
  float* Qt = V;  // staging during step 1: [DK][SLD] fits in V's [DK][LD]
  float* pc = V + DK * LD;
  float* ps = pc + NP;
  int* flag = reinterpret_cast<int*>(ps + NP);  // [0], [1]: rotations seen; [2]: max diag
  int* chosen = flag + 4;

  const int head = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- 1. M = X^T X / S ----
  const TIN* X = samples + (size_t)head * n_samples * DK;
  v4f acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_samples; s0 += SB) {
    for (int e = tid * VIN; e < SB * DK; e += 256 * VIN) {
      const int s = e / DK, d = e % DK;
      float f[VIN];
      if (s0 + s < n_samples) {
        Packed<TIN, VIN> x;
        x.load(X + (size_t)(s0 + s) * DK + d);
        x.unpack(f);
      } else {
#pragma unroll
        for (int j = 0; j < VIN; ++j) f[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < VIN; ++j) Qt[(d + j) * SLD + s] = f[j];
    }
    __syncthreads();
    const int i = lane & 15, kk = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < SB; k0 += 4) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int tile = wave + 4 * t;
        if (tile < NTL * NTL) {  // uniform per wave
          const int ti = tile / NTL, tj = tile % NTL;
          const float a = Qt[(ti * 16 + i) * SLD + k0 + kk];
          const float b = Qt[(tj * 16 + i) * SLD + k0 + kk];
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  const float inv_s = 1.f / (float)n_samples;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + 4 * t;
    if (tile < NTL * NTL) {
      const int ti = tile / NTL, tj = tile % NTL;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        M[(ti * 16 + 4 * (lane >> 4) + e) * LD + tj * 16 + (lane & 15)] = acc[t][e] * inv_s;
    }
  }
  __syncthreads();  // M complete; the staging block is no longer read
  for (int e = tid; e < DK * DK; e += 256) V[(e / DK) * LD + e % DK] = (e / DK == e % DK) ? 1.f : 0.f;
  if (tid == 0) {
    float mx = 0.f;
    for (int i = 0; i < DK; ++i) mx = fmaxf(mx, fabsf(M[i * LD + i]));
    flag[0] = 0;
    flag[1] = 0;
    flag[2] = __float_as_int(mx);
  }
  __syncthreads();

  // ---- 2. cyclic Jacobi ----
  const float floor_abs = kFitEps * kFitEps * __int_as_float(flag[2]);
  for (int sweep = 0; sweep < kFitMaxSweeps; ++sweep) {
    int* rotated = flag + (sweep & 1);
    for (int r = 0; r < DK - 1; ++r) {
      if (tid < NP) {
        int p, q;
        round_pair<DK>(r, tid, p, q);
        const float app = M[p * LD + p], aqq = M[q * LD + q], apq = M[p * LD + q];
        float c = 1.f, s = 0.f;
        if (fabsf(apq) > kFitEps * fmaxf(sqrtf(fabsf(app)) * sqrtf(fabsf(aqq)), floor_abs)) {
          const float theta = (aqq - app) / (2.f * apq);
          // t = sign(theta) / (|theta| + sqrt(theta^2 + 1)), the smaller root of
          // t^2 + 2 theta t - 1 = 0; 1 / (2 theta) where theta^2 would overflow
          const float at = fabsf(theta);
          const float t = copysignf(at > 1e18f ? 0.5f / at : 1.f / (at + sqrtf(fmaf(at, at, 1.f))), theta);
          c = 1.f / sqrtf(fmaf(t, t, 1.f));
          s = t * c;
          *rotated = 1;  // every writer stores the same value
        }
        pc[tid] = c;
        ps[tid] = s;
      }
      __syncthreads();
      for (int e = tid; e < NP * DK; e += 256) {  // rows p, q of M
        const int j = e / DK, k = e % DK;
        const float s = ps[j];
        if (s != 0.f) {
          int p, q;
          round_pair<DK>(r, j, p, q);
          const float c = pc[j];
          const float x = M[p * LD + k], y = M[q * LD + k];
          M[p * LD + k] = c * x - s * y;
          M[q * LD + k] = s * x + c * y;
        }
      }
      __syncthreads();
      for (int e = tid; e < NP * DK; e += 256) {  // columns p, q of M and V
        const int j = e / DK, k = e % DK;
        const float s = ps[j];
        if (s != 0.f) {
          int p, q;
          round_pair<DK>(r, j, p, q);
          const float c = pc[j];
          float x = M[k * LD + p], y = M[k * LD + q];
          M[k * LD + p] = c * x - s * y;
          M[k * LD + q] = s * x + c * y;
          x = V[k * LD + p];
          y = V[k * LD + q];
          V[k * LD + p] = c * x - s * y;
          V[k * LD + q] = s * x + c * y;
        }
      }
      __syncthreads();
    }
    const int any = *rotated;
    __syncthreads();  // every thread has read the flag before it is cleared for sweep + 2
    if (tid == 0) *rotated = 0;
    if (!any) break;  // uniform
  }

  // ---- 3. the rank largest eigenvalues, orthonormal rows, sign rule ----
  if (tid == 0) {
    uint32_t used[4] = {0u, 0u, 0u, 0u};
    for (int m = 0; m < rank; ++m) {
      int best = -1;
      float bv = 0.f;
      for (int i = 0; i < DK; ++i) {
        if ((used[i >> 5] >> (i & 31)) & 1u) continue;
        const float v = M[i * LD + i];
        if (best < 0 || v > bv) {
          best = i;
          bv = v;
        }
      }
      used[best >> 5] |= 1u << (best & 31);
      chosen[m] = best;
    }
  }
  __syncthreads();
  float* B = M;  // [rank][LD]: M is not read any more
  if (wave == 0) {
    auto wsum = [](float x) { return group_allreduce<64>(x); };
    for (int m = 0; m < rank; ++m) {
      float x[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int i = lane + 64 * e;
        x[e] = i < DK ? V[i * LD + chosen[m]] : 0.f;
      }
      for (int pass = 0; pass < 2; ++pass) {
        for (int p = 0; p < m; ++p) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            if (lane + 64 * e < DK) a = fmaf(x[e], B[p * LD + lane + 64 * e], a);
          const float dp = wsum(a);
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            if (lane + 64 * e < DK) x[e] = fmaf(-dp, B[p * LD + lane + 64 * e], x[e]);
        }
      }
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = fmaf(x[e], x[e], a);
      const float n2 = wsum(a);
      const float scale = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
      // entry of largest magnitude, the lowest index on a tie
      float bv = -1.f;
      int bi = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int i = lane + 64 * e;
        if (i < DK && fabsf(x[e]) > bv) {
          bv = fabsf(x[e]);
          bi = i;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      float big = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float v = __shfl(x[e], bi & 63);
        if ((bi >> 6) == e) big = v;
      }
      const float sg = big < 0.f ? -scale : scale;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if (lane + 64 * e < DK) B[m * LD + lane + 64 * e] = x[e] * sg;
    }
  }
  __syncthreads();
  float* out = basis + (size_t)head * rank * DK;
  for (int e = tid; e < rank * DK; e += 256) out[e] = B[(e / DK) * LD + e % DK];
}

template <int DK, typename TIN>
hipError_t launch_fit(const void* samples, int n_samples, int heads, int rank, float* basis,
                      hipStream_t stream) {
  constexpr size_t lds = fit_lds_floats<DK>() * sizeof(float);
  auto kern = fit_basis_kernel<DK, TIN>;
  // on every call (a setup-time launch), so it holds on whichever device is current
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(256), lds, stream, static_cast<const TIN*>(samples),
                     n_samples, rank, basis);
  return hipGetLastError();
}

}  // namespace

size_t fit_basis_lds_bytes(int dk) {
  switch (dk) {
    case 16: return fit_lds_floats<16>() * sizeof(float);
    case 32: return fit_lds_floats<32>() * sizeof(float);
    case 64: return fit_lds_floats<64>() * sizeof(float);
    case 128: return fit_lds_floats<128>() * sizeof(float);
  }
  return 0;
}

hipError_t launch_fit_basis(const ssm_dims& d, const void* samples, int n_samples, float* basis,
                            hipStream_t stream) {
  return dispatch_shape(d.in_dtype, d.d_k, 32, [&](auto DK, auto, auto T) {
    using TIN = typename decltype(T)::type;
    return launch_fit<decltype(DK)::value, TIN>(samples, n_samples, d.heads, d.rank, basis, stream);
  });
}

}  // namespace ssm
