// stream_probe.hip -- in-place streaming of a state-sized buffer (read, scale by
// a runtime 1.0, write back) in two access shapes. It measures the HBM rate
// that the window update's read + write of S can reach on the device it runs
// on; it is a measurement aid beside the path, not a step of the method.
//
// The buffer is a sequence of 64 KB tiles (16384 floats, one 128 x 128 fp32
// state). Every lane moves 16 float4 per tile with non-temporal accesses, all
// loads before any store, as the update kernel does.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

namespace {

constexpr int kTileFloats = 16384;

// SHAPE 0, the update kernel's order: one 256-thread workgroup per tile seen as
//   128 rows x 128 columns; wave w holds columns 32w .. 32w + 31, lane group rg
//   the interleaved rows rg, rg + 8, ...; consecutive tiles go to one XCD.
// SHAPE 1, two tiles per 512-thread workgroup read as one flat 128 KB run: each
//   load instruction of the workgroup covers 8 KB contiguous; natural order.
template <int SHAPE>
__global__ void __launch_bounds__(SHAPE == 0 ? 256 : 512)
stream_inplace_kernel(float* __restrict__ a, float g) {
  const int tid = threadIdx.x;
  float* base;
  int off0, step;
  if constexpr (SHAPE == 0) {
    const int G = gridDim.x, xcd = blockIdx.x & 7, q8 = G >> 3, rem = G & 7;
    const int tile = xcd * q8 + min(xcd, rem) + (blockIdx.x >> 3);
    base = a + (size_t)tile * kTileFloats;
    const int lane = tid & 63, wave = tid >> 6, cg = lane & 7, rg = lane >> 3;
    off0 = rg * 128 + wave * 32 + cg * 4;  // row m * 8 + rg starts 1024 m floats later
    step = 8 * 128;
  } else {
    base = a + (size_t)blockIdx.x * (2 * kTileFloats);
    off0 = tid * 4;
    step = 512 * 4;
  }
  float4 s[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) s[m] = load_stream(base + off0 + m * step);
  asm volatile("" ::: "memory");  // every load before the first store
#pragma unroll
  for (int m = 0; m < 16; ++m) store_stream(base + off0 + m * step, scale4(g, s[m]));
}

}  // namespace

hipError_t launch_stream_probe(float* buf, long long n_tiles, int shape, hipStream_t stream) {
  if (shape == 0) {
    hipLaunchKernelGGL(stream_inplace_kernel<0>, dim3((unsigned)n_tiles), dim3(256), 0, stream,
                       buf, 1.0f);
  } else {
    hipLaunchKernelGGL(stream_inplace_kernel<1>, dim3((unsigned)(n_tiles / 2)), dim3(512), 0,
                       stream, buf, 1.0f);
  }
  return hipGetLastError();
}

}  // namespace ssm
