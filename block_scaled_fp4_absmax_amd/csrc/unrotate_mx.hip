// unrotate_mx.hip -- MXFP4 dequantization with the inverse rotation (kernel in
// unrotate_kernels.hpp), and the channel-energy statistic that calibrates the
// permutation ("TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
// technical summary sec. 2(a): the permutation balances the energy of the
// blocks, measured here per channel over the calibration rows).
#include "unrotate_kernels.hpp"

namespace fp4 {

void launch_mx_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard, bool mxint,
                                const void* codes, const void* scales, void* out, hipStream_t st) {
  auto c = static_cast<const uint8_t*>(codes);
  auto sc = static_cast<const uint8_t*>(scales);
  auto o = static_cast<uint16_t*>(out);
  const RotGeom g = rot_geom(s, 0);
  if (mxint) mxint_dequant_unrotate(s, perm, hadamard != 0, c, sc, o, g, st);
  else unrot_variants<0, false>(s, perm, hadamard != 0, c, sc, nullptr, o, g, st);
}

// ============================== channel energy ==============================
// One work-group per 32-column slice; lane (q, rg) = (t & 3, t >> 2) adds the
// squares of chunk q of rows rg, rg + 64, ... in fp64; the 64 partial sums of
// each column are then added in row-group order, so the result does not
// depend on scheduling.
__global__ __launch_bounds__(kThreads) void channel_energy_kernel(const uint16_t* __restrict__ x,
                                                                  float* __restrict__ energy,
                                                                  int64_t rows, int64_t ld_x) {
  __shared__ double part[kThreads / 4][33];
  const int q = threadIdx.x & 3, rg = threadIdx.x >> 2;
  const int64_t col0 = 32 * (int64_t)blockIdx.x + 8 * q;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = rg; r < rows; r += kThreads / 4) {
    u32x4_t d = *reinterpret_cast<const u32x4_t*>(x + r * ld_x + col0);
    float v[8];
    widen8(d, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += (double)v[k] * (double)v[k];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[rg][8 * q + k] = acc[k];
  __syncthreads();
  if (threadIdx.x < 32) {
    double s = 0.0;
    for (int i = 0; i < kThreads / 4; ++i) s += part[i][threadIdx.x];
    energy[32 * (int64_t)blockIdx.x + threadIdx.x] = (float)s;
  }
}

void launch_channel_energy(int64_t rows, int64_t cols, int64_t ld_x, const void* x, float* energy,
                           hipStream_t st) {
  hipLaunchKernelGGL(channel_energy_kernel, dim3((int)(cols / 32)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), energy, rows, ld_x);
}

}  // namespace fp4
