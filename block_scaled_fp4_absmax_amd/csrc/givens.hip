// givens.hip -- the inter-block transform on every row: permutation, then
// layers of disjoint Givens rotations of channel pairs ("TORQ: Two-Level
// Orthogonal Rotation for MXFP4 Quantization", technical summary sec. 2(a):
// an orthogonal transform built from Givens rotations that evens out the
// block variances). The same call folds the transform into the rows of a
// consumer's weight matrix.
#include <algorithm>

#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {
namespace {

__device__ __forceinline__ int clamp_index(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// A work-group takes rows blockIdx.x, blockIdx.x + gridDim.x, ... The row is
// read with 16-byte loads (into LDS as bf16 when it is then gathered through
// the permutation), widened to an fp32 LDS row, rotated layer by layer (the
// pairs of a layer are disjoint: one thread per pair, a barrier between
// layers), and written back as bf16 (RNE) with 16-byte stores. Every index
// read from memory is clamped into the row.
__global__ __launch_bounds__(kThreads) void givens_rows_kernel(
    const uint16_t* x, int64_t ld_x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ pairs, const float* __restrict__ cs,
    const int32_t* __restrict__ layer_start, int n_layers, int n_rot, uint16_t* out,
    int64_t ld_out, int64_t rows, int cols) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* z = reinterpret_cast<float*>(smem);                           // cols fp32
  uint16_t* raw = reinterpret_cast<uint16_t*>(smem + 4 * (size_t)cols);  // cols bf16
  const int chunks = cols / 8;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + r * ld_x);
    if (perm) {
      for (int c = threadIdx.x; c < chunks; c += kThreads)
        reinterpret_cast<u32x4_t*>(raw)[c] = __builtin_nontemporal_load(src + c);
      __syncthreads();
      for (int j = threadIdx.x; j < cols; j += kThreads)
        z[j] = __uint_as_float((uint32_t)raw[clamp_index(perm[j], cols)] << 16);
    } else {
      for (int c = threadIdx.x; c < chunks; c += kThreads) {
        const u32x4_t v = __builtin_nontemporal_load(src + c);
        f32x4_t lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = __uint_as_float(e & 1 ? (v[e / 2] & 0xFFFF0000u) : (v[e / 2] << 16));
          hi[e] = __uint_as_float(e & 1 ? (v[2 + e / 2] & 0xFFFF0000u) : (v[2 + e / 2] << 16));
        }
        reinterpret_cast<f32x4_t*>(z)[2 * c] = lo;
        reinterpret_cast<f32x4_t*>(z)[2 * c + 1] = hi;
      }
    }
    __syncthreads();
    for (int L = 0; L < n_layers; ++L) {
      const int k0 = min(max(layer_start[L], 0), n_rot);
      const int k1 = min(max(layer_start[L + 1], k0), n_rot);
      for (int k = k0 + (int)threadIdx.x; k < k1; k += kThreads) {
        const int i = clamp_index(pairs[2 * k], cols), j = clamp_index(pairs[2 * k + 1], cols);
        const float c = cs[2 * k], s = cs[2 * k + 1];
        const float zi = z[i], zj = z[j];
        z[i] = c * zi - s * zj;
        z[j] = s * zi + c * zj;
      }
      __syncthreads();
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + r * ld_out);
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
      const f32x4_t lo = reinterpret_cast<const f32x4_t*>(z)[2 * c];
      const f32x4_t hi = reinterpret_cast<const f32x4_t*>(z)[2 * c + 1];
      const u32x4_t w = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                         pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
      __builtin_nontemporal_store(w, dst + c);
    }
    __syncthreads();  // the LDS rows are reused by the next row
  }
}

}  // namespace

void launch_givens_rows(int64_t rows, int64_t cols, const void* x, int64_t ld_x,
                        const int32_t* perm, const int32_t* pairs, const float* cs,
                        const int32_t* layer_start, int n_layers, int n_rot, void* out,
                        int64_t ld_out, hipStream_t st) {
  const DeviceInfo di = device_info();
  const size_t lds = 6 * (size_t)cols;
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(8, (size_t)di.lds / (lds + 1024)));
  const int64_t wgs = (int64_t)di.cus * per_cu;
  const int grid = (int)(rows < wgs ? rows : wgs);
  hipLaunchKernelGGL(givens_rows_kernel, dim3(grid), dim3(kThreads), lds, st,
                     static_cast<const uint16_t*>(x), ld_x, perm, pairs, cs, layer_start,
                     n_layers, n_rot, static_cast<uint16_t*>(out), ld_out, rows, (int)cols);
}

}  // namespace fp4
