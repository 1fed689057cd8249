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

// Chunks of 8 bf16 (16 bytes) per thread: cols <= 16384 is 2048 chunks; and
// columns per thread.
constexpr int kMaxChunksPerThread = 2048 / kThreads;
constexpr int kMaxColsPerThread = 16384 / kThreads;

// Rotation tables staged in LDS: (i | j << 16) and (cos, sin) per rotation,
// then the layer starts.
struct Tables {
  uint32_t* ij;
  float2_t* cs;
  int32_t* ls;
};

// A work-group takes rows blockIdx.x, blockIdx.x + gridDim.x, ... The row is
// read with 16-byte loads (the next row's loads are issued before the current
// row is rotated, so they are in flight meanwhile), put in LDS (as bf16 when
// it is then gathered through the permutation), widened to an fp32 LDS row,
// rotated layer by layer (the pairs of a layer are disjoint: one thread per
// pair, a barrier between layers), and written back as bf16 (RNE) with
// 16-byte stores. With kStaged the rotation tables are copied to LDS once per
// work-group; otherwise they are read from memory in every layer. Every index
// read from memory is clamped into the row, every rotation number into
// 0 .. n_rot.
template <bool kPerm, bool kStaged>
__global__ __launch_bounds__(kThreads) void givens_rows_kernel(
    const uint16_t* x, int64_t ld_x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ pairs, const float* __restrict__ cs,
    const int32_t* __restrict__ layer_start, int n_layers, int n_rot, uint16_t* out,
    int64_t ld_out, int64_t rows, int cols) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* z = reinterpret_cast<float*>(smem);  // cols fp32
  uint8_t* rest = smem + 4 * (size_t)cols;
  uint16_t* raw = reinterpret_cast<uint16_t*>(rest);  // cols bf16 (kPerm)
  if (kPerm) rest += 2 * (size_t)cols;
  Tables t{reinterpret_cast<uint32_t*>(rest),
           reinterpret_cast<float2_t*>(rest + 4 * (size_t)n_rot + 4 * (n_rot & 1)),
           reinterpret_cast<int32_t*>(rest + 12 * (size_t)n_rot + 4 * (n_rot & 1))};
  if (kStaged) {
    for (int k = threadIdx.x; k < n_rot; k += kThreads) {
      t.ij[k] = (uint32_t)clamp_index(pairs[2 * k], cols) |
                ((uint32_t)clamp_index(pairs[2 * k + 1], cols) << 16);
      t.cs[k] = float2_t{cs[2 * k], cs[2 * k + 1]};
    }
    for (int L = threadIdx.x; L <= n_layers; L += kThreads)
      t.ls[L] = min(max(layer_start[L], 0), n_rot);
  }
  const int chunks = cols / 8;
  // the permutation entries of the thread's columns j = threadIdx.x + 256 u,
  // two 16-bit entries per register (read once; a load issued per row would
  // wait behind the next row's loads)
  uint32_t pj[kMaxColsPerThread / 2];
  if (kPerm) {
#pragma unroll
    for (int u = 0; u < kMaxColsPerThread; u += 2) {
      const int j0 = (int)threadIdx.x + u * kThreads, j1 = j0 + kThreads;
      const uint32_t a = j0 < cols ? (uint32_t)clamp_index(perm[j0], cols) : 0u;
      const uint32_t b = j1 < cols ? (uint32_t)clamp_index(perm[j1], cols) : 0u;
      pj[u / 2] = a | (b << 16);
    }
  }
  u32x4_t nxt[kMaxChunksPerThread];
  auto load_row = [&](int64_t r) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + r * ld_x);
#pragma unroll
    for (int u = 0; u < kMaxChunksPerThread; ++u) {
      const int c = (int)threadIdx.x + u * kThreads;
      if (c < chunks) nxt[u] = __builtin_nontemporal_load(src + c);
    }
  };
  if (blockIdx.x < rows) load_row(blockIdx.x);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
#pragma unroll
    for (int u = 0; u < kMaxChunksPerThread; ++u) {
      const int c = (int)threadIdx.x + u * kThreads;
      if (c >= chunks) continue;
      const u32x4_t v = nxt[u];
      if (kPerm) {
        reinterpret_cast<u32x4_t*>(raw)[c] = v;
      } else {
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
    if (r + gridDim.x < rows) load_row(r + gridDim.x);  // in flight during this row
    __syncthreads();
    if (kPerm) {
#pragma unroll
      for (int u = 0; u < kMaxColsPerThread; ++u) {
        const int j = (int)threadIdx.x + u * kThreads;
        if (j < cols) z[j] = __uint_as_float((uint32_t)raw[(pj[u / 2] >> (16 * (u & 1))) & 0xFFFFu] << 16);
      }
      __syncthreads();
    }
    for (int L = 0; L < n_layers; ++L) {
      int k0, k1;
      if (kStaged) {
        k0 = t.ls[L];
        k1 = max(t.ls[L + 1], k0);
      } else {
        k0 = min(max(layer_start[L], 0), n_rot);
        k1 = min(max(layer_start[L + 1], k0), n_rot);
      }
      for (int k = k0 + (int)threadIdx.x; k < k1; k += kThreads) {
        int i, j;
        float c, s;
        if (kStaged) {
          const uint32_t ij = t.ij[k];
          i = (int)(ij & 0xFFFFu);
          j = (int)(ij >> 16);
          const float2_t q = t.cs[k];
          c = q[0];
          s = q[1];
        } else {
          i = clamp_index(pairs[2 * k], cols);
          j = clamp_index(pairs[2 * k + 1], cols);
          c = cs[2 * k];
          s = cs[2 * k + 1];
        }
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
  const size_t row_lds = (perm ? 6 : 4) * (size_t)cols;
  // tables: 4 + 8 bytes per rotation (the second array 8-byte aligned), then
  // the layer starts
  const size_t tab_lds = 12 * (size_t)n_rot + 4 * (size_t)(n_rot & 1) + 4 * (size_t)(n_layers + 1);
  const bool staged = row_lds + tab_lds + 1024 <= (size_t)di.lds;
  const size_t lds = row_lds + (staged ? tab_lds : 0);
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(8, (size_t)di.lds / (lds + 1024)));
  const int64_t wgs = (int64_t)di.cus * per_cu;
  const int grid = (int)(rows < wgs ? rows : wgs);
  auto xp = static_cast<const uint16_t*>(x);
  auto op = static_cast<uint16_t*>(out);
#define FP4_GIVENS(P, S)                                                                    \
  hipLaunchKernelGGL((givens_rows_kernel<P, S>), dim3(grid), dim3(kThreads), lds, st, xp, ld_x, \
                     perm, pairs, cs, layer_start, n_layers, n_rot, op, ld_out, rows, (int)cols)
  if (perm && staged) FP4_GIVENS(true, true);
  else if (perm) FP4_GIVENS(true, false);
  else if (staged) FP4_GIVENS(false, true);
  else FP4_GIVENS(false, false);
#undef FP4_GIVENS
}

}  // namespace fp4
