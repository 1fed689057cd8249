// unrotate.hip -- MXFP4 dequantization with the inverse of the two-level
// rotation, and the channel-energy statistic that calibrates the permutation.
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2: the rotation is orthogonal, so decoding in the original
// basis applies H (its own inverse) and then the inverse permutation; the
// permutation balances the energy of the blocks (sec. 2(a)), measured here
// per channel over the calibration rows.
#include "rotation.hpp"

namespace fp4 {

// ============================ inverse rotation ==============================
// perm staged into LDS as uint16, clamped to [0, cols - 1] (cols <= 16384):
// sixteen 16-byte loads per lane in flight at once, then one wait.
__device__ __forceinline__ void stage_perm(const int32_t* __restrict__ perm, uint16_t* sperm,
                                           int32_t cols) {
  constexpr int kPv = (int)(kMaxPermCols / 4 / kThreads);
  const rsrc_t rp = make_rsrc(perm, 4u * (uint32_t)cols);
  const int32_t nv = cols / 4, cmax = cols - 1;
  i32x4_t p[kPv];
#pragma unroll
  for (int u = 0; u < kPv; ++u) {
    const int32_t v = threadIdx.x + u * kThreads;
    p[u] = __builtin_bit_cast(
        i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, v < nv ? 16u * v : kOob, 0, 0));
  }
#pragma unroll
  for (int u = 0; u < kPv; ++u) {
    const int32_t v = threadIdx.x + u * kThreads;
    if (v < nv) {
      const i32x4_t q = p[u];
      const uint32_t c0 = (uint32_t)min(max(q.x, 0), cmax), c1 = (uint32_t)min(max(q.y, 0), cmax);
      const uint32_t c2 = (uint32_t)min(max(q.z, 0), cmax), c3 = (uint32_t)min(max(q.w, 0), cmax);
      reinterpret_cast<u32x2_t*>(sperm)[v] = u32x2_t{c0 | (c1 << 16), c2 | (c3 << 16)};
    }
  }
  __syncthreads();
}

// Decode MXFP4 exactly to fp32, apply H (its own inverse) with the butterfly,
// then scatter element j to column perm[j] through LDS.
template <bool kHad, bool kPerm>
__global__ __launch_bounds__(kThreads) void mx_dequant_unrotate_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ perm, uint16_t* __restrict__ out, RotGeom g) {
  extern __shared__ uint16_t smem[];
  uint16_t* srow = smem;
  uint16_t* sperm = smem + g.cols;
  const uint32_t q = threadIdx.x & 3u;
  const int32_t cpr = g.cols / 8;
  if (kPerm) stage_perm(perm, sperm, g.cols);
  for (int32_t r = blockIdx.x; r < g.rows; r += gridDim.x) {
    if (kPerm) __syncthreads();  // previous row copied out, indices visible
    for (int32_t c = threadIdx.x; c < cpr; c += kThreads) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * g.ld_c + 4 * (int64_t)c);
      float s = e8m0_operand(scales[r * g.ld_s + c / 4]);
      float y[8];
      float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
      float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
      float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
      float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
      y[0] = p0.x; y[1] = p0.y; y[2] = p1.x; y[3] = p1.y;
      y[4] = p2.x; y[5] = p2.y; y[6] = p3.x; y[7] = p3.y;
      if (kHad) hadamard_butterfly(y, q);
      u32x4_t o;
      o.x = pack_bf16x2(y[0], y[1]);
      o.y = pack_bf16x2(y[2], y[3]);
      o.z = pack_bf16x2(y[4], y[5]);
      o.w = pack_bf16x2(y[6], y[7]);
      if (kPerm) {
        u32x4_t id = reinterpret_cast<const u32x4_t*>(sperm)[c];
        srow[id.x & 0xFFFFu] = (uint16_t)(o.x & 0xFFFFu);
        srow[id.x >> 16] = (uint16_t)(o.x >> 16);
        srow[id.y & 0xFFFFu] = (uint16_t)(o.y & 0xFFFFu);
        srow[id.y >> 16] = (uint16_t)(o.y >> 16);
        srow[id.z & 0xFFFFu] = (uint16_t)(o.z & 0xFFFFu);
        srow[id.z >> 16] = (uint16_t)(o.z >> 16);
        srow[id.w & 0xFFFFu] = (uint16_t)(o.w & 0xFFFFu);
        srow[id.w >> 16] = (uint16_t)(o.w >> 16);
      } else {
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + r * g.ld_x) + c);
      }
    }
    if (kPerm) {
      __syncthreads();
      for (int32_t c = threadIdx.x; c < cpr; c += kThreads)
        __builtin_nontemporal_store(reinterpret_cast<const u32x4_t*>(srow)[c],
                                    reinterpret_cast<u32x4_t*>(out + r * g.ld_x) + c);
    }
  }
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

// ================================ launchers =================================
static int perm_grid(int64_t rows) { return (int)(rows < kPermGrid ? rows : kPermGrid); }

void launch_mx_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard,
                                const void* codes, const void* scales, void* out, hipStream_t st) {
  RotGeom g = rot_geom(s, 0);
  auto cp = static_cast<const uint8_t*>(codes);
  auto sp = static_cast<const uint8_t*>(scales);
  auto op = static_cast<uint16_t*>(out);
  const int grid = perm_grid(s.rows);
  size_t lds = perm ? (size_t)4 * s.cols : 0;
  if (hadamard && perm)
    hipLaunchKernelGGL((mx_dequant_unrotate_kernel<true, true>), dim3(grid), dim3(kThreads), lds,
                       st, cp, sp, perm, op, g);
  if (hadamard && !perm)
    hipLaunchKernelGGL((mx_dequant_unrotate_kernel<true, false>), dim3(grid), dim3(kThreads), lds,
                       st, cp, sp, perm, op, g);
  if (!hadamard && perm)
    hipLaunchKernelGGL((mx_dequant_unrotate_kernel<false, true>), dim3(grid), dim3(kThreads), lds,
                       st, cp, sp, perm, op, g);
}

void launch_channel_energy(int64_t rows, int64_t cols, int64_t ld_x, const void* x, float* energy,
                           hipStream_t st) {
  hipLaunchKernelGGL(channel_energy_kernel, dim3((int)(cols / 32)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), energy, rows, ld_x);
}

}  // namespace fp4
