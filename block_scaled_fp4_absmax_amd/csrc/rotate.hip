// rotate.hip -- two-level rotation fused with MXFP4 quantize + pack, the
// inverse rotation for dequantization, and the channel-energy statistic.
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2(a): an inter-block orthogonal transform that evens out the
// block variances (here a channel permutation computed offline); sec. 2(b): a
// rotation inside each 32-block (here the orthonormal Sylvester-Hadamard
// matrix, H[i][j] = (-1)^popcount(i & j) / sqrt(32)).
//
// Layout in registers: lane q of a group of four holds elements 8q..8q+7 of a
// block. H32 = H2 (x) H2 (x) H2 (x) H2 (x) H2 over the five index bits; bits
// 0-2 are butterflies inside a lane, bits 3-4 are butterflies with the lane
// xor 1 / xor 2 partner through DPP. The result is scaled by fp32(1/sqrt(32)).
//
// The permutation x'[j] = x[perm[j]] is applied by staging whole rows in LDS:
// a work-group loads a row with coalesced 16-byte loads, then each lane
// gathers its eight permuted elements with 2-byte LDS reads. The next row's
// global loads are issued before the current row is processed.
#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {

constexpr int kRotUnroll = 2;
constexpr float kInvSqrt32 = 0.17677669529663688f;

__device__ __forceinline__ void widen8(u32x4_t d, float* v) {
  v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
  v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
  v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
  v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
}

// In-place y = H32 v / sqrt(32) for the lane's eight elements (see header).
__device__ __forceinline__ void hadamard32(float* v, uint32_t lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k & h) continue;
      float a = v[k], b = v[k + h];
      v[k] = a + b;
      v[k + h] = a - b;
    }
  }
  // partner value t: lower lane takes own + t, upper lane t - own
  const float s1 = (lane & 1u) ? -1.0f : 1.0f;
  const float s2 = (lane & 2u) ? -1.0f : 1.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(s1, v[k], dpp_xor1f(v[k]));
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(s2, v[k], dpp_xor2f(v[k]));
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] *= kInvSqrt32;
}

// MXFP4 quantization of eight fp32 values whose block spans the lane's quad.
template <bool kFloor>
__device__ __forceinline__ void mx_quant8_f32(const float* y, uint32_t& w, uint32_t& byte) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, __float_as_uint(y[k]) & 0x7FFFFFFFu);
  m = max(m, dpp_xor1(m));
  m = max(m, dpp_xor2(m));
  byte = e8m0_byte<kFloor>(m);
  w = byte == 0xFFu ? 0u : cvt8_f32(y, e8m0_operand(byte));
}

__device__ __forceinline__ void store_rot(float* rot, const float* y) {
  f32x4_t a = {y[0], y[1], y[2], y[3]};
  f32x4_t b = {y[4], y[5], y[6], y[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(rot));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(rot) + 1);
}

struct RotGeom {
  int32_t rows, cols, cpr;  // cpr = chunks (of 8 elements) per row
  int64_t ld_x, ld_c, ld_s, ld_rot;
};

// ---- no permutation: streaming, one chunk per lane ------------------------
template <bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads) void mx_rotq_stream_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ rot, RotGeom g, uint32_t n) {
  const uint32_t stride = gridDim.x * kThreads;
  const uint32_t lane = threadIdx.x & 3u;
  for (uint32_t base = blockIdx.x * kThreads + threadIdx.x; base < n;
       base += kRotUnroll * stride) {
    u32x4_t d[kRotUnroll];
    uint32_t rr[kRotUnroll], cc[kRotUnroll];
#pragma unroll
    for (int u = 0; u < kRotUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v < n) {
        rr[u] = v / (uint32_t)g.cpr;
        cc[u] = v - rr[u] * (uint32_t)g.cpr;
        d[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(x + rr[u] * g.ld_x + 8 * (int64_t)cc[u]));
      }
    }
#pragma unroll
    for (int u = 0; u < kRotUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v >= n) continue;
      float y[8];
      widen8(d[u], y);
      if (kHad) hadamard32(y, lane);
      uint32_t w, byte;
      mx_quant8_f32<kFloor>(y, w, byte);
      __builtin_nontemporal_store(
          w, reinterpret_cast<uint32_t*>(codes + rr[u] * g.ld_c + 4 * (int64_t)cc[u]));
      if (lane == 0) scales[rr[u] * g.ld_s + cc[u] / 4] = (uint8_t)byte;
      if (kRot) store_rot(rot + rr[u] * g.ld_rot + 8 * (int64_t)cc[u], y);
    }
  }
}

// ---- with permutation: one row at a time through LDS ---------------------
// Dynamic LDS: row[cols] bf16 followed by perm[cols] uint16.
constexpr int kMaxChunksPerLane = (int)(kMaxPermCols / 8 / kThreads);  // 8

template <bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads) void mx_rotq_perm_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ rot, RotGeom g) {
  extern __shared__ uint16_t smem[];
  uint16_t* srow = smem;
  uint16_t* sperm = smem + g.cols;
  const uint32_t lane = threadIdx.x & 3u;
  const int32_t cmax = g.cols - 1;
  for (int32_t j = threadIdx.x; j < g.cols; j += kThreads) {
    int32_t p = perm[j];
    p = p < 0 ? 0 : (p > cmax ? cmax : p);  // an invalid entry cannot leave the row
    sperm[j] = (uint16_t)p;
  }
  u32x4_t pre[kMaxChunksPerLane];
  int32_t r = blockIdx.x;
  if (r < g.rows) {
#pragma unroll
    for (int i = 0; i < kMaxChunksPerLane; ++i) {
      int32_t c = threadIdx.x + i * kThreads;
      if (c < g.cpr)
        pre[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(x + r * g.ld_x + 8 * (int64_t)c));
    }
  }
  for (; r < g.rows; r += gridDim.x) {
    __syncthreads();  // the previous row's gathers are done
#pragma unroll
    for (int i = 0; i < kMaxChunksPerLane; ++i) {
      int32_t c = threadIdx.x + i * kThreads;
      if (c < g.cpr) reinterpret_cast<u32x4_t*>(srow)[c] = pre[i];
    }
    __syncthreads();
    const int32_t rn = r + gridDim.x;
    if (rn < g.rows) {
#pragma unroll
      for (int i = 0; i < kMaxChunksPerLane; ++i) {
        int32_t c = threadIdx.x + i * kThreads;
        if (c < g.cpr)
          pre[i] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4_t*>(x + rn * g.ld_x + 8 * (int64_t)c));
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxChunksPerLane; ++i) {
      int32_t c = threadIdx.x + i * kThreads;
      if (c >= g.cpr) continue;
      u32x4_t id = reinterpret_cast<const u32x4_t*>(sperm)[c];
      float y[8];
      y[0] = __uint_as_float((uint32_t)srow[id.x & 0xFFFFu] << 16);
      y[1] = __uint_as_float((uint32_t)srow[id.x >> 16] << 16);
      y[2] = __uint_as_float((uint32_t)srow[id.y & 0xFFFFu] << 16);
      y[3] = __uint_as_float((uint32_t)srow[id.y >> 16] << 16);
      y[4] = __uint_as_float((uint32_t)srow[id.z & 0xFFFFu] << 16);
      y[5] = __uint_as_float((uint32_t)srow[id.z >> 16] << 16);
      y[6] = __uint_as_float((uint32_t)srow[id.w & 0xFFFFu] << 16);
      y[7] = __uint_as_float((uint32_t)srow[id.w >> 16] << 16);
      if (kHad) hadamard32(y, lane);
      uint32_t w, byte;
      mx_quant8_f32<kFloor>(y, w, byte);
      __builtin_nontemporal_store(
          w, reinterpret_cast<uint32_t*>(codes + r * g.ld_c + 4 * (int64_t)c));
      if (lane == 0) scales[r * g.ld_s + c / 4] = (uint8_t)byte;
      if (kRot) store_rot(rot + r * g.ld_rot + 8 * (int64_t)c, y);
    }
  }
}

// ---- inverse rotation after MXFP4 decoding --------------------------------
template <bool kHad, bool kPerm>
__global__ __launch_bounds__(kThreads) void mx_dequant_unrotate_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ perm, uint16_t* __restrict__ out, RotGeom g) {
  extern __shared__ uint16_t smem[];
  uint16_t* srow = smem;
  uint16_t* sperm = smem + g.cols;
  const uint32_t lane = threadIdx.x & 3u;
  const int32_t cmax = g.cols - 1;
  if (kPerm) {
    for (int32_t j = threadIdx.x; j < g.cols; j += kThreads) {
      int32_t p = perm[j];
      p = p < 0 ? 0 : (p > cmax ? cmax : p);
      sperm[j] = (uint16_t)p;
    }
  }
  for (int32_t r = blockIdx.x; r < g.rows; r += gridDim.x) {
    if (kPerm) __syncthreads();  // previous row copied out, indices visible
    for (int32_t c = threadIdx.x; c < g.cpr; c += kThreads) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(codes + r * g.ld_c + 4 * (int64_t)c);
      float s = e8m0_operand(scales[r * g.ld_s + c / 4]);
      float y[8];
      float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
      float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
      float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
      float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
      y[0] = p0.x; y[1] = p0.y; y[2] = p1.x; y[3] = p1.y;
      y[4] = p2.x; y[5] = p2.y; y[6] = p3.x; y[7] = p3.y;
      if (kHad) hadamard32(y, lane);  // H is symmetric and orthonormal: its own inverse
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
        *reinterpret_cast<u32x4_t*>(out + r * g.ld_x + 8 * (int64_t)c) = o;
      }
    }
    if (kPerm) {
      __syncthreads();
      for (int32_t c = threadIdx.x; c < g.cpr; c += kThreads)
        *reinterpret_cast<u32x4_t*>(out + r * g.ld_x + 8 * (int64_t)c) =
            reinterpret_cast<const u32x4_t*>(srow)[c];
    }
  }
}

// ---- channel energy ------------------------------------------------------
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

// --------------------------------------------------------------- launchers ----
static RotGeom rot_geom(const Shape& s, int64_t ld_rot) {
  RotGeom g;
  g.rows = (int32_t)s.rows;
  g.cols = (int32_t)s.cols;
  g.cpr = (int32_t)(s.cols / 8);
  g.ld_x = s.ld_x;
  g.ld_c = s.ld_c;
  g.ld_s = s.ld_s;
  g.ld_rot = ld_rot;
  return g;
}

template <bool kHad, bool kFloor, bool kRot>
static void rotq_dispatch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                          uint8_t* sc, float* rot, const RotGeom& g, hipStream_t st) {
  if (perm) {
    int grid = (int)(s.rows < 2048 ? s.rows : 2048);
    size_t lds = (size_t)4 * s.cols;
    hipLaunchKernelGGL((mx_rotq_perm_kernel<kHad, kFloor, kRot>), dim3(grid), dim3(kThreads), lds,
                       st, x, perm, c, sc, rot, g);
  } else {
    uint32_t n = (uint32_t)(s.rows * s.cols / 8);
    uint64_t per = (uint64_t)kThreads * kRotUnroll;
    uint64_t grid = (n + per - 1) / per;
    if (grid > (uint64_t)kMaxGrid) grid = kMaxGrid;
    hipLaunchKernelGGL((mx_rotq_stream_kernel<kHad, kFloor, kRot>), dim3((int)grid),
                       dim3(kThreads), 0, st, x, c, sc, rot, g, n);
  }
}

void launch_mx_rotate_quant(const Shape& s, const int32_t* perm, int hadamard, bool floor_rule,
                            const void* x, void* codes, void* scales, float* rot, int64_t ld_rot,
                            hipStream_t st) {
  RotGeom g = rot_geom(s, ld_rot);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  const bool had = hadamard != 0, r = rot != nullptr;
  if (had && !floor_rule && !r) rotq_dispatch<true, false, false>(s, perm, xp, cp, sp, rot, g, st);
  if (had && !floor_rule && r) rotq_dispatch<true, false, true>(s, perm, xp, cp, sp, rot, g, st);
  if (had && floor_rule && !r) rotq_dispatch<true, true, false>(s, perm, xp, cp, sp, rot, g, st);
  if (had && floor_rule && r) rotq_dispatch<true, true, true>(s, perm, xp, cp, sp, rot, g, st);
  if (!had && !floor_rule && !r) rotq_dispatch<false, false, false>(s, perm, xp, cp, sp, rot, g, st);
  if (!had && !floor_rule && r) rotq_dispatch<false, false, true>(s, perm, xp, cp, sp, rot, g, st);
  if (!had && floor_rule && !r) rotq_dispatch<false, true, false>(s, perm, xp, cp, sp, rot, g, st);
  if (!had && floor_rule && r) rotq_dispatch<false, true, true>(s, perm, xp, cp, sp, rot, g, st);
}

void launch_mx_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard,
                                const void* codes, const void* scales, void* out, hipStream_t st) {
  RotGeom g = rot_geom(s, 0);
  auto cp = static_cast<const uint8_t*>(codes);
  auto sp = static_cast<const uint8_t*>(scales);
  auto op = static_cast<uint16_t*>(out);
  int grid = (int)(s.rows < 2048 ? s.rows : 2048);
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
