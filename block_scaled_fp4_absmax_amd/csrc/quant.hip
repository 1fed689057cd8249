// quant.hip -- MXFP4 / MXINT4 / NVFP4 (+RaZeR) quantize + pack, tensor amax,
// dequantize.
//
// Work decomposition: one lane owns one 16-byte chunk of eight consecutive
// bf16 (a coalesced dwordx4 load), so four neighbouring lanes hold one
// 32-element MXFP4 block and two hold one 16-element NVFP4 block. Block-wide
// reductions are one or two DPP quad_perm steps; no LDS is used. The chunk
// index v walks the matrix row-major. Each work-group makes a single pass over
// one contiguous range of kThreads * kUnroll chunks (lane t takes chunks
// base + u * kThreads + t), issuing all its loads before any arithmetic: on
// MI355X this keeps whole cache lines of codes and scales inside one
// work-group and measured faster than grid-stride loops. Since cols is a
// multiple of the block, the chunks of one block are always held by adjacent
// lanes at the same u.
#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {

#ifndef FP4_UNROLL
#define FP4_UNROLL 4
#endif
constexpr int kUnroll = FP4_UNROLL;  // chunks per lane (one pass per work-group)

// Address arithmetic for chunk v. kFlat: rows are contiguous in every array,
// so the matrix is a single row of rows * cols elements.
struct Geom {
  uint32_t n;    // number of chunks = rows * cols / 8
  uint32_t cpr;  // chunks per row
  int64_t ld_x, ld_c, ld_s;
  bool s_gemm;   // scale bytes in the GEMM order (never with kFlat)
};

template <bool kFlat, int kBlock>
__device__ __forceinline__ void locate(const Geom& g, uint32_t v, int64_t& xo, int64_t& co,
                                       int64_t& so) {
  if (kFlat) {
    xo = 8 * (int64_t)v;
    co = 4 * (int64_t)v;
    so = (int64_t)(v / (kBlock / 8));
  } else {
    uint32_t r = v / g.cpr, c = v - r * g.cpr;
    xo = r * g.ld_x + 8 * (int64_t)c;
    co = r * g.ld_c + 4 * (int64_t)c;
    so = scale_row_off(r, g.ld_s, g.s_gemm) + scale_col_off(c / (kBlock / 8), g.s_gemm);
  }
}

// ------------------------------------------------------- MXFP4 / MXINT4 ----
// kInt: MXINT4 elements (two's complement k / 4) instead of E2M1.
template <bool kFlat, bool kFloor, bool kInt>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, Geom g) {
  const bool leader = (threadIdx.x & 3) == 0;
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  constexpr uint32_t stride = kThreads;
  {
    u32x4_t d[kUnroll];
    int64_t xo[kUnroll], co[kUnroll], so[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v < g.n) {
        locate<kFlat, 32>(g, v, xo[u], co[u], so[u]);
        d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xo[u]));
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v < g.n) {
        uint32_t m = absmax8_bf16(d[u]);
        m = max(m, dpp_xor1(m));
        m = max(m, dpp_xor2(m));
        uint32_t byte, w;
        if constexpr (kInt) {
          byte = mxint_byte<kFloor>(m << 16);
          float v[8];
          widen8(d[u], v);
          w = byte == 0xFFu ? 0u : int4x8_f32(v, 129 - (int)byte);
        } else {
          byte = e8m0_byte<kFloor>(m << 16);
          w = byte == 0xFFu ? 0u : cvt8_bf16(d[u], e8m0_operand(byte));
        }
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + co[u]));
        if (leader) scales[so[u]] = (uint8_t)byte;
      }
    }
  }
}

// ---------------------------------------------------------------- NVFP4 ----
// Tensor amax without atomics or scratch memory: each work-group reduces its
// chunks to max |x| (the fp32 bit pattern, which orders like the magnitude)
// and work-group i stores it in the code slot of chunk i -- output space that
// the quantize kernel overwrites later in the same call, and contiguous (row
// by row for strided codes) so the reduction reads it with coalesced loads. A
// single work-group then reduces those partials and writes s_t = amax / 2688
// (6 * 448), or 1 for an all-zero tensor.
// Read-only, so each lane keeps kAmaxUnroll loads in flight and the pass
// leaves one partial per kThreads * kAmaxUnroll chunks.
constexpr int kAmaxUnroll = 16;

template <bool kFlat>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ codes, Geom g) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0;
  const uint32_t base = blockIdx.x * (kThreads * kAmaxUnroll) + threadIdx.x;
  u32x4_t d[kAmaxUnroll];
#pragma unroll
  for (int u = 0; u < kAmaxUnroll; ++u) {
    uint32_t v = base + u * kThreads;
    d[u] = u32x4_t{0u, 0u, 0u, 0u};
    if (v < g.n) {
      int64_t xo, co, so;
      locate<kFlat, 16>(g, v, xo, co, so);
      d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xo));
    }
  }
#pragma unroll
  for (int u = 0; u < kAmaxUnroll; ++u) m = max(m, absmax8_bf16(d[u]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
    int64_t xo, co, so;
    locate<kFlat, 16>(g, blockIdx.x, xo, co, so);
    *reinterpret_cast<uint32_t*>(codes + co) = r << 16;
  }
}

// One work-group of kScaleThreads reduces the partials; each lane keeps 16
// loads in flight, so a tensor of up to 16 * kScaleThreads partials takes a
// single round trip.
constexpr int kScaleThreads = 1024;

// top: the largest scaled block maximum, 6 * 448 = 2688 (E4M3 scales) or
// 6 * 30 = 180 (E3M3 scales of RaZeR for weights).
template <bool kFlat>
__global__ __launch_bounds__(kScaleThreads) void nv_tensor_scale_kernel(
    const uint8_t* __restrict__ codes, uint32_t nparts, Geom g, float top,
    float* __restrict__ ts) {
  __shared__ uint32_t red[kScaleThreads / 64];
  uint32_t m = 0;
  for (uint32_t i0 = threadIdx.x; i0 < nparts; i0 += 16 * kScaleThreads) {
    uint32_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t i = i0 + u * kScaleThreads;
      v[u] = 0;
      if (i < nparts) {
        int64_t xo, co, so;
        locate<kFlat, 16>(g, i, xo, co, so);
        v[u] = *reinterpret_cast<const uint32_t*>(codes + co);
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) m = max(m, v[u]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
    for (int i = 1; i < kScaleThreads / 64; ++i) r = max(r, red[i]);
    const float amax = __uint_as_float(r);
    *ts = amax == 0.0f ? 1.0f : amax / top;
  }
}

// Empty tensor: nothing to reduce, s_t = 1.
__global__ void nv_unit_scale_kernel(float* ts) { *ts = 1.0f; }

// One NVFP4 chunk (half a block; the block spans lanes l and l ^ 1): the scale
// arithmetic is in fp4_device.hpp (nv_block_code, nv_rcp_table).
// kMode: 0 plain NVFP4, 1 RaZeR (E4M3 scale, +-5 by the scale's sign bit),
// 2 RaZeR for weights (E3M3 scale, {+5, -5, +2.5, -2.5} by bits 6-7).
template <int kMode>
__device__ __forceinline__ void nv_quant_chunk(u32x4_t d, const NvScale& ns, const float* rcp_tab,
                                               uint32_t& w, uint32_t& byte) {
  uint32_t m = absmax8_bf16(d);
  m = max(m, dpp_xor1(m));
  const float amax = __uint_as_float(m << 16);
  const uint32_t sb = kMode == 2 ? nvw_block_code(amax, ns) : nv_block_code(amax, ns);
  w = 0;
  byte = 0;
  if (sb != 0u) {
    const float r = rcp_tab[sb];
    float y[8];
    y[0] = bf16_lo(d.x) * r; y[1] = bf16_hi(d.x) * r;
    y[2] = bf16_lo(d.y) * r; y[3] = bf16_hi(d.y) * r;
    y[4] = bf16_lo(d.z) * r; y[5] = bf16_hi(d.z) * r;
    y[6] = bf16_lo(d.w) * r; y[7] = bf16_hi(d.w) * r;
    w = cvt8_f32(y, 1.0f);
    byte = sb;
    if constexpr (kMode == 1) {
      // selector = [gains of negative elements exceed those of positive ones]
      float dsum = 0.0f;
      float gk[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        gk[k] = razer_gain(y[k]);  // in [0, 1]
        dsum -= __builtin_copysignf(gk[k], y[k]);
      }
      const uint32_t cm = razer_flags8(gk);
      dsum += dpp_xor1f(dsum);
      const uint32_t sel = dsum > 0.0f ? 1u : 0u;
      w = razer_apply(w, cm, sel);
      byte |= sel << 7;
    } else if constexpr (kMode == 2) {
      // block gains of the four specials; the largest wins, ties to the
      // lower selector. Per pair, s = G+ + G- and d = G+ - G- (the sign of y
      // as a +-1 factor of one fma), then G+- = (s +- d) / 2: every sum is
      // exact (multiples of 2^-20 or 2^-22, at most 16 or 4), and s +- d is
      // the exact 2 G+-, so the gains equal the separate sums bit for bit.
      float s5 = 0.0f, d5 = 0.0f, s2 = 0.0f, d2 = 0.0f;
      float g5[8], g2[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        g5[k] = razer_gain(y[k]);
        g2[k] = razer_gain_pair2(y[k]);
        const float sg = __builtin_copysignf(1.0f, y[k]);
        s5 += g5[k];
        d5 = __builtin_fmaf(sg, g5[k], d5);
        s2 += g2[k];
        d2 = __builtin_fmaf(sg, g2[k], d2);
      }
      const uint32_t cm5 = razer_flags8(g5), cm2 = razer_flags8(g2);
      s5 += dpp_xor1f(s5);
      d5 += dpp_xor1f(d5);
      s2 += dpp_xor1f(s2);
      d2 += dpp_xor1f(d2);
      const float g[4] = {0.5f * (s5 + d5), 0.5f * (s5 - d5), 0.5f * (s2 + d2),
                          0.5f * (s2 - d2)};  // +5, -5, +2.5, -2.5
      uint32_t sel = 0;
      float best = g[0];
      if (g[1] > best) { best = g[1]; sel = 1; }
      if (g[2] > best) { best = g[2]; sel = 2; }
      if (g[3] > best) { sel = 3; }
      w = razer_apply(w, sel >= 2u ? cm2 : cm5, sel & 1u);
      byte |= sel << 6;
    }
  }
}

// kFull: the work-group's kThreads * kUnroll chunks all exist (every
// work-group but the last), so loads and stores need no bounds check.
template <bool kFlat, int kMode, bool kFull>
__device__ __forceinline__ void nv_quant_pass(const uint16_t* __restrict__ x,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales, const float* rcp_tab,
                                              const NvScale& ns, const Geom& g, const u32x4_t* d,
                                              const int64_t* co, const int64_t* so) {
  const bool leader = (threadIdx.x & 1) == 0;
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (!kFull && base + u * kThreads >= g.n) continue;
    uint32_t w, byte;
    nv_quant_chunk<kMode>(d[u], ns, rcp_tab, w, byte);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + co[u]));
    if (leader) scales[so[u]] = (uint8_t)byte;
  }
}

template <bool kFlat, int kMode>
__global__ __launch_bounds__(kThreads) void nv_quant_kernel(const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            const float* __restrict__ ts, Geom g) {
  __shared__ float rcp_tab[128];
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  const bool full = (blockIdx.x + 1) * (kThreads * kUnroll) <= g.n;  // uniform
  u32x4_t d[kUnroll];
  int64_t xo[kUnroll], co[kUnroll], so[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t v = base + u * kThreads;
    locate<kFlat, 16>(g, v < g.n ? v : 0, xo[u], co[u], so[u]);
  }
  if (full) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xo[u]));
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * kThreads < g.n)
        d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xo[u]));
  }
  const float s_t = *ts;
  const NvScale ns = nv_scale_setup(s_t);
  if (kMode == 2)
    nvw_rcp_table(rcp_tab, s_t);
  else
    nv_rcp_table(rcp_tab, s_t);
  __syncthreads();
  if (full)
    nv_quant_pass<kFlat, kMode, true>(x, codes, scales, rcp_tab, ns, g, d, co, so);
  else
    nv_quant_pass<kFlat, kMode, false>(x, codes, scales, rcp_tab, ns, g, d, co, so);
}

// ------------------------------------------------------------ dequantize ----
template <bool kFlat, bool kInt>
__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              uint16_t* __restrict__ out, Geom g) {
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  constexpr uint32_t stride = kThreads;
  {
    uint32_t w[kUnroll], sb[kUnroll];
    int64_t xo[kUnroll], co[kUnroll], so[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v < g.n) {
        locate<kFlat, 32>(g, v, xo[u], co[u], so[u]);
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + co[u]));
        sb[u] = scales[so[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v >= g.n) continue;
      u32x4_t o;
      if constexpr (kInt) {
        o = int4x8_decode(w[u], sb[u]);
      } else {
        const float s = e8m0_operand(sb[u]);  // byte 0xFF -> NaN scale -> NaN outputs
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], s, 0));
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], s, 1));
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], s, 2));
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[u], s, 3));
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + xo[u]));
    }
  }
}

template <bool kFlat, int kMode>
__global__ __launch_bounds__(kThreads) void nv_dequant_kernel(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ ts,
                                                              uint16_t* __restrict__ out, Geom g) {
  const float s_t = *ts;
  const uint32_t base = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  constexpr uint32_t stride = kThreads;
  {
    uint32_t w[kUnroll], sb[kUnroll];
    int64_t xo[kUnroll], co[kUnroll], so[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v < g.n) {
        locate<kFlat, 16>(g, v, xo[u], co[u], so[u]);
        w[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + co[u]));
        sb[u] = scales[so[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t v = base + u * stride;
      if (v >= g.n) continue;
      const uint32_t byte = sb[u];
      const float s_eff = (kMode == 2 ? e3m3_decode(byte) : e4m3_decode(kMode ? (byte & 0x7Fu) : byte)) * s_t;
      const float special = kMode == 2 ? weight_special(byte) : (byte & 0x80u) ? -5.0f : 5.0f;
      float val[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float2_t p;
        if (k == 0) p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 0);
        if (k == 1) p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 1);
        if (k == 2) p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 2);
        if (k == 3) p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 3);
        val[2 * k] = p.x;
        val[2 * k + 1] = p.y;
      }
      if (kMode) {  // code 8 is the only code that decodes to -0.0
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (__float_as_uint(val[k]) == 0x80000000u) val[k] = special;
      }
      u32x4_t o;
      o.x = pack_bf16x2(val[0] * s_eff, val[1] * s_eff);
      o.y = pack_bf16x2(val[2] * s_eff, val[3] * s_eff);
      o.z = pack_bf16x2(val[4] * s_eff, val[5] * s_eff);
      o.w = pack_bf16x2(val[6] * s_eff, val[7] * s_eff);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + xo[u]));
    }
  }
}

// --------------------------------------------------------------- launchers ----
// One work-group per kThreads * kUnroll chunks (n < 2^31, so this fits).
static inline int grid_for(uint32_t n) {
  uint64_t per = (uint64_t)kThreads * kUnroll;
  uint64_t gsz = (n + per - 1) / per;
  return (int)(gsz ? gsz : 1);
}

static inline Geom make_geom(const Shape& s, int block) {
  Geom g;
  g.n = (uint32_t)(s.rows * s.cols / 8);
  g.cpr = (uint32_t)(s.cols / 8);
  g.ld_x = s.ld_x;
  g.ld_c = s.ld_c;
  g.ld_s = s.ld_s;
  g.s_gemm = s.s_gemm;
  (void)block;
  return g;
}

#define FP4_LAUNCH(kern, grid, stream, ...) \
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, __VA_ARGS__)

template <bool kInt>
static void mx_quant_variants(const Shape& s, bool floor_rule, const void* x, void* codes,
                              void* scales, hipStream_t st) {
  Geom g = make_geom(s, 32);
  const bool flat =
      s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / 32 && !s.s_gemm;
  const int grid = grid_for(g.n);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  if (flat && !floor_rule) FP4_LAUNCH((mx_quant_kernel<true, false, kInt>), grid, st, xp, cp, sp, g);
  if (flat && floor_rule) FP4_LAUNCH((mx_quant_kernel<true, true, kInt>), grid, st, xp, cp, sp, g);
  if (!flat && !floor_rule) FP4_LAUNCH((mx_quant_kernel<false, false, kInt>), grid, st, xp, cp, sp, g);
  if (!flat && floor_rule) FP4_LAUNCH((mx_quant_kernel<false, true, kInt>), grid, st, xp, cp, sp, g);
}

void launch_mx_quant(const Shape& s, bool floor_rule, bool mxint, const void* x, void* codes,
                     void* scales, hipStream_t st) {
  if (mxint) mx_quant_variants<true>(s, floor_rule, x, codes, scales, st);
  else mx_quant_variants<false>(s, floor_rule, x, codes, scales, st);
}

void launch_nv_tensor_scale(const Shape& s, const void* x, void* codes, float top, float* ts,
                            hipStream_t st) {
  Geom g = make_geom(s, 16);
  if (g.n == 0) {
    hipLaunchKernelGGL(nv_unit_scale_kernel, dim3(1), dim3(1), 0, st, ts);
    return;
  }
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2;
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  const uint64_t per = (uint64_t)kThreads * kAmaxUnroll;
  const int grid = (int)((g.n + per - 1) / per);
  if (flat) {
    FP4_LAUNCH((nv_amax_kernel<true>), grid, st, xp, cp, g);
    hipLaunchKernelGGL((nv_tensor_scale_kernel<true>), dim3(1), dim3(kScaleThreads), 0, st, cp,
                       (uint32_t)grid, g, top, ts);
  } else {
    FP4_LAUNCH((nv_amax_kernel<false>), grid, st, xp, cp, g);
    hipLaunchKernelGGL((nv_tensor_scale_kernel<false>), dim3(1), dim3(kScaleThreads), 0, st, cp,
                       (uint32_t)grid, g, top, ts);
  }
}

void launch_nv_scale_from_partials(const Shape& s, void* codes, uint32_t nparts, float* ts,
                                   hipStream_t st) {
  if (nparts == 0) {
    hipLaunchKernelGGL(nv_unit_scale_kernel, dim3(1), dim3(1), 0, st, ts);
    return;
  }
  Geom g = make_geom(s, 16);
  hipLaunchKernelGGL((nv_tensor_scale_kernel<false>), dim3(1), dim3(kScaleThreads), 0, st,
                     static_cast<const uint8_t*>(codes), nparts, g, 2688.0f, ts);
}

template <int kMode>
static void nv_quant_variants(const Shape& s, const void* x, void* codes, void* scales,
                              const float* ts, hipStream_t st) {
  Geom g = make_geom(s, 16);
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / 16;
  const int grid = grid_for(g.n);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  if (flat) FP4_LAUNCH((nv_quant_kernel<true, kMode>), grid, st, xp, cp, sp, ts, g);
  else FP4_LAUNCH((nv_quant_kernel<false, kMode>), grid, st, xp, cp, sp, ts, g);
}

void launch_nv_quant(const Shape& s, int mode, const void* x, void* codes, void* scales,
                     const float* ts, hipStream_t st) {
  if (mode == 2) nv_quant_variants<2>(s, x, codes, scales, ts, st);
  else if (mode == 1) nv_quant_variants<1>(s, x, codes, scales, ts, st);
  else nv_quant_variants<0>(s, x, codes, scales, ts, st);
}

void launch_dequant(const Shape& s, int format, int mode, const void* codes, const void* scales,
                    const float* ts, void* out, hipStream_t st) {
  const int block = format == 1 ? 16 : 32;
  Geom g = make_geom(s, block);
  // here ld_x is the output row stride
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / block;
  const int grid = grid_for(g.n);
  auto cp = static_cast<const uint8_t*>(codes);
  auto sp = static_cast<const uint8_t*>(scales);
  auto op = static_cast<uint16_t*>(out);
  if (format == 0) {
    if (flat) FP4_LAUNCH((mx_dequant_kernel<true, false>), grid, st, cp, sp, op, g);
    else FP4_LAUNCH((mx_dequant_kernel<false, false>), grid, st, cp, sp, op, g);
  } else if (format == 2) {
    if (flat) FP4_LAUNCH((mx_dequant_kernel<true, true>), grid, st, cp, sp, op, g);
    else FP4_LAUNCH((mx_dequant_kernel<false, true>), grid, st, cp, sp, op, g);
  } else {
#define FP4_NV_DQ(M)                                                                   \
  if (mode == M) {                                                                     \
    if (flat) FP4_LAUNCH((nv_dequant_kernel<true, M>), grid, st, cp, sp, ts, op, g);   \
    else FP4_LAUNCH((nv_dequant_kernel<false, M>), grid, st, cp, sp, ts, op, g);       \
  }
    FP4_NV_DQ(0) FP4_NV_DQ(1) FP4_NV_DQ(2)
#undef FP4_NV_DQ
  }
}

}  // namespace fp4
