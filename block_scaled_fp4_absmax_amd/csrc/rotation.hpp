// rotation.hpp -- helpers shared by the rotation kernels: the 32-point block
// Hadamard (MFMA and butterfly forms), MXFP4 quantization of rotated fp32
// values, and the row geometry.
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2(b): a rotation inside each 32-block, here the orthonormal
// Sylvester-Hadamard matrix H[i][j] = (-1)^popcount(i & j) / sqrt(32).
#pragma once

#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {

constexpr float kInvSqrt32 = 0.17677669529663688f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_rot8(float* rot, const float* y) {
  f32x4_t a = {y[0], y[1], y[2], y[3]};
  f32x4_t b = {y[4], y[5], y[6], y[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(rot));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(rot) + 1);
}

// Largest |y| of n fp32 values as a bit pattern (NaN above Inf above finite).
template <int n>
__device__ __forceinline__ uint32_t absmax_bits(const float* y) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < n; ++k) m = max(m, __float_as_uint(y[k]) & 0x7FFFFFFFu);
  return m;
}

// ============================ MFMA implementation ===========================
// Row tau(m) of H held in MFMA output row m: lane half h' = (m / 4) % 2 owns
// outputs 16h'..16h'+15, register r = 4 (m / 8) + m % 4 holds output 16h' + r.
__device__ __forceinline__ uint32_t out_index_of_row(uint32_t m) {
  return 16u * ((m >> 2) & 1u) + 4u * (m >> 3) + (m & 3u);
}

// Constant A operands: lane l holds A[m = l % 32][kk = 8 (l / 32) + j]; for
// the first MFMA kk stands for element 16 (kk / 8) + kk % 8, for the second
// 16 (kk / 8) + 8 + kk % 8 (matching the B halves each lane loads). So the 16
// operand entries of lane l are A[tau(l % 32)][k0 + j], k0 = 16 (l / 32),
// j = 0..15. For the 32-point transform A = H32, with sign
// parity(row & (k0 + j)) = parity(row & k0) ^ parity(row & j); bit j of the
// Walsh mask W(row & 15) is parity(row & j). For 16-point blocks A is
// diag(H16, H16) on each 32-element segment: entries couple an output row
// only to inputs of the same half (row / 16 == l / 32), with sign W(row & 15).
// The 16-point entries are +-1/4 (exact in bf16), which carries the transform's
// 1/sqrt(16) into the MFMA; the 32-point ones are +-1 (1/sqrt(32) is not exact).
template <int kN>
__device__ __forceinline__ void hadamard_operands(bf16x8_t& a0, bf16x8_t& a1) {
  static_assert(kN == 16 || kN == 32, "block Hadamard of 16 or 32 points");
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t row = out_index_of_row(lane & 31u);
  uint32_t m = ((row & 1u) ? 0xAAAAu : 0u) ^ ((row & 2u) ? 0xCCCCu : 0u) ^
               ((row & 4u) ? 0xF0F0u : 0u) ^ ((row & 8u) ? 0xFF00u : 0u);
  if (kN == 32 && ((lane >> 5) & (row >> 4))) m ^= 0xFFFFu;
  constexpr uint32_t kUnit = kN == 16 ? 0x3E803E80u : 0x3F803F80u;  // bf16 pair 1/4 or 1
  const uint32_t one = (kN == 16 && (row >> 4) != (lane >> 5)) ? 0u : kUnit;
  u32x4_t v0, v1;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)  // bf16 pair: the unit with the sign bit from the mask
    w[i] = one ? (one | (((m >> (2 * i)) & 1u) << 15) | (((m >> (2 * i + 1)) & 1u) << 31)) : 0u;
  v0 = u32x4_t{w[0], w[1], w[2], w[3]};
  v1 = u32x4_t{w[4], w[5], w[6], w[7]};
  a0 = __builtin_bit_cast(bf16x8_t, v0);
  a1 = __builtin_bit_cast(bf16x8_t, v1);
}

// y[0..15] = (A x)[16h .. 16h+15] / sqrt(kN) for this lane's segment (for
// kN = 32, times `scale` in place of 1/sqrt(32) where the caller folds a
// power of two into it), from
// the lane's 16 inputs x[16h .. 16h+15] (bf16 pairs in lo/hi); for kN = 16
// these are the 16 outputs of one 16-element block, scaled by the operand's
// exact 1/4 (every product and partial sum is the unscaled one times 1/4).
template <int kN>
__device__ __forceinline__ void hadamard_mfma(const bf16x8_t& a0, const bf16x8_t& a1,
                                              u32x4_t lo, u32x4_t hi, float* y,
                                              float scale = kInvSqrt32) {
  f32x16_t acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) y[r] = kN == 32 ? acc[r] * scale : acc[r];
}

// A general 32x32 block matrix M (row-major fp32 in device memory), for the
// learned intra-block rotation: lane l holds M[tau(l % 32)][16 (l / 32) + j],
// j = 0..15 (tau = out_index_of_row, the operand order of hadamard_operands),
// as three bf16 terms t0 + t1 + t2 = M exactly (each term takes the next 8
// significant bits; the differences are exact in fp32); with transpose, M^T.
__device__ __forceinline__ void matrix_operands(const float* __restrict__ M, bool transpose,
                                                bf16x8_t (&a)[3][2]) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t row = out_index_of_row(lane & 31u), k0 = 16u * (lane >> 5);
  uint32_t w[3][8];
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    float t[3][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t k = k0 + (uint32_t)(j + e);
      const float v = transpose ? M[32u * k + row] : M[32u * row + k];
      const float t0 = __uint_as_float(pack_bf16x2(v, 0.0f) << 16);
      const float r1 = v - t0;
      const float t1 = __uint_as_float(pack_bf16x2(r1, 0.0f) << 16);
      t[0][e] = t0;
      t[1][e] = t1;
      t[2][e] = r1 - t1;  // at most 8 significant bits: exact in bf16
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) w[q][j / 2] = pack_bf16x2(t[q][0], t[q][1]);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    a[q][0] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[q][0], w[q][1], w[q][2], w[q][3]});
    a[q][1] = __builtin_bit_cast(bf16x8_t, u32x4_t{w[q][4], w[q][5], w[q][6], w[q][7]});
  }
}

// y[0..15] = (M x)[16h .. 16h + 15] for the lane's segment: products of bf16
// are exact, so the only rounding is the fp32 accumulation of the six MFMAs.
__device__ __forceinline__ void matrix_mfma(const bf16x8_t (&a)[3][2], u32x4_t lo, u32x4_t hi,
                                            float* y) {
  f32x16_t acc = {};
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q][0], __builtin_bit_cast(bf16x8_t, lo), acc,
                                                  0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q][1], __builtin_bit_cast(bf16x8_t, hi), acc,
                                                  0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) y[r] = acc[r];
}

// Largest |y| of 16 fp32 values as a bit pattern, for values that are the
// Hadamard transform or a learned-matrix product of a block: a NaN or Inf
// input makes every output of the block NaN or +-Inf (0 * Inf and 0 * NaN are
// NaN), so a float maximum of magnitudes (which may drop a NaN
// operand in favour of another) still yields a non-finite result for such a
// block, and for finite values its bits order like the magnitudes.
__device__ __forceinline__ uint32_t absmax16_mixed(const float* y) {
  float m = __builtin_fmaxf(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
  for (int k = 2; k < 16; k += 2)  // three-operand maxima
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(y[k])), __builtin_fabsf(y[k + 1]));
  return __float_as_uint(m);
}

// ---- the 32-point transform as two 16x16x32 MFMAs (streaming layout) ----
// A tile is 16 consecutive blocks (1 KB of bf16): lane l = 16 q + n loads the
// 16 bytes of elements 8q .. 8q + 7 of block n, so the 64 lanes of one load
// cover the whole kilobyte. As the B operand of v_mfma_f32_16x16x32_bf16
// (column l % 16, k = 8 (l / 16) .. + 7) that is column n = block n with
// k = element, so both MFMAs below transform all 16 blocks at once. The C
// output gives lane l rows 4 (l / 16) .. + 3 of column l % 16; row m of the
// first A operand is output 8 (m / 4) + m % 4 of H32 and of the second
// output 8 (m / 4) + 4 + m % 4, so lane (n, q) receives the 8 consecutive
// outputs 8q .. 8q + 7 of block n, whose codes are 4 consecutive bytes.
// Operand entries are +-1 (the 1/sqrt(32) follows as one multiply).
__device__ __forceinline__ void hadamard32_spread_operands(bf16x8_t& a0, bf16x8_t& a1) {
  const uint32_t lane = threadIdx.x & 63u, m = lane & 15u, k0 = 8u * (lane >> 4);
  const uint32_t o0 = 8u * (m >> 2) + (m & 3u), o1 = o0 + 4u;
  uint32_t w0[4], w1[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const uint32_t k = k0 + (uint32_t)j;
    w0[j / 2] = 0x3F803F80u | (((uint32_t)__builtin_popcount(o0 & k) & 1u) << 15) |
                (((uint32_t)__builtin_popcount(o0 & (k + 1u)) & 1u) << 31);
    w1[j / 2] = 0x3F803F80u | (((uint32_t)__builtin_popcount(o1 & k) & 1u) << 15) |
                (((uint32_t)__builtin_popcount(o1 & (k + 1u)) & 1u) << 31);
  }
  a0 = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w0[2], w0[3]});
  a1 = __builtin_bit_cast(bf16x8_t, u32x4_t{w1[0], w1[1], w1[2], w1[3]});
}

// y[0..7] = outputs 8q .. 8q + 7 of H32 x / sqrt(32) for the lane's block,
// from its 8 inputs (elements 8q .. 8q + 7): see hadamard32_spread_operands.
__device__ __forceinline__ void hadamard32_spread(const bf16x8_t& a0, const bf16x8_t& a1,
                                                  u32x4_t x, float* y) {
  const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, x);
  const f32x4_t c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, z, 0, 0, 0);
  const f32x4_t c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, z, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = c0[i] * kInvSqrt32;
    y[4 + i] = c1[i] * kInvSqrt32;
  }
}

// Largest |y| of 8 fp32 values as a bit pattern, for Hadamard outputs (the
// reasoning of absmax16_mixed: a non-finite block makes all 8 non-finite).
__device__ __forceinline__ uint32_t absmax8_mixed(const float* y) {
  float m = __builtin_fmaxf(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
  for (int k = 2; k < 8; k += 2)
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(y[k])), __builtin_fabsf(y[k + 1]));
  return __float_as_uint(m);
}

// Largest of v over the lanes l, l ^ 16, l ^ 32, l ^ 48 (one block of the
// streaming layout), by gfx950's row and lane-half swaps.
__device__ __forceinline__ uint32_t max_spread4(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)r[0], (uint32_t)r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

// MXFP4 / MXINT4 of the lane's 8 outputs, the block spread over 4 lanes.
template <bool kFloor, bool kMixed>
__device__ __forceinline__ void mx_quant8_spread(const float* y, uint32_t& w, uint32_t& byte) {
  byte = e8m0_byte<kFloor>(max_spread4(kMixed ? absmax8_mixed(y) : absmax_bits<8>(y)));
  w = byte == 0xFFu ? 0u : cvt8_f32(y, e8m0_operand(byte));
}

template <bool kFloor, bool kMixed>
__device__ __forceinline__ void mxint_quant8_spread(const float* y, uint32_t& w, uint32_t& byte) {
  byte = mxint_byte<kFloor>(max_spread4(kMixed ? absmax8_mixed(y) : absmax_bits<8>(y)));
  w = byte == 0xFFu ? 0u : int4x8_f32(y, 129 - (int)byte);
}

// Larger of v in lanes l and l ^ 32 (gfx950 lane-half swap).
__device__ __forceinline__ uint32_t max_xor32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}

// MXFP4-quantize the lane's 16 outputs; the block spans lanes l and l ^ 32.
// kMixed: y is a Hadamard transform of the block (see absmax16_mixed).
template <bool kFloor, bool kMixed>
__device__ __forceinline__ void mx_quant16_pair(const float* y, uint32_t& w0, uint32_t& w1,
                                                uint32_t& byte) {
  const uint32_t m = max_xor32(kMixed ? absmax16_mixed(y) : absmax_bits<16>(y));
  byte = e8m0_byte<kFloor>(m);
  if (byte == 0xFFu) {
    w0 = w1 = 0u;
  } else {
    const float s = e8m0_operand(byte);
    w0 = cvt8_f32(y, s);
    w1 = cvt8_f32(y + 8, s);
  }
}

// MXINT4 of the lane's 16 outputs (block across lanes l and l ^ 32).
template <bool kFloor, bool kMixed>
__device__ __forceinline__ void mxint_quant16_pair(const float* y, uint32_t& w0, uint32_t& w1,
                                                   uint32_t& byte) {
  const uint32_t m = max_xor32(kMixed ? absmax16_mixed(y) : absmax_bits<16>(y));
  byte = mxint_byte<kFloor>(m);
  const int sh = 129 - (int)byte;
  w0 = byte == 0xFFu ? 0u : int4x8_f32(y, sh);
  w1 = byte == 0xFFu ? 0u : int4x8_f32(y + 8, sh);
}

// Largest magnitude of 16 fp32 values (a NaN operand may be dropped).
__device__ __forceinline__ float absmax16f(const float* y) {
  float m = __builtin_fmaxf(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
  for (int k = 2; k < 16; k += 2)
    m = __builtin_fmaxf(__builtin_fmaxf(m, __builtin_fabsf(y[k])), __builtin_fabsf(y[k + 1]));
  return m;
}

// NVFP4 of the lane's 16 values, one whole 16-element block (the arithmetic of
// nv_block_code and the RaZeR selection of the streaming NVFP4 quantizer,
// here inside one lane). Non-finite values give unspecified codes.
template <bool kRazer>
__device__ __forceinline__ void nv_quant16(const float* y, const NvScale& ns, const float* rcp_tab,
                                           uint32_t& w0, uint32_t& w1, uint32_t& byte) {
  const uint32_t sb = nv_block_code(absmax16f(y), ns);
  w0 = w1 = 0u;
  byte = 0u;
  if (sb != 0u) {
    const float r = rcp_tab[sb];
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = y[k] * r;
    w0 = cvt8_f32(v, 1.0f);
    w1 = cvt8_f32(v + 8, 1.0f);
    byte = sb;
    if (kRazer) {
      float dsum = 0.0f;
      float g[16];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        g[k] = razer_gain(v[k]);
        g[k + 8] = razer_gain(v[k + 8]);
        dsum -= __builtin_copysignf(g[k], v[k]);
        dsum -= __builtin_copysignf(g[k + 8], v[k + 8]);
      }
      const uint32_t cm0 = razer_flags8(g), cm1 = razer_flags8(g + 8);
      const uint32_t sel = dsum > 0.0f ? 1u : 0u;
      w0 = razer_apply(w0, cm0, sel);
      w1 = razer_apply(w1, cm1, sel);
      byte |= sel << 7;
    }
  }
}

// ========================= butterfly implementation =========================
// Lane q of a group of four holds elements 8q..8q+7: bits 0-2 of the index
// are butterflies inside the lane, bits 3-4 exchanges with lane q ^ 1 and
// q ^ 2 (DPP), folded as partner + (+-own) and, for the last stage,
// partner * c + (+-c * own) with c = 1/sqrt(32).
__device__ __forceinline__ float dpp1(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0xB1,
                                                               0xF, 0xF, true));
}
__device__ __forceinline__ float dpp2(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x4E,
                                                               0xF, 0xF, true));
}

__device__ __forceinline__ void hadamard_butterfly(float* v, uint32_t q) {
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
  const float s1 = (q & 1u) ? -1.0f : 1.0f;
  const float s2 = (q & 2u) ? -kInvSqrt32 : kInvSqrt32;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float u = s1 * v[k];
    v[k] = dpp1(v[k]) + u;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float u = s2 * v[k];
    v[k] = __builtin_fmaf(dpp2(v[k]), kInvSqrt32, u);
  }
}

template <bool kFloor>
__device__ __forceinline__ void mx_quant8_quad(const float* y, uint32_t& w, uint32_t& byte) {
  uint32_t m = absmax_bits<8>(y);
  m = max(m, dpp_xor1(m));
  m = max(m, dpp_xor2(m));
  byte = e8m0_byte<kFloor>(m);
  w = byte == 0xFFu ? 0u : cvt8_f32(y, e8m0_operand(byte));
}

constexpr int kWaves = kThreads / 64;  // waves per work-group

struct RotGeom {
  int32_t rows, cols;
  int32_t bpr;   // 32-element segments per row (MXFP4 blocks; two NVFP4 blocks each)
  uint32_t nblk; // rows * bpr
  int32_t spr;   // scale bytes per row: cols / block
  int32_t s_ext; // bytes from a row's first scale byte past its last one
  bool s_gemm;   // MXFP4 scale bytes in the GEMM order
  int64_t ld_x, ld_c, ld_s, ld_rot;
};

// Formats of the rotation kernels (the C ABI's format numbers): MXFP4 and
// MXINT4 (32-point transform), NVFP4 (16-point), the NVFP4 pre-pass that
// only finds the largest rotated magnitude (for a computed tensor scale), and
// MXFP4 after a learned 32x32 block matrix instead of the Hadamard.
enum RotFmt : int { kFmtMx = 0, kFmtNv = 1, kFmtMxInt = 2, kFmtNvAmax = 3, kFmtMxMat = 4 };

inline RotGeom rot_geom(const Shape& s, int64_t ld_rot, int block = 32) {
  RotGeom g;
  g.rows = (int32_t)s.rows;
  g.cols = (int32_t)s.cols;
  g.bpr = (int32_t)(s.cols / 32);
  g.nblk = (uint32_t)(s.rows * (s.cols / 32));
  g.spr = (int32_t)(s.cols / block);
  g.s_gemm = s.s_gemm;
  // GEMM order: block b of a row at 256 (b / 8) + b % 8
  g.s_ext = !s.s_gemm ? g.spr : g.spr == 0 ? 0 : 256 * ((g.spr + 7) / 8 - 1) + 8;
  g.ld_x = s.ld_x;
  g.ld_c = s.ld_c;
  g.ld_s = s.ld_s;
  g.ld_rot = ld_rot;
  return g;
}

// Where work-group i of an amax pre-pass leaves its partial: the code slot of
// chunk i (row-major chunks of 8 elements, 4 code bytes each), which the
// quantize pass overwrites afterwards.
__device__ __forceinline__ uint32_t* amax_partial_slot(uint8_t* codes, uint32_t i,
                                                       const RotGeom& g) {
  const uint32_t cpr = (uint32_t)g.cols / 8u, r = i / cpr;
  return reinterpret_cast<uint32_t*>(codes + r * g.ld_c + 4 * (int64_t)(i - r * cpr));
}

// Work-group maximum of a non-negative per-lane value; lane 0 of the
// work-group receives it. red: kWaves floats of shared memory.
template <int kW = kWaves>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kW; ++i) m = __builtin_fmaxf(m, red[i]);
  return m;
}


// ---- per-lane permutation entries (MFMA tile layout) ----------------------
// Lane (n, h) of wave w handles, for i < kTpw, tile t = w + kW i (kW waves): block
// b = 32 t + n, elements e0 .. e0 + 15 with e0 = 32 b + 16 h, whose row
// positions are perm[e0 .. e0 + 15]. The positions are the same for every
// row, so a lane loads them once and keeps them as LDS byte offsets (clamped
// to the row), packed in pairs.

// Issue the loads of this lane's perm entries (16 per tile, zeros for tiles
// past the row).
template <int kTpw, int kW = kWaves>
__device__ __forceinline__ void load_lane_perm(const int32_t* __restrict__ perm,
                                               const RotGeom& g, i32x4_t (*v)[4]) {
  const rsrc_t rp = make_rsrc(perm, 4u * (uint32_t)g.cols);
  const int32_t lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int32_t b = 32 * (w + kW * i) + n;
    const uint32_t o = b < g.bpr ? 4u * (32u * b + 16u * h) : kOob;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[i][q] = __builtin_bit_cast(
          i32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, o == kOob ? kOob : o + 16u * q, 0, 0));
  }
}

// Clamp to the row, convert to byte offsets packed in pairs, and return the
// largest run length G in {8, 4, 2, 1} such that the lane's indices form
// aligned runs of G consecutive channels (lanes without a block: 8).
template <int kTpw, int kW = kWaves>
__device__ __forceinline__ int pack_lane_perm(const i32x4_t (*v)[4], const RotGeom& g,
                                              uint32_t (*off)[8]) {
  const int32_t lane = threadIdx.x & 63, n = lane & 31, w = threadIdx.x >> 6;
  const int32_t cmax = g.cols - 1;
  bool r8 = true, r4 = true, r2 = true;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    int32_t p[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[4 * q + 0] = min(max(v[i][q].x, 0), cmax);
      p[4 * q + 1] = min(max(v[i][q].y, 0), cmax);
      p[4 * q + 2] = min(max(v[i][q].z, 0), cmax);
      p[4 * q + 3] = min(max(v[i][q].w, 0), cmax);
    }
    if (32 * (w + kW * i) + n < g.bpr) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        r8 = r8 && p[k] == p[k & 8] + (k & 7) && (p[k & 8] & 7) == 0;
        r4 = r4 && p[k] == p[k & 12] + (k & 3) && (p[k & 12] & 3) == 0;
        r2 = r2 && p[k] == p[k & 14] + (k & 1) && (p[k & 14] & 1) == 0;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) off[i][k] = 2u * (uint32_t)p[2 * k] | (2u * (uint32_t)p[2 * k + 1]) << 16;
  }
  return r8 ? 8 : r4 ? 4 : r2 ? 2 : 1;
}

}  // namespace fp4
