// fp4_device.hpp -- gfx950 device helpers for block-scaled FP4 kernels.
//
// Element code: FP4 E2M1, sign << 3 | magnitude index, magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} ("RaZeR: Pushing the Limits of NVFP4 Quantization
// with Redundant Zero Remapping", technical summary sec. 1). Rounding to E2M1
// uses gfx950's v_cvt_scalef32_pk_fp4_{bf16,f32}: it divides by the E8M0 scale
// held in the exponent field of its fp32 scale operand, rounds to nearest with
// ties to the even code, saturates at 6 and keeps the sign of zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // work-group size of the streaming kernels

// ---- buffer resources -----------------------------------------------------
// A raw buffer resource covers [base, base + bytes) and the hardware
// range-checks every access through it: a load at an offset past the end
// returns zero without touching memory, a store there is dropped. Kernels
// that keep loads in flight across rows use this to issue every load and store
// unconditionally (offset kOob for a lane or row with nothing to do). With no
// branch around a memory operation, the compiler knows how many operations
// were issued after each load and waits for that load alone, instead of
// draining the whole vector-memory counter, which on gfx9 also counts stores.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;  // beyond every resource (byte counts < 2^31)
constexpr int kNt = 2;                  // cache policy bit: nontemporal

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3: raw (unswizzled, stride 0) buffer with 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// ---- scale byte placement --------------------------------------------------
// Row-major: row r at r * ld_s, block b at b. GEMM order (MXFP4): rows in
// groups of 32 at stride ld_s; inside a group, the 8 blocks of each
// 256-element step of the row are 256 contiguous bytes, row r % 32 at
// 8 (r % 32), block b at 256 (b / 8) + b % 8. Row and block parts add.
__device__ __forceinline__ int64_t scale_row_off(int64_t r, int64_t ld_s, bool gemm) {
  return gemm ? (r >> 5) * ld_s + 8 * (r & 31) : r * ld_s;
}
__device__ __forceinline__ uint32_t scale_col_off(uint32_t b, bool gemm) {
  return gemm ? ((b >> 3) << 8) | (b & 7u) : b;
}

// Bit casts take a scalar by value: clang's __builtin_bit_cast applied
// directly to an ext-vector element (v.y) reads element 0 instead.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
__device__ __forceinline__ u16x2_t as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2_t, v); }

// ---- cross-lane ---------------------------------------------------------
// quad_perm DPP controls: [1,0,3,2] swaps lane pairs, [2,3,0,1] swaps halves
// of each group of four lanes.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ float dpp_xor1f(float v) {
  return __uint_as_float(dpp_xor1(__float_as_uint(v)));
}
__device__ __forceinline__ float dpp_xor2f(float v) {
  return __uint_as_float(dpp_xor2(__float_as_uint(v)));
}

// ---- bf16 ---------------------------------------------------------------
// Largest |x| of eight bf16 held in four dwords, as a 16-bit pattern (bits
// order like magnitudes for non-negative values; NaN > Inf > finite).
__device__ __forceinline__ uint32_t absmax8_bf16(u32x4_t d) {
  const u16x2_t m = {0x7FFF, 0x7FFF};
  u16x2_t a = as_u16x2(d.x) & m;
  u16x2_t b = as_u16x2(d.y) & m;
  u16x2_t c = as_u16x2(d.z) & m;
  u16x2_t e = as_u16x2(d.w) & m;
  u16x2_t r = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                        __builtin_elementwise_max(c, e));
  return r.x > r.y ? r.x : r.y;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  float2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));  // RNE
}

// ---- E8M0 shared exponent (MXFP4) -----------------------------------------
// From the fp32 bit pattern m of a block's largest magnitude. Default: the
// smallest e in [-127, 127] with amax <= 6 * 2^e. For normal amax =
// (1 + f) * 2^(E-127), 6 * 2^e = 1.5 * 2^(e+2), so e = E - 129 when f <= 0.5
// and E - 128 otherwise; byte = e + 127, clamped to 0 for tiny amax.
// kFloor: e = floor(log2 amax) - 2 = E - 129. Inf/NaN -> 0xFF.
template <bool kFloor>
__device__ __forceinline__ uint32_t e8m0_byte(uint32_t m) {
  if (m >= 0x7F800000u) return 0xFFu;
  int E = (int)(m >> 23);
  int b = kFloor ? E - 2 : E - 2 + ((m & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  return (uint32_t)(b < 0 ? 0 : b);
}

__device__ __forceinline__ float e8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// Eight values (four bf16 pairs) -> eight E2M1 codes in one dword, element k
// in nibble k.
__device__ __forceinline__ uint32_t cvt8_bf16(u32x4_t d, float scale) {
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, as_bf16x2(d.x), scale, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, as_bf16x2(d.y), scale, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, as_bf16x2(d.z), scale, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(o, as_bf16x2(d.w), scale, 3);
  return o;
}

__device__ __forceinline__ uint32_t cvt8_f32(const float* y, float scale) {
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[0], y[1], scale, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[2], y[3], scale, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[4], y[5], scale, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, y[6], y[7], scale, 3);
  return o;
}

// ---- MXINT4 -----------------------------------------------------------------
// Element: a two's complement nibble k in [-8, 7] with value k / 4, one E8M0
// byte per 32-element block. Default scale: the smallest e in [-127, 127]
// with amax <= 1.75 * 2^e (the top symmetric code, so nothing is clipped):
// for normal amax = (1 + f) 2^(E - 127) that is e = E - 127 + [f > 0.75],
// capped at 127 (larger magnitudes saturate); a subnormal amax = f 2^-149
// fits e = -127 while f <= 1.75 * 2^22. Floor rule: e = floor(log2 amax) =
// E - 127 (byte 0 for zero and subnormal amax). m: fp32 bits of amax.
template <bool kFloor>
__device__ __forceinline__ uint32_t mxint_byte(uint32_t m) {
  if (m >= 0x7F800000u) return 0xFFu;
  const uint32_t E = m >> 23, f = m & 0x7FFFFFu;
  if (kFloor) return E;
  if (E == 0u) return f > 0x700000u ? 1u : 0u;
  const uint32_t b = E + (f > 0x600000u ? 1u : 0u);
  return b > 254u ? 254u : b;
}

// Eight values -> eight nibbles, element k in nibble k: y 2^sh (sh = 2 - e,
// an exact rescale wherever the result can round to a non-zero k) clamped to
// [-7, 7], then rounded to the nearest integer with ties to even by adding
// 1.5 * 2^23, which leaves k in the low mantissa bits (two's complement mod 16).
__device__ __forceinline__ uint32_t int4x8_f32(const float* y, int sh) {
  uint32_t o = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float t = __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(y[k], sh), -7.0f, 7.0f);
    o |= (__float_as_uint(t + 12582912.0f) & 15u) << (4 * k);
  }
  return o;
}

// Eight nibbles -> bf16 pairs of k 2^(e - 2), exact (k has at most 3
// significant bits); the NaN scale byte decodes to NaN.
__device__ __forceinline__ u32x4_t int4x8_decode(uint32_t w, uint32_t byte) {
  const int sh = (int)byte - 129;
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v[k] = __builtin_amdgcn_ldexpf((float)((int32_t)(w << (28 - 4 * k)) >> 28), sh);
  if (byte == 0xFFu) return u32x4_t{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  return u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
}

// Eight nibbles -> bf16 pairs of k itself (exact), for a scale applied later.
__device__ __forceinline__ u32x4_t int4x8_decode_unit(uint32_t w) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (float)((int32_t)(w << (28 - 4 * k)) >> 28);
  return u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
}

__device__ __forceinline__ void widen8(u32x4_t d, float* v) {
  v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
  v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
  v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
  v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
}

// ---- E4M3 block scale (NVFP4) ---------------------------------------------
// OCP E4M3 "fn": bias 7, subnormals m * 2^-9, largest finite 448, 0x7F NaN.
// Nearest code to s >= 0 with ties to the even code, saturating at 448:
// gfx950's v_cvt_pk_fp8_f32 rounds to the OCP E4M3 code this way (checked on
// MI355X against an integer-arithmetic encoder -- subnormals m 2^-9 by an
// exact rescale and round half even, normals by rounding the 20 dropped
// mantissa bits with ties to even -- for every non-negative fp32 bit pattern
// up to +Inf) except that it gives NaN (0x7F) where the value rounds past
// 448, so the value is first clamped to 448 (a NaN s, which fminf drops, also
// gives 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s, 448.0f), 0.0f, 0, false) &
         0xFFu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  const float nrm = __uint_as_float((((mag >> 3) + 120u) << 23) | ((mag & 7u) << 20));
  const float sub = (float)mag * 0x1p-9f;
  float v = mag >= 8u ? nrm : sub;
  if (mag == 0x7Fu) v = __builtin_nanf("");
  return (c & 0x80u) ? -v : v;
}

// ---- RaZeR gain ---------------------------------------------------------
// Squared-error gain of replacing an element's standard code by the special
// value 5 of the same sign: with d = |y| - 5, the standard neighbour is 4 or
// 6 and (|y| - std)^2 - d^2 = 1 - 2|d| on |d| < 0.5, and no gain outside.
// Exact in fp32: for |y| in [2.5, 10], |y| - 5 is exact (Sterbenz), and
// where the gain is positive |y| lies in [4, 8), so d is a multiple of 2^-21
// and 1 - 2|d| a multiple of 2^-20 in (0, 1]; elsewhere 1 - 2|d| < 0 whatever
// the rounding and is clamped to 0. A block sum of 16 such gains, signed (at
// most 16 in magnitude, on the 2^-20 grid), is exact too.
__device__ __forceinline__ float razer_gain(float y) {
  const float d = __builtin_fabsf(y) - 5.0f;
  return __builtin_amdgcn_fmed3f(__builtin_fmaf(-2.0f, __builtin_fabsf(d), 1.0f), 0.0f, 1.0f);
}

// Code dword with every nibble whose magnitude is zero cleared to 0x0.
__device__ __forceinline__ uint32_t canonical_zero(uint32_t w) {
  uint32_t nz = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;  // bit 3 set iff |code| != 0
  return w & (nz | 0x77777777u);
}

// ---- NVFP4 block scale ------------------------------------------------------
// Per block: s_raw = RN(amax / d6) with d6 = RN(6 s_t), s_b = E4M3(s_raw),
// r = RN(1 / RN(e4m3(s_b) s_t)), y = RN(x r). Two reductions of the divisions:
//  - r depends only on the 7-bit code s_b, so a work-group tabulates it once
//    (nv_rcp_table, 128 correctly rounded divisions) and a block reads it;
//  - with y6 = RN(1 / d6), q = RN(amax y6) and the exact residual
//    fma(-q, d6, amax), q' = fma(residual, y6, q) is the correctly rounded
//    quotient whenever the residual does not underflow (amax >= 2^-100).
//    With d6 in [2^-80, 2^125] every quotient that can round to a code other
//    than 0 or 0x7E comes from such an amax; smaller ones stay below 2^-11
//    (code 0) and overflowing ones give Inf or NaN, both code 0x7E like the
//    Inf of the true division. (Checked against IEEE division for all finite
//    bf16 amax and 40000 divisors.) Outside that range of d6 the caller
//    passes rcp_quotient = false and the quotient is divided.
struct NvScale {
  float d6, y6;
  bool rcp_quotient;  // uniform
};

__device__ __forceinline__ NvScale nv_scale_setup(float s_t) {
  NvScale n;
  n.d6 = 6.0f * s_t;
  n.y6 = 1.0f / n.d6;
  n.rcp_quotient = n.d6 >= 0x1p-80f && n.d6 <= 0x1p125f;
  return n;
}

// E4M3 code of the block with largest magnitude amax.
__device__ __forceinline__ uint32_t nv_block_code(float amax, const NvScale& n) {
  float s_raw;
  if (__builtin_expect(n.rcp_quotient, 1)) {
    const float q = amax * n.y6;
    s_raw = __builtin_fmaf(__builtin_fmaf(-q, n.d6, amax), n.y6, q);
  } else {
    s_raw = amax / n.d6;
  }
  return e4m3_encode(s_raw);
}

// tab[c] = RN(1 / RN(e4m3(c) s_t)) for the 128 codes; the first 128 lanes of
// the work-group write it, the caller synchronises before reading.
__device__ __forceinline__ void nv_rcp_table(float* tab, float s_t) {
  if (threadIdx.x < 128) tab[threadIdx.x] = 1.0f / (e4m3_decode(threadIdx.x) * s_t);
}

// RaZeR: apply the selector to a code word w (standard codes) given the
// candidate flags cm (bit 3 of each nibble: the element's gain is > 0). A
// candidate's standard code is non-zero, so its bit 3 is the sign of y: it
// takes the special code 0x8 when that sign is the selected one. Zeros are
// stored as 0x0.
__device__ __forceinline__ uint32_t razer_apply(uint32_t w, uint32_t cm, uint32_t sel) {
  const uint32_t spm = cm & ~(w ^ (sel ? 0x88888888u : 0u));
  w = canonical_zero(w);
  // nibble mask 0xF where spm has bit 3: 15 b 16^k summed = (spm << 1) -
  // (spm >> 3) modulo 2^32 (full-rate shifts in place of a 32-bit multiply)
  return (w & ~((spm << 1) - (spm >> 3))) | spm;
}

// Gain flags of eight elements (see razer_gain): bit 3 of nibble k is set iff
// g[k] > 0. The gains lie in [+0, 1] and the positive ones are multiples of
// 2^-22, so the FP4 conversion at scale 2^-100 sends each positive gain far
// past 6, which saturates to code 7, and +0 to code 0 (checked on the GPU):
// bit 2 of each nibble is the flag. Four conversions for eight elements, in
// place of three integer instructions per element.
__device__ __forceinline__ uint32_t razer_flags8(const float* g) {
  return (cvt8_f32(g, 0x1p-100f) & 0x44444444u) << 1;
}

// ---- RaZeR for weights --------------------------------------------------------
// Weights take a 6-bit E3M3 block scale ("fn"-style: bias 3, subnormals
// m 2^-5, largest 30), freeing two bits that select the special value of code
// 0x8 among {+5, -5, +2.5, -2.5} (selector 0..3 in bits 6-7 of the scale byte;
// +-2.5 is the second pair, chosen offline). s_t = amax_t / 180 maps the
// largest block onto 6 * 30.
constexpr float kWeightPair = 2.5f;

// Nearest E3M3 code to s >= 0, ties to the even code, saturating at 30 (no
// hardware format has this layout): subnormals m 2^-5 (below 2^-2) by an exact
// rescale and round half even; normals by rounding the 20 dropped mantissa
// bits with ties to even and rebiasing 127 -> 3.
__device__ __forceinline__ uint32_t e3m3_encode(float s) {
  const uint32_t sub = (uint32_t)__builtin_rintf(s * 32.0f);
  uint32_t u = __float_as_uint(s);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  const uint32_t nrm = (u >> 20) - (124u << 3);
  const uint32_t c = s < 0x1p-2f ? sub : nrm;
  return s <= 30.0f ? c : 63u;
}

__device__ __forceinline__ float e3m3_decode(uint32_t c) {
  const uint32_t mag = c & 63u;
  const float nrm = __uint_as_float((((mag >> 3) + 124u) << 23) | ((mag & 7u) << 20));
  const float sub = (float)mag * 0x1p-5f;
  return mag >= 8u ? nrm : sub;
}

// E3M3 block code of a block maximum (the quotient as in nv_block_code).
__device__ __forceinline__ uint32_t nvw_block_code(float amax, const NvScale& n) {
  float s_raw;
  if (__builtin_expect(n.rcp_quotient, 1)) {
    const float q = amax * n.y6;
    s_raw = __builtin_fmaf(__builtin_fmaf(-q, n.d6, amax), n.y6, q);
  } else {
    s_raw = amax / n.d6;
  }
  return e3m3_encode(s_raw);
}

// r[c] = RN(1 / RN(e3m3(c) * s_t)) for the 64 codes (threads 0..63).
__device__ __forceinline__ void nvw_rcp_table(float* tab, float s_t) {
  if (threadIdx.x < 64) tab[threadIdx.x] = 1.0f / (e3m3_decode(threadIdx.x) * s_t);
}

// Squared-error gain of the special value 2.5 (same sign): its standard
// neighbours 2 and 3 are 0.5 away, so with d = |y| - 2.5 the gain is
// 0.25 - |d| on |d| < 0.25 and none outside. Exact in fp32: where it is
// positive |y| lies in [2, 4) (d a multiple of 2^-22, Sterbenz), and a block
// sum of 16 (at most 4, on the 2^-22 grid) is exact too.
__device__ __forceinline__ float razer_gain_pair2(float y) {
  const float d = __builtin_fabsf(y) - kWeightPair;
  // 0.25 - |d| <= 0.25, so clamping to [0, 1] (the instruction's clamp bit)
  // is clamping to [0, 0.25]
  return __builtin_amdgcn_fmed3f(0.25f - __builtin_fabsf(d), 0.0f, 1.0f);
}

__device__ __forceinline__ float weight_special(uint32_t byte) {
  const uint32_t sel = (byte >> 6) & 3u;
  const float mag = sel >= 2u ? kWeightPair : 5.0f;
  return (sel & 1u) ? -mag : mag;
}

}  // namespace fp4
