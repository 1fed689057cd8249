// unrotate_kernels.hpp -- dequantization (MXFP4, MXINT4, NVFP4) with the
// inverse of the two-level rotation: the kernel and its launch templates,
// compiled per format in unrotate_mx.hip, unrotate_int.hip and unrotate_nv.hip.
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2: the rotation is orthogonal, so decoding in the original
// basis applies H (its own inverse) and then the inverse permutation.
#ifndef FP4_UNROTATE_KERNELS_HPP
#define FP4_UNROTATE_KERNELS_HPP

#include <utility>

#include "launch.hpp"
#include "rotation.hpp"

namespace fp4 {

// ============================ inverse rotation ==============================
// Lane (n, h) of wave w decodes, per row and for i < kTpw, the 16 elements
// 16h .. 16h + 15 of block b = 32 (w + kWaves i) + n -- the MFMA tile layout
// of the forward kernel. Decoded MXFP4 values (code * 2^e) are exact in bf16,
// and the 32 products of a block's Hadamard row sum exactly in fp32, so the
// transform runs on the matrix cores (two v_mfma_f32_32x32x16_bf16 per tile)
// and gives the same fp32 results as any exact-sum order; then y * 1/sqrt(32)
// is rounded to bf16. Element j = e0 + k goes to column perm[j]: the lane
// scatters its 16 values into an LDS copy of the output row (2-byte writes,
// or wider ones when perm moves aligned runs of channels), and the
// work-group writes the row out with coalesced 16-byte stores. Rows alternate
// between two LDS buffers with one barrier per row; the codes and scales of
// the next kAhead rows are in flight in registers. Without a permutation the
// row takes the same way with the identity (16-byte LDS writes): each lane
// storing its 32 contiguous bytes directly left every store instruction half
// of each 128-byte line (MXFP4, 16384 x 8192: 74.8 us, against 61.3 with a
// permutation).

// The entries of the identity permutation in the layout of load_lane_perm
// (zeros for tiles past the row).
template <int kTpw, int kW = kWaves>
__device__ __forceinline__ void identity_lane_perm(const RotGeom& g, i32x4_t (*v)[4]) {
  const int32_t lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int32_t b = 32 * (w + kW * i) + n;
    const int32_t e0 = b < g.bpr ? 32 * b + 16 * h : 0;
    const int32_t d = b < g.bpr ? 1 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[i][q] = i32x4_t{e0 + d * 4 * q, e0 + d * (4 * q + 1), e0 + d * (4 * q + 2),
                        e0 + d * (4 * q + 3)};
  }
}

// Per-row buffer resources of the inverse (empty for rows past the end).
struct UnrotRsrc {
  rsrc_t c, s, o;
};
__device__ __forceinline__ UnrotRsrc unrot_rsrc(const uint8_t* codes, const uint8_t* scales,
                                                uint16_t* out, int32_t r, const RotGeom& g) {
  const bool in = r < g.rows;
  const int64_t rr = in ? r : 0;
  UnrotRsrc q;
  q.c = make_rsrc(codes + rr * g.ld_c, in ? (uint32_t)g.cols / 2u : 0u);
  q.s = make_rsrc(scales + rr * g.ld_s, in ? (uint32_t)g.spr : 0u);
  q.o = make_rsrc(out + rr * g.ld_x, in ? 2u * (uint32_t)g.cols : 0u);
  return q;
}

// Codes (8 bytes) and scale byte of the lane's half-blocks of one row.
template <int kTpw>
struct RowCodes {
  u32x2_t c[kTpw];
  uint32_t s[kTpw];
};

// kNv: the lane's 16 elements are NVFP4 block 2 b + h with its own scale byte.
template <int kTpw, bool kNv, int kW = kWaves>
__device__ __forceinline__ void load_codes(const UnrotRsrc& q, const RotGeom& g,
                                           RowCodes<kTpw>& rc) {
  const uint32_t lane = threadIdx.x & 63u, n = lane & 31u, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int32_t b = 32 * ((int32_t)(threadIdx.x >> 6) + kW * i) + (int32_t)n;
    const bool ok = b < g.bpr;
    rc.c[i] = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(q.c, ok ? 16u * b + 8u * h : kOob, 0, kNt));
    const uint32_t so = kNv ? 2u * b + h : (uint32_t)b;
    rc.s[i] = __builtin_amdgcn_raw_buffer_load_b8(q.s, ok ? so : kOob, 0, 0);
  }
}

// bf16 outputs of one MXFP4 (kInt: MXINT4) tile: decode (exact), Hadamard
// (kHad), scale, round.
template <bool kHad, bool kInt>
__device__ __forceinline__ void unrotate_tile(u32x2_t c, uint32_t sbyte, const bf16x8_t& a0,
                                              const bf16x8_t& a1, u32x4_t& lo, u32x4_t& hi) {
  if constexpr (kInt && kHad) {
    // The block scale 2^(e - 2) is a power of two, so it can follow the
    // Hadamard: k decodes to bf16 as is, the integer sums (at most 256 in
    // magnitude) are exact, and one multiply by 2^(e - 2) / sqrt(32) rounds
    // the exact real result once, as scaling first would, while that factor
    // is a normal float (byte >= 6). It also keeps large scales right: scaled
    // first, k 2^(e - 2) overflows bf16 for byte 254 (k = -8) and partial sums
    // overflow fp32 from byte 249 on, where the transformed value may still
    // be finite. Tiny scales (bytes 0..5) and NaN (255) decode scaled.
    // The MFMA combines lanes, so it runs on every lane outside the choice;
    // the two lanes of a block share its byte and so its choice.
    const uint32_t byte = sbyte & 0xFFu;
    const bool fast = byte >= 6u && byte != 0xFFu;
    u32x4_t dl, dh;
    if (fast) {
      dl = int4x8_decode_unit(c.x);
      dh = int4x8_decode_unit(c.y);
    } else {
      dl = int4x8_decode(c.x, byte);
      dh = int4x8_decode(c.y, byte);
    }
    float y[16];
    hadamard_mfma<32>(a0, a1, dl, dh, y,
                      fast ? __builtin_amdgcn_ldexpf(kInvSqrt32, (int)byte - 129) : kInvSqrt32);
    lo = u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                 pack_bf16x2(y[6], y[7])};
    hi = u32x4_t{pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]), pack_bf16x2(y[12], y[13]),
                 pack_bf16x2(y[14], y[15])};
    return;
  } else if constexpr (kInt) {
    lo = int4x8_decode(c.x, sbyte & 0xFFu);
    hi = int4x8_decode(c.y, sbyte & 0xFFu);
  } else {
    const float s = e8m0_operand(sbyte & 0xFFu);
#define FP4_CVT2(w, k) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, k))
    const uint32_t d[8] = {FP4_CVT2(c.x, 0), FP4_CVT2(c.x, 1), FP4_CVT2(c.x, 2), FP4_CVT2(c.x, 3),
                           FP4_CVT2(c.y, 0), FP4_CVT2(c.y, 1), FP4_CVT2(c.y, 2), FP4_CVT2(c.y, 3)};
#undef FP4_CVT2
    lo = u32x4_t{d[0], d[1], d[2], d[3]};
    hi = u32x4_t{d[4], d[5], d[6], d[7]};
  }
  if (kHad) {
    float y[16];
    hadamard_mfma<32>(a0, a1, lo, hi, y);
    lo = u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                 pack_bf16x2(y[6], y[7])};
    hi = u32x4_t{pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]), pack_bf16x2(y[12], y[13]),
                 pack_bf16x2(y[14], y[15])};
  }
}

// MXFP4 after a learned block matrix M: decode (exact in bf16), multiply by
// M^T (m holds its operands), round to bf16.
__device__ __forceinline__ void unrotate_tile_mat(u32x2_t c, uint32_t sbyte,
                                                  const bf16x8_t (&m)[3][2], u32x4_t& lo,
                                                  u32x4_t& hi) {
  const float s = e8m0_operand(sbyte & 0xFFu);
#define FP4_CVT2(w, k) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, k))
  const uint32_t d[8] = {FP4_CVT2(c.x, 0), FP4_CVT2(c.x, 1), FP4_CVT2(c.x, 2), FP4_CVT2(c.x, 3),
                         FP4_CVT2(c.y, 0), FP4_CVT2(c.y, 1), FP4_CVT2(c.y, 2), FP4_CVT2(c.y, 3)};
#undef FP4_CVT2
  float y[16];
  matrix_mfma(m, u32x4_t{d[0], d[1], d[2], d[3]}, u32x4_t{d[4], d[5], d[6], d[7]}, y);
  lo = u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
               pack_bf16x2(y[6], y[7])};
  hi = u32x4_t{pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]), pack_bf16x2(y[12], y[13]),
               pack_bf16x2(y[14], y[15])};
}

// NVFP4: one whole 16-element block per lane. The E2M1 values (RaZeR: code 8
// is the block's +-5) are exact in bf16 and the 16-point transform of them is
// exact (sums of at most 16 multiples of 0.5 below 100, then times 1/4); the
// block scale commutes with a transform inside the block, so s_eff multiplies
// once afterwards: one fp32 rounding, then bf16.
template <bool kHad, bool kRazer>
__device__ __forceinline__ void nv_unrotate_tile(u32x2_t c, uint32_t sbyte, float s_t,
                                                 const bf16x8_t& a0, const bf16x8_t& a1,
                                                 u32x4_t& lo, u32x4_t& hi) {
  const float s_eff = e4m3_decode(kRazer ? (sbyte & 0x7Fu) : (sbyte & 0xFFu)) * s_t;
  const float special = (sbyte & 0x80u) ? -5.0f : 5.0f;
  float v[16];
#define FP4_DEC2(w, k, o)                                                      \
  {                                                                            \
    const float2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, k); \
    v[o] = p.x;                                                                \
    v[o + 1] = p.y;                                                            \
  }
  FP4_DEC2(c.x, 0, 0) FP4_DEC2(c.x, 1, 2) FP4_DEC2(c.x, 2, 4) FP4_DEC2(c.x, 3, 6)
  FP4_DEC2(c.y, 0, 8) FP4_DEC2(c.y, 1, 10) FP4_DEC2(c.y, 2, 12) FP4_DEC2(c.y, 3, 14)
#undef FP4_DEC2
  if (kRazer) {  // code 8 is the only code that decodes to -0.0
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (__float_as_uint(v[k]) == 0x80000000u) v[k] = special;
  }
  if (kHad) {
    lo = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
    hi = u32x4_t{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                 pack_bf16x2(v[14], v[15])};
    hadamard_mfma<16>(a0, a1, lo, hi, v);
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] *= s_eff;
  lo = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
  hi = u32x4_t{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
               pack_bf16x2(v[14], v[15])};
}

// Scatter one tile's 16 bf16 (lo: elements 0..7, hi: 8..15 of the lane's
// half-block) into the row staged at LDS byte kOff of buf; G as for the
// gather of the forward kernel.
template <int G, uint32_t kOff>
__device__ __forceinline__ void scatter_tile(uint8_t* buf, const uint32_t* off, u32x4_t lo,
                                             u32x4_t hi) {
  uint8_t* base = buf + kOff;
  const uint32_t v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  if constexpr (G == 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      *reinterpret_cast<uint16_t*>(base + (off[k] & 0xFFFFu)) = (uint16_t)(v[k] & 0xFFFFu);
      *reinterpret_cast<uint16_t*>(base + (off[k] >> 16)) = (uint16_t)(v[k] >> 16);
    }
  } else if constexpr (G == 2) {
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<uint32_t*>(base + (off[k] & 0xFFFFu)) = v[k];
  } else if constexpr (G == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<u32x2_t*>(base + (off[2 * k] & 0xFFFFu)) = u32x2_t{v[2 * k], v[2 * k + 1]};
  } else {
    *reinterpret_cast<u32x4_t*>(base + (off[0] & 0xFFFFu)) = lo;
    *reinterpret_cast<u32x4_t*>(base + (off[4] & 0xFFFFu)) = hi;
  }
}

template <int kTpw, int kAhead>
struct UnrotCtx {
  const uint8_t* __restrict__ codes;
  const uint8_t* __restrict__ scales;
  uint16_t* __restrict__ out;
  uint8_t* sbuf;        // two LDS row buffers (with a permutation)
  uint32_t (*off)[8];   // the lane's scatter offsets, per tile
  bf16x8_t a0, a1;      // Hadamard MFMA operands
  bf16x8_t m[3][2];     // kFmt 3: the learned block matrix, transposed
  RotGeom g;
  RowCodes<kTpw>* rc;   // kAhead + 1 register buffers: rows k .. k + kAhead
  float s_t;            // NVFP4 tensor scale
};

// Rows r0 + k G (G = grid size), k < K, row k's codes in register buffer
// k % (kAhead + 1). Step k decodes row k, loads the codes of row
// k + kAhead + 1 into the buffer just used, and (with a permutation)
// scatters into LDS buffer k % 2, waits at a barrier and writes the row out.
// The loop runs whole groups of U = lcm(2, kAhead + 1) steps so every buffer
// choice is a compile-time constant; a tail takes the last steps.
// kFmt: the C ABI's format number; NVFP4 (kRazer: RaZeR codes) with the
// 16-point transform, MXFP4 or MXINT4 with the 32-point one.
template <int G, int kTpw, int kAhead, int kFmt, bool kRazer, bool kHad, int kW>
struct UnrotRows {
  static constexpr bool kNv = kFmt == 1;
  using Ctx = UnrotCtx<kTpw, kAhead>;
  static constexpr int kCpl = 2 * kTpw;
  static constexpr uint32_t kBufBytes = 2048u * kW * kTpw;
  static constexpr int kRing = kAhead + 1;
  static constexpr int U = kRing % 2 == 0 ? kRing : 2 * kRing;

  template <int kS>
  static __device__ __forceinline__ void step(const Ctx& c, int32_t r) {
    constexpr int kBuf = kS & 1;
    RowCodes<kTpw>& rc = c.rc[kS % kRing];
    const RotGeom& g = c.g;
    const int32_t G_ = gridDim.x;
    const uint32_t n = threadIdx.x & 31u;
    u32x4_t lo[kTpw], hi[kTpw];
#pragma unroll
    for (int i = 0; i < kTpw; ++i) {
      if constexpr (kNv)
        nv_unrotate_tile<kHad, kRazer>(rc.c[i], rc.s[i], c.s_t, c.a0, c.a1, lo[i], hi[i]);
      else if constexpr (kFmt == 3)
        unrotate_tile_mat(rc.c[i], rc.s[i], c.m, lo[i], hi[i]);
      else
        unrotate_tile<kHad, kFmt == 2>(rc.c[i], rc.s[i], c.a0, c.a1, lo[i], hi[i]);
    }
    load_codes<kTpw, kNv, kW>(unrot_rsrc(c.codes, c.scales, c.out, r + kRing * G_, g), g, rc);
    const UnrotRsrc q = unrot_rsrc(c.codes, c.scales, c.out, r, g);
#pragma unroll
    for (int i = 0; i < kTpw; ++i) {  // lanes without a block (offsets 0) write nothing
      const int32_t b = 32 * ((int32_t)(threadIdx.x >> 6) + kW * i) + (int32_t)n;
      if (b < g.bpr) scatter_tile<G, kBuf * kBufBytes>(c.sbuf, c.off[i], lo[i], hi[i]);
    }
    __syncthreads();
    const int32_t cpr = g.cols / 8;
#pragma unroll
    for (int i = 0; i < kCpl; ++i) {
      const int32_t ch = threadIdx.x + i * 64 * kW;
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(c.sbuf + kBuf * kBufBytes)[ch < cpr ? ch : 0];
      __builtin_amdgcn_raw_buffer_store_b128(v, q.o, ch < cpr ? 16u * ch : kOob, 0, kNt);
    }
  }

  template <int... us>
  static __device__ __forceinline__ void group(const Ctx& c, int32_t k,
                                               std::integer_sequence<int, us...>) {
    const int32_t G_ = gridDim.x, r0 = blockIdx.x;
    (step<us>(c, r0 + (k + us) * G_), ...);
  }

  template <int... us>
  static __device__ __forceinline__ void tail(const Ctx& c, int32_t k, int32_t K,
                                              std::integer_sequence<int, us...>) {
    const int32_t G_ = gridDim.x, r0 = blockIdx.x;
    (void)((k + us < K ? (step<us>(c, r0 + (k + us) * G_), true) : false) && ...);
  }

  static __device__ __forceinline__ void run(const Ctx& c) {
    const int32_t G_ = gridDim.x, r0 = blockIdx.x;
    const int32_t K = (c.g.rows - r0 + G_ - 1) / G_;
    int32_t k = 0;
    for (; k + U - 1 < K; k += U) group(c, k, std::make_integer_sequence<int, U>{});
    tail(c, k, K, std::make_integer_sequence<int, U - 1>{});
  }
};

// Tuning (measured on MI355X at 16384 x 8192): work-groups per CU and rows of
// codes in flight (a row's codes take 3 registers per tile). One work-group
// per CU ran about 2% faster than two and 7% faster than four; the
// look-ahead made little difference.
// Eight waves of one tile (two work-groups per CU for MXINT4, one for
// NVFP4) instead of four waves of two tiles, for rows of 4097..8192 columns
// in the formats with the most arithmetic per element. 16384 x 8192 with a
// permutation: NVFP4 + RaZeR 71.1 -> 63.0 us, MXINT4 72.1 -> 62.7 us; MXFP4
// (61.3 -> 62.2) and the learned matrix (61.8 -> 62.6) keep four waves.
// FP4_UNROT_W8 = 0 or 1 forces one choice for every format.
#ifndef FP4_UNROT_W8
#define FP4_UNROT_W8 (-1)
#endif
template <int kFmt, bool kPerm>
constexpr bool unrot_eight_waves() {
  return FP4_UNROT_W8 >= 0 ? FP4_UNROT_W8 != 0 : kFmt == 1 || kFmt == 2;
}
template <int kTpw, int kW, int kFmt>
constexpr int unrot_wgs_per_cu() {
#ifdef FP4_UNROT_W8_WGS
  if (kW == 8) return FP4_UNROT_W8_WGS;
#endif
  return kW == 8 ? (kFmt == 2 ? 2 : 1) : kTpw == 1 ? 2 : 1;
}
template <int kTpw, int kW, int kFmt>
constexpr int unrot_waves_cap() {
  return kW == 8 ? 2 * unrot_wgs_per_cu<kTpw, kW, kFmt>() : kTpw >= 3 ? 1 : 2;
}
#ifndef FP4_UNROT_AHEAD
#define FP4_UNROT_AHEAD 3
#endif

// kFmt 1 (NVFP4): blocks of 16 (scales 2 b + h, tensor scale *ts), the
// 16-point transform; 0 (MXFP4) and 2 (MXINT4): blocks of 32, the 32-point
// one; 3: MXFP4 with the transpose of the learned 32x32 matrix at ts.
// Wide rows (three or four tiles per wave) run one work-group per CU, one
// wave per SIMD, so they may use the whole register file.
template <int kTpw, int kFmt, bool kRazer, bool kHad, bool kPerm, int kW>
__global__ __launch_bounds__(64 * kW, (unrot_waves_cap<kTpw, kW, kFmt>())) void dequant_unrotate_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ ts, const int32_t* __restrict__ perm, uint16_t* __restrict__ out,
    RotGeom g) {
  // the learned matrix holds 24 more registers: less look-ahead on wide rows
  constexpr int kAhead = kFmt == 3 && kTpw >= 3 ? 1 : FP4_UNROT_AHEAD;
  constexpr bool kNv = kFmt == 1;
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * 2048 * kW * kTpw];
  i32x4_t v[kTpw][4];
  if constexpr (kPerm)
    load_lane_perm<kTpw, kW>(perm, g, v);
  else
    identity_lane_perm<kTpw, kW>(g, v);
  RowCodes<kTpw> rc[kAhead + 1];
#pragma unroll
  for (int j = 0; j <= kAhead; ++j)
    load_codes<kTpw, kNv, kW>(
        unrot_rsrc(codes, scales, out, (int32_t)(blockIdx.x + j * gridDim.x), g), g, rc[j]);
  uint32_t off[kTpw][8];
  const int lr = pack_lane_perm<kTpw, kW>(v, g, off);
  bf16x8_t a0, a1, m[3][2];
  if constexpr (kFmt == 3)
    matrix_operands(ts, true, m);
  else
    hadamard_operands<kNv ? 16 : 32>(a0, a1);
  const float s_t = kNv ? *ts : 1.0f;
  UnrotCtx<kTpw, kAhead> c{codes,
                           scales,
                           out,
                           sbuf,
                           off,
                           a0,
                           a1,
                           {{m[0][0], m[0][1]}, {m[1][0], m[1][1]}, {m[2][0], m[2][1]}},
                           g,
                           rc,
                           s_t};
  // run length agreed by the whole work-group (8 for the identity)
  const int run = !kPerm || __syncthreads_and(lr >= 8) ? 8
                  : __syncthreads_and(lr >= 4) ? 4
                  : __syncthreads_and(lr >= 2) ? 2 : 1;
  if (run == 8)
    UnrotRows<8, kTpw, kAhead, kFmt, kRazer, kHad, kW>::run(c);
  else if (run == 4)
    UnrotRows<4, kTpw, kAhead, kFmt, kRazer, kHad, kW>::run(c);
  else if (run == 2)
    UnrotRows<2, kTpw, kAhead, kFmt, kRazer, kHad, kW>::run(c);
  else
    UnrotRows<1, kTpw, kAhead, kFmt, kRazer, kHad, kW>::run(c);
}

// ================================ launchers =================================
template <int kTpw, int kFmt, bool kRazer, bool kHad, bool kPerm, int kW = kWaves>
static void unrot_launch(const Shape& s, const int32_t* perm, const uint8_t* c, const uint8_t* sc,
                         const float* ts, uint16_t* o, const RotGeom& g, hipStream_t st) {
  // as for the forward kernel: pad LDS so that exactly kWgs work-groups fit per CU
#ifdef FP4_UNROT_WG_PER_CU
  constexpr int kWgs = FP4_UNROT_WG_PER_CU;
#else
  constexpr int kWgs = unrot_wgs_per_cu<kTpw, kW, kFmt>();
#endif
  const DeviceInfo di = device_info();
  const int64_t wgs = (int64_t)di.cus * kWgs;
  const int grid = (int)(s.rows < wgs ? s.rows : wgs);
  constexpr size_t kStatic = 2 * 2048 * kW * kTpw;
  const size_t share = (size_t)di.lds / kWgs;
  const size_t pad = share > kStatic + 1024 ? share - kStatic - 1024 : 0;
  hipLaunchKernelGGL((dequant_unrotate_kernel<kTpw, kFmt, kRazer, kHad, kPerm, kW>), dim3(grid),
                     dim3(64 * kW), pad, st, c, sc, ts, perm, o, g);
}

template <int kFmt, bool kRazer, bool kHad, bool kPerm>
static void unrot_dispatch(const Shape& s, const int32_t* perm, const uint8_t* c,
                           const uint8_t* sc, const float* ts, uint16_t* o, const RotGeom& g,
                           hipStream_t st) {
  const int64_t tpw = (s.cols + 32 * 32 * kWaves - 1) / (32 * 32 * kWaves);
  if (tpw <= 1) unrot_launch<1, kFmt, kRazer, kHad, kPerm>(s, perm, c, sc, ts, o, g, st);
  else if (tpw <= 2 && unrot_eight_waves<kFmt, kPerm>())
    unrot_launch<1, kFmt, kRazer, kHad, kPerm, 8>(s, perm, c, sc, ts, o, g, st);
  else if (tpw <= 2) unrot_launch<2, kFmt, kRazer, kHad, kPerm>(s, perm, c, sc, ts, o, g, st);
  else if (tpw <= 3) unrot_launch<3, kFmt, kRazer, kHad, kPerm>(s, perm, c, sc, ts, o, g, st);
  else unrot_launch<4, kFmt, kRazer, kHad, kPerm>(s, perm, c, sc, ts, o, g, st);
}

template <int kFmt, bool kRazer>
static void unrot_variants(const Shape& s, const int32_t* perm, bool hadamard, const uint8_t* c,
                           const uint8_t* sc, const float* ts, uint16_t* o, const RotGeom& g,
                           hipStream_t st) {
  if (hadamard && perm) unrot_dispatch<kFmt, kRazer, true, true>(s, perm, c, sc, ts, o, g, st);
  if (hadamard && !perm) unrot_dispatch<kFmt, kRazer, true, false>(s, perm, c, sc, ts, o, g, st);
  if (!hadamard && perm) unrot_dispatch<kFmt, kRazer, false, true>(s, perm, c, sc, ts, o, g, st);
}

// MXINT4 instances of the above, compiled in unrotate_int.hip.
void mxint_dequant_unrotate(const Shape& s, const int32_t* perm, bool hadamard,
                            const uint8_t* codes, const uint8_t* scales, uint16_t* out,
                            const RotGeom& g, hipStream_t st);

}  // namespace fp4

#endif  // FP4_UNROTATE_KERNELS_HPP
