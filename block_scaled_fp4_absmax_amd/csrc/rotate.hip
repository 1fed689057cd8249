// rotate.hip -- two-level rotation fused with MXFP4 quantize + pack, the
// inverse rotation for dequantization, and the channel-energy statistic.
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2(a): an inter-block orthogonal transform that evens out the
// block variances (here a channel permutation computed offline); sec. 2(b): a
// rotation inside each 32-block (here the orthonormal Sylvester-Hadamard
// matrix, H[i][j] = (-1)^popcount(i & j) / sqrt(32)).
//
// The block Hadamard is a dense contraction y = H x over 32-element blocks, so
// it runs on the matrix cores: one wave takes 32 blocks as the columns of a
// 32x32 bf16 operand X and computes D = H X with two
// v_mfma_f32_32x32x16_bf16 (K = 16 each) against the constant +-1 matrix H,
// accumulating in fp32; bf16 inputs and +-1 entries make every product exact.
// The MFMA's K order and output-row order are free to choose, so they are
// chosen such that lane (n, h) -- block n = lane % 32, half h = lane / 32 --
// loads the 32 contiguous bytes holding elements 16h..16h+15 of block n and
// receives outputs 16h..16h+15 of the same block: loads and packed stores
// stay contiguous and no lane exchange is needed except one max for the
// block's absmax. The result is scaled by fp32(1/sqrt(32)).
//
// A second implementation of the streaming (no permutation) kernel,
// compile-time FP4_HADAMARD_MFMA=0, runs the transform as a radix-2 butterfly
// in registers and DPP lane exchanges; it is kept for measuring one against
// the other. The inverse rotation uses the butterfly (decode gives fp32 there).
//
// The permutation x'[j] = x[perm[j]] is applied by staging whole rows in LDS.
// A work-group alternates between two LDS row buffers: while its lanes gather
// the permuted elements of one row from one buffer (LDS reads of 2 bytes, or
// 4, 8, 16 when perm moves aligned runs of channels), the next row, fetched
// with coalesced 16-byte loads, is written to the other.
#include "fp4_device.hpp"
#include "launch.hpp"

#ifndef FP4_HADAMARD_MFMA
#define FP4_HADAMARD_MFMA 1
#endif

namespace fp4 {

constexpr bool kUseMfma = FP4_HADAMARD_MFMA != 0;
constexpr float kInvSqrt32 = 0.17677669529663688f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen8(u32x4_t d, float* v) {
  v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
  v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
  v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
  v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
}

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
// operand entries of lane l are H[tau(l % 32)][k0 + j], k0 = 16 (l / 32),
// j = 0..15, with sign parity(row & (k0 + j)) = parity(row & k0) ^
// parity(row & j); bit j of the Walsh mask W(row & 15) is parity(row & j).
__device__ __forceinline__ void hadamard_operands(bf16x8_t& a0, bf16x8_t& a1) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t row = out_index_of_row(lane & 31u);
  uint32_t m = ((row & 1u) ? 0xAAAAu : 0u) ^ ((row & 2u) ? 0xCCCCu : 0u) ^
               ((row & 4u) ? 0xF0F0u : 0u) ^ ((row & 8u) ? 0xFF00u : 0u);
  if ((lane >> 5) & (row >> 4)) m ^= 0xFFFFu;
  u32x4_t v0, v1;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)  // bf16 pair: +-1 = 0x3F80 with the sign bit from the mask
    w[i] = 0x3F803F80u | (((m >> (2 * i)) & 1u) << 15) | (((m >> (2 * i + 1)) & 1u) << 31);
  v0 = u32x4_t{w[0], w[1], w[2], w[3]};
  v1 = u32x4_t{w[4], w[5], w[6], w[7]};
  a0 = __builtin_bit_cast(bf16x8_t, v0);
  a1 = __builtin_bit_cast(bf16x8_t, v1);
}

// y[0..15] = (H x)[16h .. 16h+15] / sqrt(32) for this lane's block, from the
// lane's 16 inputs x[16h .. 16h+15] (bf16 pairs in lo/hi).
__device__ __forceinline__ void hadamard_mfma(const bf16x8_t& a0, const bf16x8_t& a1,
                                              u32x4_t lo, u32x4_t hi, float* y) {
  f32x16_t acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) y[r] = acc[r] * kInvSqrt32;
}

// MXFP4-quantize the lane's 16 outputs; the block spans lanes l and l ^ 32.
template <bool kFloor>
__device__ __forceinline__ void mx_quant16_pair(const float* y, uint32_t& w0, uint32_t& w1,
                                                uint32_t& byte) {
  uint32_t m = absmax_bits<16>(y);
  m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
  byte = e8m0_byte<kFloor>(m);
  if (byte == 0xFFu) {
    w0 = w1 = 0u;
  } else {
    const float s = e8m0_operand(byte);
    w0 = cvt8_f32(y, s);
    w1 = cvt8_f32(y + 8, s);
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

struct RotGeom {
  int32_t rows, cols;
  int32_t bpr;   // 32-element blocks per row
  uint32_t nblk; // rows * bpr
  int64_t ld_x, ld_c, ld_s, ld_rot;
};

// ===================== streaming kernels (no permutation) ===================
// MFMA: a wave owns a tile of 32 consecutive blocks (row-major block order).
// Each work-group makes one pass over kWaves * kTiles consecutive tiles; wave w
// takes tiles base + u * kWaves + w, so at each u the work-group covers one
// contiguous stretch of input, codes and scales.
#ifndef FP4_TILES
#define FP4_TILES 1
#endif
constexpr int kTiles = FP4_TILES;

constexpr int kWaves = kThreads / 64;

template <bool kFlat, bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads) void mx_rotq_stream_mfma_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ rot, RotGeom g) {
  bf16x8_t a0, a1;
  hadamard_operands(a0, a1);
  const uint32_t lane = threadIdx.x & 63u, n = lane & 31u, h = lane >> 5;
  const uint32_t tile0 = blockIdx.x * (kWaves * kTiles) + (threadIdx.x >> 6);
  const uint32_t ntiles = (g.nblk + 31u) >> 5;
  u32x4_t lo[kTiles], hi[kTiles];
  int64_t xo[kTiles], co[kTiles], so[kTiles], ro[kTiles];
  bool ok[kTiles];
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const uint32_t tile = tile0 + u * kWaves;
    const uint32_t b = tile * 32u + n;
    ok[u] = tile < ntiles && b < g.nblk;
    lo[u] = u32x4_t{0u, 0u, 0u, 0u};
    hi[u] = lo[u];
    if (ok[u]) {
      uint32_t r = kFlat ? 0u : b / (uint32_t)g.bpr;
      uint32_t cb = kFlat ? b : b - r * (uint32_t)g.bpr;
      xo[u] = r * g.ld_x + 32 * (int64_t)cb + 16 * h;
      co[u] = r * g.ld_c + 16 * (int64_t)cb + 8 * h;
      so[u] = r * g.ld_s + cb;
      ro[u] = r * g.ld_rot + 32 * (int64_t)cb + 16 * h;
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(x + xo[u]);
      lo[u] = __builtin_nontemporal_load(p);
      hi[u] = __builtin_nontemporal_load(p + 1);
    }
  }
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    if (tile0 + u * kWaves >= ntiles) break;  // uniform across the wave
    float y[16];
    if (kHad) {
      hadamard_mfma(a0, a1, lo[u], hi[u], y);
    } else {
      widen8(lo[u], y);
      widen8(hi[u], y + 8);
    }
    uint32_t w0, w1, byte;
    mx_quant16_pair<kFloor>(y, w0, w1, byte);
    if (ok[u]) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(codes + co[u]);
      __builtin_nontemporal_store(w0, cp);
      __builtin_nontemporal_store(w1, cp + 1);
      if (h == 0) scales[so[u]] = (uint8_t)byte;
      if (kRot) {
        store_rot8(rot + ro[u], y);
        store_rot8(rot + ro[u] + 8, y + 8);
      }
    }
  }
}

// Butterfly: one 16-byte chunk of eight elements per lane, four lanes per
// block; each work-group makes one pass over kThreads * 4 consecutive chunks.
template <bool kFlat, bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads) void mx_rotq_stream_bfly_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ rot, RotGeom g) {
  const uint32_t q = threadIdx.x & 3u;
  const uint32_t n = g.nblk * 4u;
  constexpr int U = 4;
  const uint32_t base = blockIdx.x * (kThreads * U) + threadIdx.x;
  u32x4_t d[U];
  int64_t xo[U], co[U], so[U], ro[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t v = base + u * kThreads;
    if (v < n) {
      uint32_t cpr = 4u * (uint32_t)g.bpr;
      uint32_t r = kFlat ? 0u : v / cpr;
      uint32_t c = kFlat ? v : v - r * cpr;
      xo[u] = r * g.ld_x + 8 * (int64_t)c;
      co[u] = r * g.ld_c + 4 * (int64_t)c;
      so[u] = r * g.ld_s + c / 4;
      ro[u] = r * g.ld_rot + 8 * (int64_t)c;
      d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xo[u]));
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t v = base + u * kThreads;
    if (v >= n) continue;
    float y[8];
    widen8(d[u], y);
    if (kHad) hadamard_butterfly(y, q);
    uint32_t w, byte;
    mx_quant8_quad<kFloor>(y, w, byte);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + co[u]));
    if (q == 0) scales[so[u]] = (uint8_t)byte;
    if (kRot) store_rot8(rot + ro[u], y);
  }
}

// ================== permuting kernel (rows staged in LDS) ===================
// A work-group walks rows r0 + k G (G = grid size) and stages each row in one
// of two LDS buffers of 8192 kTpw bytes (cols <= 4096 kTpw), so a single
// barrier per row suffices: row k + 1 is written to one buffer while row k is
// gathered from the other. Global loads run one row ahead in registers.
//
// Lane (n, h) of wave w handles, for i < kTpw, tile t = w + kWaves i: block
// b = 32 t + n, elements e0 .. e0 + 15 with e0 = 32 b + 16 h, gathered from
// row positions perm[e0 .. e0 + 15]. Those positions are the same for every
// row, so each lane loads them once and keeps them in registers as LDS byte
// offsets (clamped to the row), packed in pairs.
//
// Every global load and store goes through a per-row buffer resource and is
// issued by every lane (rows past the end and idle lanes use out-of-range
// offsets): with a fixed count of memory operations per row, the wait before
// a row is staged covers that row's loads and not the stores issued since.

// Per-row buffer resources (empty for rows past the end).
struct RowRsrc {
  rsrc_t x, c, s, rot;
};

template <bool kRot>
__device__ __forceinline__ RowRsrc row_rsrc(const uint16_t* x, uint8_t* codes, uint8_t* scales,
                                            float* rot, int32_t r, const RotGeom& g) {
  const bool in = r < g.rows;
  const int64_t rr = in ? r : 0;
  RowRsrc q;
  q.x = make_rsrc(x + rr * g.ld_x, in ? 2u * (uint32_t)g.cols : 0u);
  q.c = make_rsrc(codes + rr * g.ld_c, in ? (uint32_t)g.cols / 2u : 0u);
  q.s = make_rsrc(scales + rr * g.ld_s, in ? (uint32_t)g.bpr : 0u);
  if (kRot) q.rot = make_rsrc(rot + rr * g.ld_rot, in ? 4u * (uint32_t)g.cols : 0u);
  return q;
}

template <int kCpl>
__device__ __forceinline__ void load_row(rsrc_t src, int32_t cpr, u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    const int32_t c = threadIdx.x + i * kThreads;
    pre[i] = __builtin_amdgcn_raw_buffer_load_b128(src, c < cpr ? 16u * c : kOob, 0, kNt);
  }
}

template <int kCpl>
__device__ __forceinline__ void put_row(uint8_t* buf, int32_t cpr, const u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    int32_t c = threadIdx.x + i * kThreads;
    if (c < cpr) reinterpret_cast<u32x4_t*>(buf)[c] = pre[i];
  }
}

// Issue the loads of this lane's perm entries (16 per tile, zeros for tiles
// past the row).
template <int kTpw>
__device__ __forceinline__ void load_lane_perm(const int32_t* __restrict__ perm,
                                               const RotGeom& g, i32x4_t (*v)[4]) {
  const rsrc_t rp = make_rsrc(perm, 4u * (uint32_t)g.cols);
  const int32_t lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int32_t b = 32 * (w + kWaves * i) + n;
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
template <int kTpw>
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
    if (32 * (w + kWaves * i) + n < g.bpr) {
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

// The 16 gathered bf16 of one tile (MFMA B halves lo, hi) from the row staged
// at LDS byte kOff of buf; G: the packed offsets form aligned runs of G, read
// 2G bytes at a time.
template <int G, uint32_t kOff>
__device__ __forceinline__ void gather_tile(const uint8_t* buf, const uint32_t* off, u32x4_t& lo,
                                            u32x4_t& hi) {
  const uint8_t* base = buf + kOff;
  if constexpr (G == 1) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = (uint32_t)*reinterpret_cast<const uint16_t*>(base + (off[k] & 0xFFFFu)) |
             ((uint32_t)*reinterpret_cast<const uint16_t*>(base + (off[k] >> 16)) << 16);
    lo = u32x4_t{v[0], v[1], v[2], v[3]};
    hi = u32x4_t{v[4], v[5], v[6], v[7]};
  } else if constexpr (G == 2) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const uint32_t*>(base + (off[k] & 0xFFFFu));
    lo = u32x4_t{v[0], v[1], v[2], v[3]};
    hi = u32x4_t{v[4], v[5], v[6], v[7]};
  } else if constexpr (G == 4) {
    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(base + (off[0] & 0xFFFFu));
    const u32x2_t b = *reinterpret_cast<const u32x2_t*>(base + (off[2] & 0xFFFFu));
    const u32x2_t c = *reinterpret_cast<const u32x2_t*>(base + (off[4] & 0xFFFFu));
    const u32x2_t d = *reinterpret_cast<const u32x2_t*>(base + (off[6] & 0xFFFFu));
    lo = u32x4_t{a.x, a.y, b.x, b.y};
    hi = u32x4_t{c.x, c.y, d.x, d.y};
  } else {
    lo = *reinterpret_cast<const u32x4_t*>(base + (off[0] & 0xFFFFu));
    hi = *reinterpret_cast<const u32x4_t*>(base + (off[4] & 0xFFFFu));
  }
}

// One row step: stage the next row (already loaded into pre) into the other
// buffer, load the row after it into pre, then gather, rotate, quantize and
// store row r from buffer kBuf; a barrier closes the step.
template <int G, int kTpw, int kBuf, bool kHad, bool kFloor, bool kRot>
__device__ __forceinline__ void perm_step(const uint16_t* __restrict__ x, uint8_t* sbuf,
                                          const uint32_t (*off)[8], const bf16x8_t& a0,
                                          const bf16x8_t& a1, uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales, float* __restrict__ rot,
                                          const RotGeom& g, int32_t r, bool has_next,
                                          u32x4_t* pre) {
  constexpr int kCpl = 2 * kTpw;
  constexpr uint32_t kBufBytes = 8192u * kTpw;
  const int32_t cpr = g.cols / 8;
  const int32_t G_ = gridDim.x;
  if (has_next) put_row<kCpl>(sbuf + (1 - kBuf) * kBufBytes, cpr, pre);
  load_row<kCpl>(row_rsrc<kRot>(x, codes, scales, rot, r + 2 * G_, g).x, cpr, pre);
  const RowRsrc q = row_rsrc<kRot>(x, codes, scales, rot, r, g);
  const uint32_t lane = threadIdx.x & 63u, n = lane & 31u, h = lane >> 5;
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int32_t b = 32 * ((int32_t)(threadIdx.x >> 6) + kWaves * i) + (int32_t)n;
    const bool ok = b < g.bpr;
    u32x4_t lo, hi;
    gather_tile<G, kBuf * kBufBytes>(sbuf, off[i], lo, hi);
    float y[16];
    if (kHad) {
      hadamard_mfma(a0, a1, lo, hi, y);
    } else {
      widen8(lo, y);
      widen8(hi, y + 8);
    }
    uint32_t w0, w1, byte;
    mx_quant16_pair<kFloor>(y, w0, w1, byte);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w0, w1}, q.c, ok ? 16u * b + 8u * h : kOob, 0,
                                          kNt);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, q.s, ok && h == 0 ? (uint32_t)b : kOob,
                                         0, 0);
    if (kRot) {
      const uint32_t o = ok ? 4u * (32u * b + 16u * h) : kOob;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, f32x4_t{y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]}),
            q.rot, o == kOob ? kOob : o + 16u * k, 0, kNt);
    }
  }
  __syncthreads();
}

// Rows r0 + k G, k < K. Step 0 is peeled and the loop takes steps in pairs
// (buffer 1, then 0), so every path into a step's wait has the same memory
// operations after the loads it waits for: the previous step's stores.
template <int G, int kTpw, bool kHad, bool kFloor, bool kRot>
__device__ __forceinline__ void perm_rows(const uint16_t* __restrict__ x, uint8_t* sbuf,
                                          const uint32_t (*off)[8], const bf16x8_t& a0,
                                          const bf16x8_t& a1, uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales, float* __restrict__ rot,
                                          const RotGeom& g, u32x4_t* pre) {
  const int32_t G_ = gridDim.x, r0 = blockIdx.x;
  const int32_t K = (g.rows - r0 + G_ - 1) / G_;
  perm_step<G, kTpw, 0, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g, r0,
                                            K > 1, pre);
  int32_t k = 1;
  for (; k + 1 < K; k += 2) {
    perm_step<G, kTpw, 1, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g,
                                              r0 + k * G_, true, pre);
    perm_step<G, kTpw, 0, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g,
                                              r0 + (k + 1) * G_, k + 2 < K, pre);
  }
  if (k < K)
    perm_step<G, kTpw, 1, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g,
                                              r0 + k * G_, false, pre);
}

// Waves per SIMD the register allocation is held to, and work-groups per CU
// in the grid. Two row buffers of 8 KB kTpw each bound the work-groups a CU
// can hold; on MI355X at cols = 8192 two per CU (32 rows each) measured
// faster than three or four, and one per CU slower.
template <int kTpw>
constexpr int perm_waves_cap() {
  return kTpw <= 2 ? 4 : 2;
}
template <int kTpw>
constexpr int perm_wgs_per_cu() {
  return kTpw == 1 ? 4 : 2;
}

#ifndef FP4_PERM_WAVES
#define FP4_PERM_WAVES perm_waves_cap<kTpw>()
#endif
template <int kTpw, bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads, FP4_PERM_WAVES) void mx_rotq_perm_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ rot, RotGeom g) {
  constexpr int kCpl = 2 * kTpw;
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * 8192 * kTpw];
  const int32_t cpr = g.cols / 8;
  // perm entries first, then row r0, so the row load is in flight while the
  // entries are unpacked
  i32x4_t v[kTpw][4];
  load_lane_perm<kTpw>(perm, g, v);
  u32x4_t pre[kCpl];
  load_row<kCpl>(row_rsrc<kRot>(x, codes, scales, rot, blockIdx.x, g).x, cpr, pre);
  uint32_t off[kTpw][8];
  const int lr = pack_lane_perm<kTpw>(v, g, off);
  bf16x8_t a0, a1;
  hadamard_operands(a0, a1);
  put_row<kCpl>(sbuf, cpr, pre);
  load_row<kCpl>(row_rsrc<kRot>(x, codes, scales, rot, blockIdx.x + gridDim.x, g).x, cpr, pre);
  // run length agreed by the whole work-group (this also publishes row r0)
  const int run = __syncthreads_and(lr >= 8) ? 8
                  : __syncthreads_and(lr >= 4) ? 4
                  : __syncthreads_and(lr >= 2) ? 2 : 1;
  if (run == 8)
    perm_rows<8, kTpw, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g, pre);
  else if (run == 4)
    perm_rows<4, kTpw, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g, pre);
  else if (run == 2)
    perm_rows<2, kTpw, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g, pre);
  else
    perm_rows<1, kTpw, kHad, kFloor, kRot>(x, sbuf, off, a0, a1, codes, scales, rot, g, pre);
}

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
static RotGeom rot_geom(const Shape& s, int64_t ld_rot) {
  RotGeom g;
  g.rows = (int32_t)s.rows;
  g.cols = (int32_t)s.cols;
  g.bpr = (int32_t)(s.cols / 32);
  g.nblk = (uint32_t)(s.rows * (s.cols / 32));
  g.ld_x = s.ld_x;
  g.ld_c = s.ld_c;
  g.ld_s = s.ld_s;
  g.ld_rot = ld_rot;
  return g;
}

static int perm_grid(int64_t rows) { return (int)(rows < kPermGrid ? rows : kPermGrid); }

// Compute units of the current device.
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

template <int kTpw, bool kHad, bool kFloor, bool kRot>
static void perm_launch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                        uint8_t* sc, float* rot, const RotGeom& g, hipStream_t st) {
#ifdef FP4_PERM_WG_PER_CU
  const int64_t wgs = (int64_t)cu_count() * FP4_PERM_WG_PER_CU;
#else
  const int64_t wgs = (int64_t)cu_count() * perm_wgs_per_cu<kTpw>();
#endif
  const int grid = (int)(s.rows < wgs ? s.rows : wgs);
  hipLaunchKernelGGL((mx_rotq_perm_kernel<kTpw, kHad, kFloor, kRot>), dim3(grid), dim3(kThreads),
                     0, st, x, perm, c, sc, rot, g);
}

template <bool kHad, bool kFloor, bool kRot>
static void rotq_dispatch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                          uint8_t* sc, float* rot, const RotGeom& g, bool flat, hipStream_t st) {
  if (perm) {
    // MFMA tiles (32 blocks) per wave per row
    const int64_t tpw = (s.cols + 32 * 32 * kWaves - 1) / (32 * 32 * kWaves);
    if (tpw <= 1) perm_launch<1, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else if (tpw <= 2) perm_launch<2, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else if (tpw <= 3) perm_launch<3, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else perm_launch<4, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    return;
  }
  if constexpr (kUseMfma) {
    const uint64_t tiles = ((uint64_t)g.nblk + 31) / 32;
    const uint64_t grid = (tiles + kWaves * kTiles - 1) / (kWaves * kTiles);
    if (flat)
      hipLaunchKernelGGL((mx_rotq_stream_mfma_kernel<true, kHad, kFloor, kRot>), dim3((int)grid),
                         dim3(kThreads), 0, st, x, c, sc, rot, g);
    else
      hipLaunchKernelGGL((mx_rotq_stream_mfma_kernel<false, kHad, kFloor, kRot>), dim3((int)grid),
                         dim3(kThreads), 0, st, x, c, sc, rot, g);
  } else {
    const uint64_t chunks = (uint64_t)g.nblk * 4;
    const uint64_t grid = (chunks + kThreads * 4 - 1) / (kThreads * 4);
    if (flat)
      hipLaunchKernelGGL((mx_rotq_stream_bfly_kernel<true, kHad, kFloor, kRot>), dim3((int)grid),
                         dim3(kThreads), 0, st, x, c, sc, rot, g);
    else
      hipLaunchKernelGGL((mx_rotq_stream_bfly_kernel<false, kHad, kFloor, kRot>), dim3((int)grid),
                         dim3(kThreads), 0, st, x, c, sc, rot, g);
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
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / 32 &&
                    (!r || ld_rot == s.cols);
  if (had && !floor_rule && !r) rotq_dispatch<true, false, false>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && !floor_rule && r) rotq_dispatch<true, false, true>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && floor_rule && !r) rotq_dispatch<true, true, false>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && floor_rule && r) rotq_dispatch<true, true, true>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && !floor_rule && !r) rotq_dispatch<false, false, false>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && !floor_rule && r) rotq_dispatch<false, false, true>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && floor_rule && !r) rotq_dispatch<false, true, false>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && floor_rule && r) rotq_dispatch<false, true, true>(s, perm, xp, cp, sp, rot, g, flat, st);
}

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
