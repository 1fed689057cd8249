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
// A second implementation (compile-time, FP4_HADAMARD_MFMA=0) runs the
// transform as a radix-2 butterfly in registers and DPP lane exchanges; it is
// kept for measuring one against the other.
//
// The permutation x'[j] = x[perm[j]] is applied by staging whole rows in LDS:
// a work-group loads a row with coalesced 16-byte loads, then each lane
// gathers its permuted elements with 2-byte LDS reads. The next row's global
// loads are issued before the current row is processed.
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
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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

// ================== permuting kernels (one row at a time, LDS) ==============
// Dynamic LDS: row[cols] bf16 followed by perm[cols] uint16 (entries clamped
// to cols - 1, so no gather leaves the row). A work-group walks rows
// r0, r0 + G, r0 + 2G, ... (G = grid size). The global loads of the row kDepth
// steps ahead are issued into registers before the current row is processed,
// so kDepth rows per work-group are in flight; kCpl = 16-byte chunks per lane
// per row (cols <= 8 * kThreads * kCpl).
constexpr int kMaxChunksPerLane = (int)(kMaxPermCols / 8 / kThreads);  // 8

// Stage perm into LDS as uint16 (clamped to the row) and return the largest
// run length G in {8, 4, 2, 1} such that perm maps every aligned run of G
// positions onto an aligned run of G consecutive channels (same for the whole
// work-group, so the caller's branch on it is uniform).
__device__ __forceinline__ int stage_perm(const int32_t* __restrict__ perm, uint16_t* sperm,
                                          int32_t cols) {
  const int32_t cmax = cols - 1;
  for (int32_t j = threadIdx.x; j < cols; j += kThreads) {
    int32_t p = perm[j];
    p = p < 0 ? 0 : (p > cmax ? cmax : p);
    sperm[j] = (uint16_t)p;
  }
  __syncthreads();
  int ok2 = 1, ok4 = 1, ok8 = 1;
  for (int32_t j = threadIdx.x; j < cols; j += kThreads) {
    const uint32_t p = sperm[j];
    const uint32_t b2 = sperm[j & ~1], b4 = sperm[j & ~3], b8 = sperm[j & ~7];
    ok2 &= (p == b2 + (uint32_t)(j & 1)) && (b2 % 2u == 0u);
    ok4 &= (p == b4 + (uint32_t)(j & 3)) && (b4 % 4u == 0u);
    ok8 &= (p == b8 + (uint32_t)(j & 7)) && (b8 % 8u == 0u);
  }
  if (__syncthreads_and(ok8)) return 8;
  if (__syncthreads_and(ok4)) return 4;
  if (__syncthreads_and(ok2)) return 2;
  return 1;
}

template <int kCpl>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ src, int32_t cpr,
                                         u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    int32_t c = threadIdx.x + i * kThreads;
    if (c < cpr) pre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src) + c);
  }
}

template <int kCpl>
__device__ __forceinline__ void put_row(uint16_t* srow, int32_t cpr, const u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    int32_t c = threadIdx.x + i * kThreads;
    if (c < cpr) reinterpret_cast<u32x4_t*>(srow)[c] = pre[i];
  }
}

// Eight gathered bf16, packed in pairs, from eight LDS indices.
__device__ __forceinline__ u32x4_t gather8(const uint16_t* srow, u32x4_t id) {
  u32x4_t r;
  r.x = (uint32_t)srow[id.x & 0xFFFFu] | ((uint32_t)srow[id.x >> 16] << 16);
  r.y = (uint32_t)srow[id.y & 0xFFFFu] | ((uint32_t)srow[id.y >> 16] << 16);
  r.z = (uint32_t)srow[id.z & 0xFFFFu] | ((uint32_t)srow[id.z >> 16] << 16);
  r.w = (uint32_t)srow[id.w & 0xFFFFu] | ((uint32_t)srow[id.w >> 16] << 16);
  return r;
}

// The 16 gathered bf16 x'[e0 .. e0+15] (e0 a multiple of 16), as the MFMA's two
// B halves, when perm is made of aligned runs of G channels: one LDS read of
// 2G bytes per run.
template <int G>
__device__ __forceinline__ void gather16(const uint16_t* srow, const uint16_t* sperm, int32_t e0,
                                         u32x4_t& lo, u32x4_t& hi) {
  if constexpr (G == 1) {
    const u32x4_t* ip = reinterpret_cast<const u32x4_t*>(sperm + e0);
    lo = gather8(srow, ip[0]);
    hi = gather8(srow, ip[1]);
  } else if constexpr (G == 2) {
    const u32x4_t* ip = reinterpret_cast<const u32x4_t*>(sperm + e0);
    const u32x4_t i0 = ip[0], i1 = ip[1];
    const uint32_t* w = reinterpret_cast<const uint32_t*>(srow);
    lo.x = w[(i0.x & 0xFFFFu) >> 1]; lo.y = w[(i0.y & 0xFFFFu) >> 1];
    lo.z = w[(i0.z & 0xFFFFu) >> 1]; lo.w = w[(i0.w & 0xFFFFu) >> 1];
    hi.x = w[(i1.x & 0xFFFFu) >> 1]; hi.y = w[(i1.y & 0xFFFFu) >> 1];
    hi.z = w[(i1.z & 0xFFFFu) >> 1]; hi.w = w[(i1.w & 0xFFFFu) >> 1];
  } else if constexpr (G == 4) {
    const u32x2_t* w = reinterpret_cast<const u32x2_t*>(srow);
    const u32x2_t a = w[sperm[e0] >> 2], b = w[sperm[e0 + 4] >> 2];
    const u32x2_t c = w[sperm[e0 + 8] >> 2], d = w[sperm[e0 + 12] >> 2];
    lo = u32x4_t{a.x, a.y, b.x, b.y};
    hi = u32x4_t{c.x, c.y, d.x, d.y};
  } else {
    const u32x4_t* w = reinterpret_cast<const u32x4_t*>(srow);
    lo = w[sperm[e0] >> 3];
    hi = w[sperm[e0 + 8] >> 3];
  }
}

// Permute + Hadamard + quantize one staged row (MFMA: a wave takes tiles of 32
// blocks, lane (n, h) gathers elements 16h..16h+15 of block n).
template <int G, bool kHad, bool kFloor, bool kRot>
__device__ __forceinline__ void rotq_row_mfma(const uint16_t* srow, const uint16_t* sperm,
                                              const bf16x8_t& a0, const bf16x8_t& a1, int32_t r,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales,
                                              float* __restrict__ rot, const RotGeom& g) {
  const uint32_t lane = threadIdx.x & 63u, n = lane & 31u, h = lane >> 5;
  const int32_t ntiles = (g.bpr + 31) / 32;
  for (int32_t t = threadIdx.x >> 6; t < ntiles; t += kWaves) {
    const int32_t b = 32 * t + (int32_t)n;
    const bool ok = b < g.bpr;
    u32x4_t lo = {0u, 0u, 0u, 0u}, hi = lo;
    if (ok) gather16<G>(srow, sperm, 32 * b + 16 * (int32_t)h, lo, hi);
    float y[16];
    if (kHad) {
      hadamard_mfma(a0, a1, lo, hi, y);
    } else {
      widen8(lo, y);
      widen8(hi, y + 8);
    }
    uint32_t w0, w1, byte;
    mx_quant16_pair<kFloor>(y, w0, w1, byte);
    if (ok) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(codes + r * g.ld_c + 16 * (int64_t)b + 8 * h);
      __builtin_nontemporal_store(w0, cp);
      __builtin_nontemporal_store(w1, cp + 1);
      if (h == 0) scales[r * g.ld_s + b] = (uint8_t)byte;
      if (kRot) {
        float* rp = rot + r * g.ld_rot + 32 * (int64_t)b + 16 * h;
        store_rot8(rp, y);
        store_rot8(rp + 8, y + 8);
      }
    }
  }
}

// Same row, butterfly implementation: lane takes 16-byte chunks c = t + i * kThreads.
template <bool kHad, bool kFloor, bool kRot>
__device__ __forceinline__ void rotq_row_bfly(const uint16_t* srow, const uint16_t* sperm,
                                              int32_t r, uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales,
                                              float* __restrict__ rot, const RotGeom& g) {
  const uint32_t q = threadIdx.x & 3u;
  const int32_t cpr = g.cols / 8;
  for (int32_t c = threadIdx.x; c < cpr; c += kThreads) {
    float y[8];
    widen8(gather8(srow, reinterpret_cast<const u32x4_t*>(sperm)[c]), y);
    if (kHad) hadamard_butterfly(y, q);
    uint32_t w, byte;
    mx_quant8_quad<kFloor>(y, w, byte);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + r * g.ld_c + 4 * (int64_t)c));
    if (q == 0) scales[r * g.ld_s + c / 4] = (uint8_t)byte;
    if (kRot) store_rot8(rot + r * g.ld_rot + 8 * (int64_t)c, y);
  }
}

template <int G, int kCpl, int kDepth, bool kHad, bool kFloor, bool kRot>
__device__ __forceinline__ void perm_rows(const uint16_t* __restrict__ x, uint16_t* srow,
                                          const uint16_t* sperm, const bf16x8_t& a0,
                                          const bf16x8_t& a1, uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales, float* __restrict__ rot,
                                          const RotGeom& g) {
  const int32_t cpr = g.cols / 8;
  const int32_t G_ = gridDim.x;
  u32x4_t pre[kDepth][kCpl];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int32_t rr = (int32_t)blockIdx.x + d * G_;
    if (rr < g.rows) load_row<kCpl>(x + rr * g.ld_x, cpr, pre[d]);
  }
  for (int32_t r = blockIdx.x; r < g.rows; r += kDepth * G_) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int32_t rr = r + d * G_;
      if (rr >= g.rows) break;  // uniform across the work-group
      __syncthreads();          // the previous row's gathers are done
      put_row<kCpl>(srow, cpr, pre[d]);
      __syncthreads();
      const int32_t rn = rr + kDepth * G_;
      if (rn < g.rows) load_row<kCpl>(x + rn * g.ld_x, cpr, pre[d]);
      if constexpr (kUseMfma)
        rotq_row_mfma<G, kHad, kFloor, kRot>(srow, sperm, a0, a1, rr, codes, scales, rot, g);
      else
        rotq_row_bfly<kHad, kFloor, kRot>(srow, sperm, rr, codes, scales, rot, g);
    }
  }
}

template <int kCpl, int kDepth, bool kHad, bool kFloor, bool kRot>
__global__ __launch_bounds__(kThreads) void mx_rotq_perm_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ rot, RotGeom g) {
  extern __shared__ uint16_t smem[];
  uint16_t* srow = smem;
  uint16_t* sperm = smem + g.cols;
  bf16x8_t a0, a1;
  if constexpr (kUseMfma) hadamard_operands(a0, a1);
  const int run = stage_perm(perm, sperm, g.cols);
  if constexpr (kUseMfma) {
    if (run == 8)
      perm_rows<8, kCpl, kDepth, kHad, kFloor, kRot>(x, srow, sperm, a0, a1, codes, scales, rot, g);
    else if (run == 4)
      perm_rows<4, kCpl, kDepth, kHad, kFloor, kRot>(x, srow, sperm, a0, a1, codes, scales, rot, g);
    else if (run == 2)
      perm_rows<2, kCpl, kDepth, kHad, kFloor, kRot>(x, srow, sperm, a0, a1, codes, scales, rot, g);
    else
      perm_rows<1, kCpl, kDepth, kHad, kFloor, kRot>(x, srow, sperm, a0, a1, codes, scales, rot, g);
  } else {
    perm_rows<1, kCpl, kDepth, kHad, kFloor, kRot>(x, srow, sperm, a0, a1, codes, scales, rot, g);
  }
}

// ============================ inverse rotation ==============================
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
  if (kPerm) (void)stage_perm(perm, sperm, g.cols);
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

template <int kCpl, int kDepth, bool kHad, bool kFloor, bool kRot>
static void perm_launch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                        uint8_t* sc, float* rot, const RotGeom& g, hipStream_t st) {
  const int grid = perm_grid(s.rows);
  const size_t lds = (size_t)4 * s.cols;
  hipLaunchKernelGGL((mx_rotq_perm_kernel<kCpl, kDepth, kHad, kFloor, kRot>), dim3(grid),
                     dim3(kThreads), lds, st, x, perm, c, sc, rot, g);
}

template <bool kHad, bool kFloor, bool kRot>
static void rotq_dispatch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                          uint8_t* sc, float* rot, const RotGeom& g, bool flat, hipStream_t st) {
  if (perm) {
    const int64_t cpl = (s.cols / 8 + kThreads - 1) / kThreads;
    // chunks per lane and prefetch depth: about 32 VGPRs of rows in flight
    if (cpl <= 1) perm_launch<1, 4, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else if (cpl <= 2) perm_launch<2, 4, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else if (cpl <= 4) perm_launch<4, 2, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
    else perm_launch<kMaxChunksPerLane, 1, kHad, kFloor, kRot>(s, perm, x, c, sc, rot, g, st);
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
