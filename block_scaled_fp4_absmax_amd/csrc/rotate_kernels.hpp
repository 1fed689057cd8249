// rotate_kernels.hpp -- two-level rotation fused with FP4 quantize + pack
// (MXFP4, MXINT4 and NVFP4): the kernels and their launch templates, compiled
// per format in rotate_mx.hip, rotate_int.hip and rotate_nv.hip.
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
// the other. (The inverse rotation runs on the MFMA as well.)
//
// The permutation x'[j] = x[perm[j]] is applied by staging whole rows in LDS.
// A work-group alternates between two LDS row buffers: while its lanes gather
// the permuted elements of one row from one buffer (LDS reads of 2 bytes, or
// 4, 8, 16 when perm moves aligned runs of channels), the next row, fetched
// with coalesced 16-byte loads, is written to the other.
#ifndef FP4_ROTATE_KERNELS_HPP
#define FP4_ROTATE_KERNELS_HPP

#include <utility>

#include "launch.hpp"
#include "rotation.hpp"

#ifndef FP4_HADAMARD_MFMA
#define FP4_HADAMARD_MFMA 1
#endif


namespace fp4 {

constexpr bool kUseMfma = FP4_HADAMARD_MFMA != 0;

// ===================== streaming kernels (no permutation) ===================
// MFMA: a wave owns tiles of 16 consecutive blocks (row-major block order, one
// kilobyte of input: each 16-byte load of the wave covers it whole), in the
// layout of hadamard32_spread. Each work-group makes one pass over
// kWaves * kSpreadTiles consecutive tiles; wave w takes tiles
// base + u * kWaves + w, so at each u the work-group covers one contiguous
// stretch of input, codes and scales. (Tiles of 32 blocks, each lane loading
// 32 contiguous bytes for 32x32x16 MFMAs, left every load instruction half of
// each 128-byte line: 57.1 against 54.x us at 16384 x 8192.)
#ifndef FP4_TILES
#define FP4_TILES 1
#endif
constexpr int kTiles = FP4_TILES;

constexpr int kSpreadTiles = 2;

// kInt: MXINT4 elements instead of E2M1.
template <bool kFlat, bool kHad, bool kFloor, bool kRot, bool kInt>
__global__ __launch_bounds__(kThreads) void mx_rotq_stream_mfma_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ rot, RotGeom g) {
  bf16x8_t a0, a1;
  hadamard32_spread_operands(a0, a1);
  const uint32_t lane = threadIdx.x & 63u, n = lane & 15u, q = lane >> 4;
  const uint32_t tile0 = blockIdx.x * (kWaves * kSpreadTiles) + (threadIdx.x >> 6);
  const uint32_t ntiles = (g.nblk + 15u) >> 4;
  u32x4_t d[kSpreadTiles];
  int64_t co[kSpreadTiles], so[kSpreadTiles], ro[kSpreadTiles];
  bool ok[kSpreadTiles];
#pragma unroll
  for (int u = 0; u < kSpreadTiles; ++u) {
    const uint32_t tile = tile0 + u * kWaves;
    const uint32_t b = tile * 16u + n;
    ok[u] = tile < ntiles && b < g.nblk;
    d[u] = u32x4_t{0u, 0u, 0u, 0u};
    if (ok[u]) {
      const uint32_t r = kFlat ? 0u : b / (uint32_t)g.bpr;
      const uint32_t cb = kFlat ? b : b - r * (uint32_t)g.bpr;
      co[u] = r * g.ld_c + 16 * (int64_t)cb + 4 * q;
      so[u] = scale_row_off(r, g.ld_s, g.s_gemm) + scale_col_off(cb, g.s_gemm);
      ro[u] = r * g.ld_rot + 32 * (int64_t)cb + 8 * q;
      d[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(x + r * g.ld_x + 32 * (int64_t)cb + 8 * q));
    }
  }
#pragma unroll
  for (int u = 0; u < kSpreadTiles; ++u) {
    if (tile0 + u * kWaves >= ntiles) break;  // uniform across the wave
    float y[8];
    if (kHad)
      hadamard32_spread(a0, a1, d[u], y);
    else
      widen8(d[u], y);
    uint32_t w, byte;
    if constexpr (kInt)
      mxint_quant8_spread<kFloor, kHad>(y, w, byte);
    else
      mx_quant8_spread<kFloor, kHad>(y, w, byte);
    if (ok[u]) {
      __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(codes + co[u]));
      if (q == 0) scales[so[u]] = (uint8_t)byte;
      if (kRot) store_rot8(rot + ro[u], y);
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
      so[u] = scale_row_off(r, g.ld_s, g.s_gemm) + scale_col_off(c / 4, g.s_gemm);
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
// A work-group of kW waves walks rows r0 + k G (G = grid size) and stages
// each row in one of two LDS buffers of 2048 kW kTpw bytes (cols <= 1024 kW
// kTpw), so a single
// barrier per row suffices: row k + 1 is written to one buffer while row k is
// gathered from the other. Global loads run one row ahead in registers.
//
// Lane (n, h) of wave w handles, for i < kTpw, tile t = w + kW i (kW waves): block
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
  q.s = make_rsrc(scales + scale_row_off(rr, g.ld_s, g.s_gemm), in ? (uint32_t)g.s_ext : 0u);
  if (kRot) q.rot = make_rsrc(rot + rr * g.ld_rot, in ? 4u * (uint32_t)g.cols : 0u);
  return q;
}

template <int kCpl, int kW = kWaves>
__device__ __forceinline__ void load_row(rsrc_t src, int32_t cpr, u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    const int32_t c = threadIdx.x + i * 64 * kW;
    pre[i] = __builtin_amdgcn_raw_buffer_load_b128(src, c < cpr ? 16u * c : kOob, 0, kNt);
  }
}

template <int kCpl, int kW = kWaves>
__device__ __forceinline__ void put_row(uint8_t* buf, int32_t cpr, const u32x4_t* pre) {
#pragma unroll
  for (int i = 0; i < kCpl; ++i) {
    int32_t c = threadIdx.x + i * 64 * kW;
    if (c < cpr) reinterpret_cast<u32x4_t*>(buf)[c] = pre[i];
  }
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

// State shared by the row steps of one work-group.
template <int kTpw, int kAhead>
struct PermCtx {
  const uint16_t* __restrict__ x;
  uint8_t* sbuf;                       // two LDS row buffers
  uint32_t (*off)[8];                  // the lane's gather offsets, per tile
  bf16x8_t a0, a1;                     // Hadamard MFMA operands
  bf16x8_t m[3][2];                    // kFmtMxMat: the learned block matrix
  uint8_t* __restrict__ codes;
  uint8_t* __restrict__ scales;
  float* __restrict__ rot;
  RotGeom g;
  u32x4_t (*pre)[2 * kTpw];            // kAhead register buffers of rows in flight
  NvScale ns;                          // NVFP4: tensor-scale arithmetic
  const float* rcp_tab;                // NVFP4: block reciprocals by E4M3 code
  float* amax;                         // NVFP4 pre-pass: the lane's running maximum
};

// Gather, transform, quantize and store row r, staged in LDS at buf + kOff
// (G: the gather run length). Per tile the lane issues one 8-byte code store
// and one scale-byte store (plus four 16-byte stores of the rotated values
// with kRot), whether or not it holds a block: the count of memory
// operations per row is fixed.
template <int G, uint32_t kOff, int kTpw, int kFmt, bool kHad, bool kOpt, bool kRot, class Ctx,
          int kW = kWaves>
__device__ __forceinline__ void perm_row(const Ctx& c, const uint8_t* buf, int32_t r) {
    // Code stores are nontemporal. Write-back stores looked faster for the MX
    // formats only while the same two code buffers were rewritten in turn
    // (134 MB, which the 256 MB Infinity Cache keeps, so the rewrites never
    // reached HBM); with the codes of successive calls spread over 536 MB they
    // ran 62.5 us against 58.0 (MXFP4, 16384 x 8192).
    constexpr int kCodeAux = kNt;
    const RotGeom& g = c.g;
    const RowRsrc q = row_rsrc<kRot>(c.x, c.codes, c.scales, c.rot, r, g);
    const uint32_t lane = threadIdx.x & 63u, n = lane & 31u, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < kTpw; ++i) {
      const int32_t b = 32 * ((int32_t)(threadIdx.x >> 6) + kW * i) + (int32_t)n;
      const bool ok = b < g.bpr;
      u32x4_t lo, hi;
      gather_tile<G, kOff>(buf, c.off[i], lo, hi);
      float y[16];
      if (kHad) {
        if constexpr (kFmt == kFmtMxMat)
          matrix_mfma(c.m, lo, hi, y);
        else
          hadamard_mfma<kFmt == kFmtMx || kFmt == kFmtMxInt ? 32 : 16>(c.a0, c.a1, lo, hi, y);
      } else {
        widen8(lo, y);
        widen8(hi, y + 8);
      }
      if constexpr (kFmt == kFmtNvAmax) {
        if (ok) *c.amax = __builtin_fmaxf(*c.amax, absmax16f(y));
      } else {
        uint32_t w0, w1, byte, so;
        if constexpr (kFmt == kFmtMx || kFmt == kFmtMxInt || kFmt == kFmtMxMat) {
          // kOpt: OCP floor rule
          if constexpr (kFmt != kFmtMxInt)
            mx_quant16_pair<kOpt, kHad>(y, w0, w1, byte);
          else
            mxint_quant16_pair<kOpt, kHad>(y, w0, w1, byte);
          so = ok && h == 0 ? scale_col_off((uint32_t)b, g.s_gemm) : kOob;
        } else {  // kOpt: RaZeR; lane h holds block 2 b + h
          nv_quant16<kOpt>(y, c.ns, c.rcp_tab, w0, w1, byte);
          so = ok ? 2u * b + h : kOob;
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w0, w1}, q.c,
                                              ok ? 16u * b + 8u * h : kOob, 0, kCodeAux);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, q.s, so, 0, 0);
        if (kRot) {
          const uint32_t o = ok ? 4u * (32u * b + 16u * h) : kOob;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t,
                                   f32x4_t{y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]}),
                q.rot, o == kOob ? kOob : o + 16u * k, 0, kNt);
        }
      }
    }
}

// Rows r0 + k G (G = grid size), k < K. Row k is gathered from LDS buffer
// k % 2; during its step, rows k + 1 .. k + kAhead are in flight in register
// buffers (row j in buffer j % kAhead). A step stages row k + 1 into the other
// LDS buffer, loads row k + 1 + kAhead into the register buffer just freed,
// then gathers, rotates, quantizes and stores row k; a barrier closes it.
// Step 0 is peeled and the loop runs whole groups of U = lcm(2, kAhead) steps,
// so both buffer choices are compile-time constants and every path into a
// step's wait has at least the steady state's memory operations after the
// loads it waits for; a tail takes the last steps.
template <int G, int kTpw, int kAhead, int kFmt, bool kHad, bool kOpt, bool kRot, int kW>
struct PermRows {
  using Ctx = PermCtx<kTpw, kAhead>;
  static constexpr int kCpl = 2 * kTpw;
  static constexpr uint32_t kBufBytes = 2048u * kW * kTpw;
  static constexpr int U = kAhead % 2 == 0 ? kAhead : 2 * kAhead;

  // kS = k mod U for the step of row k
  template <int kS>
  static __device__ __forceinline__ void step(const Ctx& c, int32_t r, bool has_next) {
    constexpr int kBuf = kS & 1;
    u32x4_t* pre = c.pre[(kS + 1) % kAhead];
    const RotGeom& g = c.g;
    const int32_t cpr = g.cols / 8;
    if (has_next) put_row<kCpl, kW>(c.sbuf + (1 - kBuf) * kBufBytes, cpr, pre);
    const int32_t ra = r + (1 + kAhead) * (int32_t)gridDim.x;
    load_row<kCpl, kW>(row_rsrc<kRot>(c.x, c.codes, c.scales, c.rot, ra, g).x, cpr, pre);
    perm_row<G, kBuf * kBufBytes, kTpw, kFmt, kHad, kOpt, kRot, Ctx, kW>(c, c.sbuf, r);
    __syncthreads();
  }

  // Steps k .. k + U - 1 (k = 1 mod U), all present.
  template <int... us>
  static __device__ __forceinline__ void group(const Ctx& c, int32_t k, int32_t K,
                                               std::integer_sequence<int, us...>) {
    (step<(1 + us) % U>(c, row_of(k + us), k + us + 1 < K), ...);
  }

  // Steps k .. K - 1, fewer than U.
  template <int... us>
  static __device__ __forceinline__ void tail(const Ctx& c, int32_t k, int32_t K,
                                              std::integer_sequence<int, us...>) {
    (void)((k + us < K ? (step<(1 + us) % U>(c, row_of(k + us), k + us + 1 < K), true)
                       : false) &&
           ...);
  }

  // row of step k of this work-group
  static __device__ __forceinline__ int32_t row_of(int32_t k) {
    return (int32_t)blockIdx.x + k * (int32_t)gridDim.x;
  }

  static __device__ __forceinline__ void run(const Ctx& c) {
    const int32_t G_ = gridDim.x, r0 = blockIdx.x;
    const int32_t K = (c.g.rows - r0 + G_ - 1) / G_;
    step<0>(c, row_of(0), K > 1);
    int32_t k = 1;
    for (; k + U - 1 < K; k += U) group(c, k, K, std::make_integer_sequence<int, U>{});
    tail(c, k, K, std::make_integer_sequence<int, U - 1>{});
  }
};

// Tuning per row length (kTpw tiles per wave per row, kW waves per
// work-group; measured on MI355X): work-groups per CU in the grid, rows of
// look-ahead held in registers, and the waves per SIMD the register
// allocation is held to. Two row buffers of 2 KB kW kTpw each bound the
// work-groups a CU can hold. Rows of 4097..8192 columns run eight waves of
// one tile each, two work-groups per CU (16 waves per CU): against four waves
// of two tiles, each wave's share of a row step halves and twice as many
// waves hide the gathers' LDS latency (16384 x 8192: MXFP4 59.5 -> 58.0 us,
// NVFP4 + RaZeR 65.2 -> 62.9 us). Three such work-groups per CU (with one row
// of look-ahead, to fit the registers) ran 4% slower; with four waves, three
// or four work-groups per CU ran slower than two, and one slower still. A
// second row of look-ahead gained about 1%, more none. Launching more
// work-groups than fit at once (each taking fewer rows, placed as slots free
// up) ran 8-14% slower: every work-group repeats the prologue and the ramp of
// its row pipeline.
template <int kTpw, int kW>
constexpr int perm_wgs_per_cu() {
  return kW == 8 ? 2 : kTpw == 1 ? 4 : kTpw <= 4 ? 2 : 1;
}
template <int kTpw>
constexpr int perm_ahead() {
  return kTpw <= 2 ? 2 : 1;
}
template <int kTpw, int kW>
constexpr int perm_waves_cap() {
  return (perm_wgs_per_cu<kTpw, kW>() * kW + 3) / 4;
}

#ifndef FP4_PERM_WAVES
#define FP4_PERM_WAVES (perm_waves_cap<kTpw, kW>())
#endif
#ifndef FP4_PERM_AHEAD
#define FP4_PERM_AHEAD perm_ahead<kTpw>()
#endif

// kFmt: kFmtMx or kFmtMxInt (kOpt = OCP floor rule), kFmtMxMat (MXFP4 after
// the 32x32 block matrix at ts, row-major fp32), kFmtNv (kOpt = RaZeR; ts
// holds s_t),
// kFmtNvAmax (no stores; work-group i leaves its largest rotated magnitude in
// the code slot of chunk i).
template <int kTpw, int kFmt, bool kHad, bool kOpt, bool kRot, int kW>
__global__ __launch_bounds__(64 * kW, FP4_PERM_WAVES) void rotq_perm_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const float* __restrict__ ts, float* __restrict__ rot,
    RotGeom g) {
  constexpr int kCpl = 2 * kTpw;
  constexpr int kAhead = FP4_PERM_AHEAD;  // rows in flight in registers beyond the next
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * 2048 * kW * kTpw];
  __shared__ float rcp_tab[128];
  const int32_t cpr = g.cols / 8;
  // perm entries first, then rows 0 .. kAhead, so the row loads are in flight
  // while the entries are unpacked
  i32x4_t v[kTpw][4];
  load_lane_perm<kTpw, kW>(perm, g, v);
  u32x4_t first[kCpl], pre[kAhead][kCpl];
  auto prow = [&](int32_t j) { return (int32_t)blockIdx.x + j * (int32_t)gridDim.x; };
  load_row<kCpl, kW>(row_rsrc<kRot>(x, codes, scales, rot, prow(0), g).x, cpr, first);
#pragma unroll
  for (int j = 1; j <= kAhead; ++j)
    load_row<kCpl, kW>(row_rsrc<kRot>(x, codes, scales, rot, prow(j), g).x, cpr, pre[j % kAhead]);
  NvScale ns{1.0f, 1.0f, true};
  if constexpr (kFmt == kFmtNv) {
    const float s_t = *ts;
    ns = nv_scale_setup(s_t);
    nv_rcp_table(rcp_tab, s_t);
  }
  uint32_t off[kTpw][8];
  const int lr = pack_lane_perm<kTpw, kW>(v, g, off);
  bf16x8_t a0, a1, m[3][2];
  if constexpr (kFmt == kFmtMxMat)
    matrix_operands(ts, false, m);
  else
    hadamard_operands<kFmt == kFmtMx || kFmt == kFmtMxInt ? 32 : 16>(a0, a1);
  put_row<kCpl, kW>(sbuf, cpr, first);
  // run length agreed by the whole work-group (this also publishes row r0 and
  // the reciprocal table)
  const int run = __syncthreads_and(lr >= 8) ? 8
                  : __syncthreads_and(lr >= 4) ? 4
                  : __syncthreads_and(lr >= 2) ? 2 : 1;
  float amax = 0.0f;
  PermCtx<kTpw, kAhead> c{x, sbuf, off, a0, a1, {{m[0][0], m[0][1]}, {m[1][0], m[1][1]},
                                                 {m[2][0], m[2][1]}},
                          codes, scales, rot, g, pre, ns, rcp_tab, &amax};
  if (run == 8)
    PermRows<8, kTpw, kAhead, kFmt, kHad, kOpt, kRot, kW>::run(c);
  else if (run == 4)
    PermRows<4, kTpw, kAhead, kFmt, kHad, kOpt, kRot, kW>::run(c);
  else if (run == 2)
    PermRows<2, kTpw, kAhead, kFmt, kHad, kOpt, kRot, kW>::run(c);
  else
    PermRows<1, kTpw, kAhead, kFmt, kHad, kOpt, kRot, kW>::run(c);
  if constexpr (kFmt == kFmtNvAmax) {
    const float m = block_max<kW>(amax, rcp_tab);
    if (threadIdx.x == 0) *amax_partial_slot(codes, blockIdx.x, g) = __float_as_uint(m);
  }
}

// ========= permuting kernel, rows staged by direct-to-LDS loads ============
// The same row computation as rotq_perm_kernel, with the rows brought into
// LDS by buffer_load_dwordx4 ... lds (gfx950), which writes each lane's 16
// bytes straight into LDS: no registers hold rows in flight and no LDS stores
// copy them in, so a work-group keeps a ring of kNB row buffers and kNB - 1
// rows in flight. Step k (row r0 + k G, G the grid size):
//   wait until this wave's loads of row k are done (vmcnt), barrier (every
//   wave's share of row k is in LDS, and every wave has finished reading the
//   buffer of row k - 1), issue the loads of row k + kNB - 1 into that freed
//   buffer, then gather, transform, quantize and store row k.
// Each step issues a fixed number of memory operations in a fixed order
// (kCpl loads, then kS stores; a scheduling barrier keeps them apart), so the
// loads of row k are exactly those with more than (kNB - 2) kCpl + (steps
// since) kS operations after them. The barrier is a bare s_barrier: a
// work-group fence would wait for every load in flight.
// The ring buffers are separate LDS objects so that the compiler sees which
// buffer each read touches and does not wait for loads into the others.
template <int kTpw, int kW, int kSlot>
__device__ __forceinline__ uint8_t* ring_buf() {
  __shared__ __attribute__((aligned(16))) uint8_t b[2048 * kW * kTpw];
  return b;
}

// s_waitcnt vmcnt(n) (n < 64) leaving the other counters alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int m = n < 63 ? n : 63;
  __builtin_amdgcn_s_waitcnt((m & 0xF) | ((m >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait for this wave's LDS operations, then meet the work-group, with no wait
// on vector memory (compiler-only fences keep memory accesses on their side).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// This wave's share of a row: operation u moves chunk c = 64 (u kW + w) +
// lane (16 bytes) of the row to buf + 16 c; chunks past the row read nothing.
template <int kCpl, int kW>
__device__ __forceinline__ void dma_row(rsrc_t src, uint8_t* buf, int32_t cpr) {
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int u = 0; u < kCpl; ++u) {
    const int32_t c = threadIdx.x + u * 64 * kW;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src, (__attribute__((address_space(3))) void*)(buf + 16 * (u * 64 * kW + 64 * w)), 16,
        c < cpr ? 16u * (uint32_t)c : kOob, 0, 0, kNt);
  }
}

// Rows of a work-group: row(k) = g + k G for k < count (g its index, G the
// grid size), past the end otherwise, so that all work-groups work on one
// window of consecutive rows at a time (measured on MI355X: a contiguous range
// of rows per work-group ran 8-12% slower); every work-group runs `steps`
// steps, the largest count.
struct RowMap {
  int32_t base, stride, count, steps;
  __device__ __forceinline__ int32_t row(int32_t k) const {
    return k < count ? base + k * stride : 0x7FFFFFFF;
  }
};

__device__ __forceinline__ RowMap row_map(int32_t rows) {
  const int32_t G_ = gridDim.x, g = blockIdx.x;
  return RowMap{g, G_, (rows - g + G_ - 1) / G_, (rows + G_ - 1) / G_};
}

template <int G, int kTpw, int kNB, int kFmt, bool kHad, bool kOpt, bool kRot, int kW>
struct DmaRows {
  using Ctx = PermCtx<kTpw, 1>;
  static constexpr int kCpl = 2 * kTpw;
  // vector-memory stores per step
  static constexpr int kS = kFmt == kFmtNvAmax ? 0 : kTpw * (2 + (kRot ? 4 : 0));

  // step k with kSt = k mod kNB; kFirst: the first kNB steps (fewer stores
  // issued since the prologue's loads)
  template <int kSt, bool kFirst>
  static __device__ __forceinline__ void step(const Ctx& c, const RowMap& m, int32_t k) {
    constexpr int kSince = kFirst ? kSt : kNB - 1;
    wait_vmcnt<(kNB - 2) * kCpl + kSince * kS>();
    lds_barrier();
    dma_row<kCpl, kW>(row_rsrc<false>(c.x, c.codes, c.scales, c.rot, m.row(k + kNB - 1), c.g).x,
                      ring_buf<kTpw, kW, (kSt + kNB - 1) % kNB>(), c.g.cols / 8);
    __builtin_amdgcn_sched_barrier(0);
    perm_row<G, 0, kTpw, kFmt, kHad, kOpt, kRot, Ctx, kW>(c, ring_buf<kTpw, kW, kSt>(), m.row(k));
    __builtin_amdgcn_sched_barrier(0);
  }

  template <bool kFirst, int... us>
  static __device__ __forceinline__ void group(const Ctx& c, const RowMap& m, int32_t k,
                                               std::integer_sequence<int, us...>) {
    (step<us, kFirst>(c, m, k + us), ...);
  }

  // Whole groups of kNB steps; rows past the end run with empty resources.
  static __device__ __forceinline__ void run(const Ctx& c, const RowMap& m) {
    group<true>(c, m, 0, std::make_integer_sequence<int, kNB>{});
    for (int32_t k = kNB; k < m.steps; k += kNB)
      group<false>(c, m, k, std::make_integer_sequence<int, kNB>{});
    wait_vmcnt<0>();  // no load into LDS outlives the work-group
  }
};

template <int kTpw, int kW, int kNB, int j>
__device__ __forceinline__ void dma_prologue(const uint16_t* x, const RotGeom& g,
                                             const RowMap& m) {
  if constexpr (j < kNB - 1) {
    dma_row<2 * kTpw, kW>(row_rsrc<false>(x, nullptr, nullptr, nullptr, m.row(j), g).x,
                          ring_buf<kTpw, kW, j>(), g.cols / 8);
    dma_prologue<kTpw, kW, kNB, j + 1>(x, g, m);
  }
}


template <int kTpw, int kFmt, bool kHad, bool kOpt, bool kRot, int kW, int kWgs>
__global__ __launch_bounds__(64 * kW, (kW * kWgs + 3) / 4) void rotq_perm_dma_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, const float* __restrict__ ts, float* __restrict__ rot,
    RotGeom g) {
  // as many row buffers as fit in this work-group's share of 152 KB of LDS
  // (kWgs work-groups per CU), at most four
  constexpr int kNBmax = (152 * 1024 / kWgs) / (2048 * kW * kTpw);
  constexpr int kNB = kNBmax < 4 ? kNBmax : 4;
  static_assert(kNB >= 2, "two row buffers at least");
  __shared__ float rcp_tab[128];
  __shared__ uint32_t vote[kW];
  // perm entries first, then the first kNB - 1 rows, so the row loads are in
  // flight while the entries are unpacked
  i32x4_t v[kTpw][4];
  load_lane_perm<kTpw, kW>(perm, g, v);
  const RowMap rm = row_map(g.rows);
  dma_prologue<kTpw, kW, kNB, 0>(x, g, rm);
  NvScale ns{1.0f, 1.0f, true};
  if constexpr (kFmt == kFmtNv) {
    const float s_t = *ts;
    ns = nv_scale_setup(s_t);
    nv_rcp_table(rcp_tab, s_t);
  }
  uint32_t off[kTpw][8];
  const int lr = pack_lane_perm<kTpw, kW>(v, g, off);
  bf16x8_t a0, a1, m[3][2];
  if constexpr (kFmt == kFmtMxMat)
    matrix_operands(ts, false, m);
  else
    hadamard_operands<kFmt == kFmtMx || kFmt == kFmtMxInt ? 32 : 16>(a0, a1);
  // run length agreed by the whole work-group (the barrier also publishes
  // the reciprocal table); bit i of a wave's vote: every lane has runs >= 2^i
  const uint32_t mine = (lr >= 2 ? 1u : 0u) | (lr >= 4 ? 2u : 0u) | (lr >= 8 ? 4u : 0u);
  uint32_t wv = mine;
#pragma unroll
  for (int off_ = 32; off_ >= 1; off_ >>= 1) wv &= (uint32_t)__shfl_xor((int)wv, off_, 64);
  if ((threadIdx.x & 63) == 0) vote[threadIdx.x >> 6] = wv;
  lds_barrier();
  uint32_t all = vote[0];
#pragma unroll
  for (int i = 1; i < kW; ++i) all &= vote[i];
  const int run = (all & 4u) ? 8 : (all & 2u) ? 4 : (all & 1u) ? 2 : 1;
  float amax = 0.0f;
  PermCtx<kTpw, 1> c{x, nullptr, off, a0, a1, {{m[0][0], m[0][1]}, {m[1][0], m[1][1]},
                                               {m[2][0], m[2][1]}},
                     codes, scales, rot, g, nullptr, ns, rcp_tab, &amax};
  if (run == 8)
    DmaRows<8, kTpw, kNB, kFmt, kHad, kOpt, kRot, kW>::run(c, rm);
  else if (run == 4)
    DmaRows<4, kTpw, kNB, kFmt, kHad, kOpt, kRot, kW>::run(c, rm);
  else if (run == 2)
    DmaRows<2, kTpw, kNB, kFmt, kHad, kOpt, kRot, kW>::run(c, rm);
  else
    DmaRows<1, kTpw, kNB, kFmt, kHad, kOpt, kRot, kW>::run(c, rm);
  if constexpr (kFmt == kFmtNvAmax) {
    __syncthreads();  // vote[] is reused by block_max
    const float mx = block_max<kW>(amax, reinterpret_cast<float*>(vote));
    if (threadIdx.x == 0) *amax_partial_slot(codes, blockIdx.x, g) = __float_as_uint(mx);
  }
}

// NVFP4 without a permutation: the tile layout of the MXFP4 streaming kernel
// (a wave takes 32 consecutive 32-element segments); lane (n, h) holds one
// whole 16-element block, 2 (32 t + n) + h in row-major block order.
template <bool kFlat, bool kHad, bool kRazer, bool kRot, bool kAmax>
__global__ __launch_bounds__(kThreads) void nv_rotq_stream_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    const float* __restrict__ ts, float* __restrict__ rot, RotGeom g) {
  __shared__ float rcp_tab[128];
  bf16x8_t a0, a1;
  hadamard_operands<16>(a0, a1);
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
      so[u] = r * g.ld_s + 2 * (int64_t)cb + h;
      ro[u] = r * g.ld_rot + 32 * (int64_t)cb + 16 * h;
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(x + xo[u]);
      lo[u] = __builtin_nontemporal_load(p);
      hi[u] = __builtin_nontemporal_load(p + 1);
    }
  }
  NvScale ns{1.0f, 1.0f, true};
  if constexpr (!kAmax) {
    const float s_t = *ts;
    ns = nv_scale_setup(s_t);
    nv_rcp_table(rcp_tab, s_t);
    __syncthreads();
  }
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    if (tile0 + u * kWaves >= ntiles) break;  // uniform across the wave
    float y[16];
    if (kHad) {
      hadamard_mfma<16>(a0, a1, lo[u], hi[u], y);
    } else {
      widen8(lo[u], y);
      widen8(hi[u], y + 8);
    }
    if constexpr (kAmax) {
      if (ok[u]) amax = __builtin_fmaxf(amax, absmax16f(y));
    } else {
      uint32_t w0, w1, byte;
      nv_quant16<kRazer>(y, ns, rcp_tab, w0, w1, byte);
      if (ok[u]) {
        uint32_t* cp = reinterpret_cast<uint32_t*>(codes + co[u]);
        __builtin_nontemporal_store(w0, cp);
        __builtin_nontemporal_store(w1, cp + 1);
        scales[so[u]] = (uint8_t)byte;
        if (kRot) {
          store_rot8(rot + ro[u], y);
          store_rot8(rot + ro[u] + 8, y + 8);
        }
      }
    }
  }
  if constexpr (kAmax) {
    const float m = block_max(amax, rcp_tab);
    if (threadIdx.x == 0) *amax_partial_slot(codes, blockIdx.x, g) = __float_as_uint(m);
  }
}

// ================================ launchers =================================
// Each work-group owns a fixed share of the rows, so the grid is balanced
// only if every CU holds the same number of work-groups: the launch asks for
// enough (unused) dynamic LDS that no more than perm_wgs_per_cu fit on a CU,
// and launches exactly that many per CU.
template <int kTpw, int kFmt, bool kHad, bool kOpt, bool kRot, int kW = kWaves>
static int perm_launch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                       uint8_t* sc, const float* ts, float* rot, const RotGeom& g,
                       hipStream_t st) {
#ifdef FP4_PERM_WG_PER_CU
  constexpr int kWgs = FP4_PERM_WG_PER_CU;
#else
  constexpr int kWgs = perm_wgs_per_cu<kTpw, kW>();
#endif
  const DeviceInfo ci = device_info();
  const int64_t wgs = (int64_t)ci.cus * kWgs;
  const int grid = (int)(s.rows < wgs ? s.rows : wgs);
  constexpr size_t kStatic = 2 * 2048 * kW * kTpw;
  const size_t share = (size_t)ci.lds / kWgs;  // > lds / (kWgs + 1), so kWgs fit, not more
  const size_t pad = share > kStatic + 1024 ? share - kStatic - 1024 : 0;
  hipLaunchKernelGGL((rotq_perm_kernel<kTpw, kFmt, kHad, kOpt, kRot, kW>), dim3(grid),
                     dim3(64 * kW), pad, st, x, perm, c, sc, ts, rot, g);
  return grid;
}

// Rows of 16385..32768 columns: staged by direct-to-LDS loads, one work-group
// of kW waves per CU (the ring of row slots takes most of the LDS; kW * 64
// threads share it).
template <int kTpw, int kFmt, bool kHad, bool kOpt, bool kRot, int kW, int kWgs = 1>
static int perm_dma_launch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                           uint8_t* sc, const float* ts, float* rot, const RotGeom& g,
                           hipStream_t st) {
  const DeviceInfo ci = device_info();
  const int64_t wgs = (int64_t)ci.cus * kWgs;
  const int grid = (int)(s.rows < wgs ? s.rows : wgs);
  hipLaunchKernelGGL((rotq_perm_dma_kernel<kTpw, kFmt, kHad, kOpt, kRot, kW, kWgs>), dim3(grid),
                     dim3(64 * kW), 0, st, x, perm, c, sc, ts, rot, g);
  return grid;
}

// Permuting path; returns the number of work-groups launched.
template <int kFmt, bool kHad, bool kOpt, bool kRot>
static int perm_dispatch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                         uint8_t* sc, const float* ts, float* rot, const RotGeom& g,
                         hipStream_t st) {
  // MFMA tiles (32 segments) per wave per row at four waves per work-group;
  // rows of up to 8192 columns: eight waves of one tile
  const int64_t tpw = (s.cols + 32 * 32 * kWaves - 1) / (32 * 32 * kWaves);
  if (tpw <= 1) return perm_launch<1, kFmt, kHad, kOpt, kRot>(s, perm, x, c, sc, ts, rot, g, st);
  if (tpw <= 2) return perm_launch<1, kFmt, kHad, kOpt, kRot, 8>(s, perm, x, c, sc, ts, rot, g, st);
  if (tpw <= 3) return perm_launch<3, kFmt, kHad, kOpt, kRot>(s, perm, x, c, sc, ts, rot, g, st);
  if (tpw <= 4) return perm_launch<4, kFmt, kHad, kOpt, kRot>(s, perm, x, c, sc, ts, rot, g, st);
  // rows of 16385..32768 columns: sixteen waves of two tiles (measured on
  // MI355X at 8192 x 28672 against four waves of seven tiles: MXFP4 107.1 ->
  // 100.6 us, MXINT4 138.3 -> 104.4, NVFP4 + RaZeR 146.5 -> 111.8; eight waves
  // of four tiles: 100.0, 112.9, 136.9)
  return perm_dma_launch<2, kFmt, kHad, kOpt, kRot, 16>(s, perm, x, c, sc, ts, rot, g, st);
}

template <bool kHad, bool kFloor, bool kRot, bool kInt>
static void rotq_dispatch(const Shape& s, const int32_t* perm, const uint16_t* x, uint8_t* c,
                          uint8_t* sc, float* rot, const RotGeom& g, bool flat, hipStream_t st) {
  if (perm) {
    (void)perm_dispatch<kInt ? kFmtMxInt : kFmtMx, kHad, kFloor, kRot>(s, perm, x, c, sc, nullptr,
                                                                      rot, g, st);
    return;
  }
  // the butterfly variant quantizes MXFP4 only
  if constexpr (kUseMfma || kInt) {
    const uint64_t tiles = ((uint64_t)g.nblk + 15) / 16;
    const uint64_t grid = (tiles + kWaves * kSpreadTiles - 1) / (kWaves * kSpreadTiles);
    if (flat)
      hipLaunchKernelGGL((mx_rotq_stream_mfma_kernel<true, kHad, kFloor, kRot, kInt>),
                         dim3((int)grid), dim3(kThreads), 0, st, x, c, sc, rot, g);
    else
      hipLaunchKernelGGL((mx_rotq_stream_mfma_kernel<false, kHad, kFloor, kRot, kInt>),
                         dim3((int)grid), dim3(kThreads), 0, st, x, c, sc, rot, g);
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

template <bool kInt>
static void mx_rotq_variants(const Shape& s, const int32_t* perm, bool had, bool floor_rule,
                             const uint16_t* xp, uint8_t* cp, uint8_t* sp, float* rot,
                             const RotGeom& g, bool flat, hipStream_t st) {
  const bool r = rot != nullptr;
  if (had && !floor_rule && !r) rotq_dispatch<true, false, false, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && !floor_rule && r) rotq_dispatch<true, false, true, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && floor_rule && !r) rotq_dispatch<true, true, false, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (had && floor_rule && r) rotq_dispatch<true, true, true, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && !floor_rule && !r) rotq_dispatch<false, false, false, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && !floor_rule && r) rotq_dispatch<false, false, true, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && floor_rule && !r) rotq_dispatch<false, true, false, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
  if (!had && floor_rule && r) rotq_dispatch<false, true, true, kInt>(s, perm, xp, cp, sp, rot, g, flat, st);
}

// MXINT4 instances of the above, compiled in rotate_int.hip.
void mxint_rotate_quant(const Shape& s, const int32_t* perm, bool had, bool floor_rule,
                        const uint16_t* x, uint8_t* codes, uint8_t* scales, float* rot,
                        const RotGeom& g, bool flat, hipStream_t st);

}  // namespace fp4

#endif  // FP4_ROTATE_KERNELS_HPP
