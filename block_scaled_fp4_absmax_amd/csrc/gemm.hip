// gemm.hip -- C = A B^T with both operands in MXFP4, on gfx950's scaled FP4
// matrix cores.
//
// The consumer of the quantized tensors ("RaZeR: Pushing the Limits of NVFP4
// Quantization with Redundant Zero Remapping", technical summary sec. 2.3:
// weight-and-activation GEMM kernels on the quantized formats). A is [M, K]
// (activations), B is [N, K] (weights, one row per output channel), both in
// the layout the quantizer writes: codes [rows, K/2] (element 2i in the low
// nibble of byte i) and E8M0 scales [rows, K/32], row-major. The GEMM reads
// them as they are; the per-stage copy into LDS is the only re-layout.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operand formats FP4 E2M1 computes
// a 32 x 32 tile over 64 K values: lane (r, h) = (lane % 32, lane / 32)
// supplies 16 code bytes, the 32 elements of one 32-element K block of row r
// (of A, or of B for the other operand), and that block's E8M0 byte as its
// scale; the products of E2M1 values are exact and the hardware applies
// 2^(e_a + e_b) per block pair before accumulating in fp32. The output lane
// (n, h) holds column n and rows 8 (q / 4) + 4 h + q % 4 in register q. The
// layout and the exactness of the products were confirmed on the GPU with an
// in-bounds probe.
//
// Tiling: a work-group of VM x VN waves computes a (32 WM VM) x (32 WN VN)
// tile of C (256 x 256 from eight waves for large products, 128 x 128 from
// four otherwise); wave (wm, wn) owns WM x WN MFMA tiles. K advances KB (256
// or 128) elements per stage: the work-group copies the stage's rows of KB / 2
// code bytes of A and of B, and their KB / 32 scale bytes per row, into one of
// two LDS buffers
// (16-byte chunks swizzled within each row so that the lane writes and the
// MFMA operand reads are free of bank conflicts), while the waves multiply
// out of the other; the loads of two or three stages are held in registers
// meanwhile. Loads past
// M, N or K read zeros through buffer-resource range checks (code 0 is +0),
// so any K that is a multiple of 32 works.
#include <type_traits>

#include "fp4_device.hpp"
#include "launch.hpp"
#include "split_k.hpp"

namespace fp4 {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// LDS byte offset of 16-byte chunk c of row r in a stage of KB K values
// (KB / 32 chunks per row). gfx950's LDS has 64 four-byte banks (256 bytes):
// a 16-byte access pass of 16 lanes is free of conflicts when its 16 chunks
// fall on 16 different 16-byte bank groups. KB = 256 (128-byte rows, two rows
// per bank cycle): chunk c (0..7) sits in slot c ^ ((r / 2) % 8), so a read
// pass (one logical chunk of 16 consecutive rows) covers both row parities
// times eight slots, and a write pass (two whole rows) covers them too.
// KB = 128 (64-byte rows, four per bank cycle): slot c ^ ((r / 4) % 4). The
// earlier XOR by r % 8 (or (r / 2) % 4), right for 32 banks, measured 0.35
// bank-conflict cycles per LDS-active cycle here; this one 0.
template <int KB>
__device__ __forceinline__ uint32_t lds_off(uint32_t r, uint32_t c) {
  if constexpr (KB == 128)
    return r * 64u + 16u * (c ^ ((r >> 2) & 3u));
  else
    return r * 128u + 16u * (c ^ ((r >> 1) & 7u));
}

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  int64_t ld_a, ld_sa, ld_b, ld_sb, ld_c;  // bytes (codes, scales), elements (C)
  int32_t m, n, k;
  bool sg_a, sg_b;  // scale bytes in the GEMM order (ld_s: 32-row group stride)
};

// Scale bytes of an operand tile of `rows` rows from row r0 (a multiple of
// 32), row-major or in the GEMM order (scale_row_off).
__device__ __forceinline__ rsrc_t scale_rsrc(const uint8_t* s, int64_t ld, bool gemm, int32_t r0,
                                             int32_t rows) {
  return make_rsrc(s + scale_row_off(r0, ld, gemm),
                   (uint32_t)(gemm ? (int64_t)((rows + 31) / 32) * ld : (int64_t)rows * ld));
}

// Offset in that tile of the scale dword of row `row`, blocks blk .. blk + 3
// (blk % 4 == 0, so the dword never crosses a row or an 8-block step). Both
// offsets are computed and one is kept by a mask: a select on the flag
// becomes a branch inside the K loop, which splits the loop's schedule.
__device__ __forceinline__ uint32_t scale_dword_off(uint32_t row, uint32_t blk, uint32_t ld,
                                                    bool gemm) {
  const uint32_t rm = row * ld + blk;
  const uint32_t go = (row >> 5) * ld + 8u * (row & 31u) + scale_col_off(blk, true);
  return rm ^ ((rm ^ go) & (0u - (uint32_t)gemm));
}

struct OperandRsrc {
  rsrc_t a, sa, b, sb;
};

// Work-group tile BM x BN = (32 WM VM) x (32 WN VN): VM x VN waves, wave
// (wm, wn) owns WM x WN MFMA tiles of 32 x 32 at rows 32 WM wm..,
// columns 32 WN wn..
template <int WM, int WN, int VM, int VN, int KB>
struct Tile {
  static constexpr int BM = 32 * WM * VM, BN = 32 * WN * VN;
  static constexpr int kT = 64 * VM * VN;                     // threads
  static constexpr int kRowBytes = KB / 2;                    // code bytes per row per stage
  static constexpr int kCpr = kRowBytes / 16;                 // 16-byte chunks per row
  static constexpr int kSW = KB / 128;                        // scale dwords per row
  static constexpr int kChunksA = BM * kRowBytes / 16 / kT;   // 16-byte chunks per lane
  static constexpr int kChunksB = BN * kRowBytes / 16 / kT;
  static constexpr int kScaleRows = (BM + BN) * kSW / kT;     // scale dwords per lane
  static_assert(kChunksA * kT * 16 == BM * kRowBytes && kChunksB * kT * 16 == BN * kRowBytes &&
                    kScaleRows * kT == (BM + BN) * kSW && BM % 64 == 0,
                "the stage divides evenly over the lanes");
  static constexpr int kLdsA = BM * kRowBytes, kLdsB = BN * kRowBytes;

  // One stage in flight in registers: code chunks of A and B, and the KB / 32
  // scale bytes of each scale row (kSW dwords; scale rows are 4-byte aligned).
  struct Regs {
    u32x4_t a[kChunksA], b[kChunksB];
    uint32_t s[kScaleRows];
  };

  static __device__ __forceinline__ void load(const OperandRsrc& q, const GemmArgs& g, int32_t k0,
                                              Regs& r) {
    const uint32_t t = threadIdx.x;
    const uint32_t kb0 = (uint32_t)k0 / 2u, kbytes = (uint32_t)g.k / 2u;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk / kCpr, col = 16u * (chunk % kCpr);
      r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(
          q.a, kb0 + col < kbytes ? row * (uint32_t)g.ld_a + kb0 + col : kOob, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk / kCpr, col = 16u * (chunk % kCpr);
      r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(
          q.b, kb0 + col < kbytes ? row * (uint32_t)g.ld_b + kb0 + col : kOob, 0, 0);
    }
    // scale dword e of the stage: row e / kSW (rows 0 .. BM-1 of A, then
    // BM .. BM+BN-1 of B), dword e % kSW of its KB / 32 bytes; lane t takes
    // dwords t + kT i, whose operand is uniform across a wave
    const uint32_t blk0 = (uint32_t)k0 / 32u, nblk = (uint32_t)g.k / 32u;
#pragma unroll
    for (int i = 0; i < kScaleRows; ++i) {
      const uint32_t e = t + (uint32_t)kT * i, j = e / kSW;
      const uint32_t blk = blk0 + 4u * (e % kSW);
      const bool is_a = __builtin_amdgcn_readfirstlane(e >> 6) < (uint32_t)(BM * kSW) / 64u;
      const rsrc_t rs = is_a ? q.sa : q.sb;
      const uint32_t row = is_a ? j : j - BM;
      const uint32_t off =
          scale_dword_off(row, blk, (uint32_t)(is_a ? g.ld_sa : g.ld_sb), is_a ? g.sg_a : g.sg_b);
      // blk is a multiple of 4 below nblk <= k / 32, so the dword stays
      // inside the row; bytes past K are cleared when stored
      r.s[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, blk < nblk ? off : kOob, 0, 0);
    }
  }

  // smask(d): which bytes of scale dword d (0 .. kSW - 1) of the stage lie
  // before the end of K
  template <typename Mask>
  static __device__ __forceinline__ void store(uint8_t* la, uint8_t* lb, uint32_t* ls,
                                               const Regs& r, Mask smask) {
    const uint32_t t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk / kCpr, c = chunk % kCpr;
      *reinterpret_cast<u32x4_t*>(la + lds_off<KB>(row, c)) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < kChunksB; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk / kCpr, c = chunk % kCpr;
      *reinterpret_cast<u32x4_t*>(lb + lds_off<KB>(row, c)) = r.b[i];
    }
#pragma unroll
    for (int i = 0; i < kScaleRows; ++i) {
      const uint32_t e = t + (uint32_t)kT * i;
      ls[e] = r.s[i] & smask(e % kSW);
    }
  }
};

// Epilogue of a work-group tile: lane (n, h) of MFMA tile (i, j) holds
// column n and rows 8 (e / 4) + 4 h + e % 4, e = 0..15. bf16 goes through LDS
// (kLds: the two operand buffer pairs la, lb are free after the last stage's
// barrier and hold a row half each): the waves of row half wm write their
// tiles into la (wm = 0) or lb (wm = 1), BM / 2 rows of BN bf16, then every
// thread copies 16-byte pieces of whole rows out. 16-byte piece p of row rl
// sits in slot p ^ 4 ((rl / 4) % 2), so that the two lane halves of a write
// (rows 4 apart) use different banks. That needs ld_c % 8 == 0 and a 16-byte
// aligned C; otherwise, and for fp32, each element is stored directly.
template <int WM, int WN, int VM, int VN, bool kBf16Out, bool kLds>
__device__ __forceinline__ void tile_epilogue(const f32x16_t (&acc)[WM][WN], const GemmArgs& g,
                                              int32_t m0, int32_t n0, uint32_t wm, uint32_t wn,
                                              uint32_t r, uint32_t h, uint8_t* la, uint8_t* lb) {
  constexpr int BM = 32 * WM * VM, BN = 32 * WN * VN, kT = 64 * VM * VN;
  if constexpr (kBf16Out && kLds && VM == 2) {
    const bool via_lds = g.ld_c % 8 == 0 && reinterpret_cast<uintptr_t>(g.c) % 16 == 0;
    if (via_lds) {
      constexpr int kHalf = BM / 2;
      uint8_t* half = wm == 0 ? la : lb;
      auto slot = [](uint32_t rl, uint32_t p) { return p ^ (4u * ((rl >> 2) & 1u)); };
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint32_t cl = 32u * WN * wn + 32u * j + r;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t rl = 32u * i + 8u * (e / 4) + 4u * h + (e % 4);
            const uint32_t off = rl * (2u * BN) + 16u * slot(rl, cl / 8u) + 2u * (cl % 8u);
            *reinterpret_cast<uint16_t*>(half + off) =
                (uint16_t)(pack_bf16x2(acc[i][j][e], 0.0f) & 0xFFFFu);
          }
        }
      __syncthreads();
      constexpr int kPieces = BM * BN / 8;  // 16-byte pieces of the tile
      constexpr int kPpr = BN / 8;          // per row
#pragma unroll
      for (int u = 0; u < kPieces / kT; ++u) {
        const uint32_t pc = threadIdx.x + (uint32_t)kT * u;
        const uint32_t row = pc / kPpr, p = pc % kPpr;
        const uint32_t rl = row % kHalf;
        const uint8_t* src = (row < (uint32_t)kHalf ? la : lb) + rl * (2u * BN) + 16u * slot(rl, p);
        const int32_t grow = m0 + (int32_t)row, gcol = n0 + 8 * (int32_t)p;
        if (grow >= g.m || gcol >= g.n) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src);
        uint16_t* dst = static_cast<uint16_t*>(g.c) + (int64_t)grow * g.ld_c + gcol;
        if (gcol + 8 <= g.n) {
          *reinterpret_cast<u32x4_t*>(dst) = v;
        } else {
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (gcol + t < g.n) dst[t] = (uint16_t)(w4[t / 2] >> (16 * (t % 2)));
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int32_t col = n0 + 32 * WN * (int32_t)wn + 32 * j + (int32_t)r;
      if (col >= g.n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t row =
            m0 + 32 * WM * (int32_t)wm + 32 * i + 8 * (e / 4) + 4 * (int32_t)h + e % 4;
        if (row >= g.m) continue;
        if constexpr (kBf16Out) {
          const uint32_t pv = pack_bf16x2(acc[i][j][e], 0.0f);
          static_cast<uint16_t*>(g.c)[(int64_t)row * g.ld_c + col] = (uint16_t)(pv & 0xFFFFu);
        } else {
          static_cast<float*>(g.c)[(int64_t)row * g.ld_c + col] = acc[i][j][e];
        }
      }
    }
}

template <int WM, int WN, int VM, int VN, int KB, int kSets, bool kBf16Out>
__global__ __launch_bounds__(64 * VM * VN) void mx_gemm_kernel(GemmArgs g) {
  using T = Tile<WM, WN, VM, VN, KB>;
  constexpr int BM = T::BM, BN = T::BN, kSW = T::kSW, kBK = KB;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][T::kLdsA];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][T::kLdsB];
  __shared__ uint32_t lds_s[2][(BM + BN) * kSW];

  const int32_t tiles_n = (g.n + BN - 1) / BN;
  const int32_t bm = blockIdx.x / tiles_n, bn = blockIdx.x - bm * tiles_n;
  const int32_t m0 = bm * BM, n0 = bn * BN;
  const int32_t rows_a = min(BM, g.m - m0), rows_b = min(BN, g.n - n0);
  OperandRsrc q;
  q.a = make_rsrc(g.a + (int64_t)m0 * g.ld_a, (uint32_t)(rows_a * g.ld_a));
  q.b = make_rsrc(g.b + (int64_t)n0 * g.ld_b, (uint32_t)(rows_b * g.ld_b));
  q.sa = scale_rsrc(g.sa, g.ld_sa, g.sg_a, m0, rows_a);
  q.sb = scale_rsrc(g.sb, g.ld_sb, g.sg_b, n0, rows_b);

  const uint32_t lane = threadIdx.x & 63u, r = lane & 31u, h = lane >> 5;
  const uint32_t w = threadIdx.x >> 6, wm = w / VN, wn = w % VN;

  f32x16_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // multiply out the stage held in LDS buffer buf: KB / 64 K steps of 64
  auto mma = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KB / 64; ++ks) {
      // 16-byte chunk kc of the row; its scale byte kc of the row's KB / 32
      const uint32_t kc = 2u * ks + h, sd = kc / 4u, sh = 8u * (kc % 4u);
      u32x4_t fa[WM], fb[WN];
      int32_t sa[WM], sb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const uint32_t ra = 32u * WM * wm + 32u * i + r;
        fa[i] = *reinterpret_cast<const u32x4_t*>(lds_a[buf] + lds_off<KB>(ra, kc));
        sa[i] = (int32_t)((lds_s[buf][ra * kSW + sd] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint32_t rb = 32u * WN * wn + 32u * j + r;
        fb[j] = *reinterpret_cast<const u32x4_t*>(lds_b[buf] + lds_off<KB>(rb, kc));
        sb[j] = (int32_t)((lds_s[buf][(BM + rb) * kSW + sd] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const i32x8_t va{(int32_t)fa[i].x, (int32_t)fa[i].y, (int32_t)fa[i].z,
                           (int32_t)fa[i].w, 0, 0, 0, 0};
          const i32x8_t vb{(int32_t)fb[j].x, (int32_t)fb[j].y, (int32_t)fb[j].z,
                           (int32_t)fb[j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc[i][j], 4, 4, 0,
                                                                     sa[i], 0, sb[j]);
        }
    }
  };

  // kSets stages in flight in registers: while stage s is multiplied out of
  // LDS buffer s % 2, register set s % kSets (whose stage is already in LDS)
  // receives stage s + kSets, and the other sets hold stages s + 1 ..
  // s + kSets - 1; stage s + 1 is stored into the other LDS buffer
  // afterwards. Loads are unconditional: past K they read zeros without
  // touching memory, so every stage issues the same operations and each
  // store waits for its own stage's loads only.
  const int32_t stages = (g.k + kBK - 1) / kBK;
  // scale bytes of a stage that lie past K (the last, partial stage) are
  // cleared: their codes read as zero, and a stray 0xFF would make 0 * NaN
  const uint32_t nblk = (uint32_t)g.k / 32u;
  auto smask = [&](int32_t st) {
    return [=](uint32_t d) {
      const uint32_t b0 = (uint32_t)(KB / 32) * (uint32_t)st + 4u * d;
      return b0 + 4u <= nblk ? 0xFFFFFFFFu : b0 >= nblk ? 0u : (1u << (8u * (nblk - b0))) - 1u;
    };
  };
  typename T::Regs rs[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) T::load(q, g, j * kBK, rs[j]);
  T::store(lds_a[0], lds_b[0], lds_s[0], rs[0], smask(0));
  __syncthreads();
  // stage s with register set j = s % kSets (a compile-time index)
  auto step = [&](auto J, int32_t s) {
    constexpr int j = decltype(J)::value;
    const int buf = s & 1;
    T::load(q, g, (s + kSets) * kBK, rs[j]);
    mma(buf);
    T::store(lds_a[buf ^ 1], lds_b[buf ^ 1], lds_s[buf ^ 1], rs[(j + 1) % kSets], smask(s + 1));
    __syncthreads();
  };
  auto group = [&]<int... js>(int32_t s0, std::integer_sequence<int, js...>) {
    (step(std::integral_constant<int, js>{}, s0 + js), ...);
  };
  auto tail = [&]<int... js>(int32_t s0, std::integer_sequence<int, js...>) {
    (void)((s0 + js < stages ? (step(std::integral_constant<int, js>{}, s0 + js), true) : false) &&
           ...);
  };
  int32_t s = 0;
  for (; s + kSets - 1 < stages; s += kSets) group(s, std::make_integer_sequence<int, kSets>{});
  tail(s, std::make_integer_sequence<int, kSets - 1>{});

  tile_epilogue<WM, WN, VM, VN, kBf16Out, KB >= BN>(acc, g, m0, n0, wm, wn, r, h, &lds_a[0][0],
                                                  &lds_b[0][0]);
}

// Split-K products, for few rows of A (decode and small batches) and for
// products with few 128 x 128 tiles: a work-group of eight waves computes
// MT x NT tiles of 32 x 32 of C (rows past m or n read as zeros); wave w
// takes the 256-K super-steps w, w + 8, ... (the waves of a work-group read
// neighbouring pieces of each row) and the partial tiles are added in LDS in
// wave order (deterministic). A super-step of an operand piece is 32 rows x
// 128 code bytes: it is loaded with each 128-byte row piece read by eight
// consecutive lanes (whole lines per instruction; one row per lane measured
// 1.5x slower), kept in registers while later steps load, then passed
// through the wave's own LDS buffer (16-byte chunks XOR-swizzled by row, so
// that the writes and the reads are free of bank conflicts) to the MFMA
// layout: lane (r, h) takes the 64 bytes 64 h .. 64 h + 63 of row r (blocks
// 4 h .. 4 h + 3), with the dword of their four scale bytes; MFMA c of a tile
// pair takes block 4 h + c in lane half h for both operands, which pairs the
// same K block of A and B in every lane. The operand bytes each CU streams
// bound these products, so the tile shape (1 x 1, 1 x 2 or 2 x 2) is chosen
// per product by skinny_shape; at n = k = 8192 (1 x 2 and 2 x 2 tiles):
// m = 64 in 11.4 us and m = 128 in 16.2 us, against 32-34 us for one 32 x 32
// tile per work-group or the 128 x 128 tiles.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyMaxM = 256;  // larger m always takes the 128 x 128 or 256 x 256 tiles

// A work-group's operand pieces: MT pieces of A (32 rows each) and NT of B.
template <int MT, int NT>
struct SkinnyStep {
  u32x4_t v[MT + NT][4];  // row 8 c + lane / 8 of the piece, 16-byte chunk lane % 8
  uint32_t s[MT + NT];    // row lane % 32 of the piece, blocks 4 (lane / 32) .. + 3
};

// LDS byte offset of 16-byte chunk j (0..7) of row r in a 32 x 128-byte
// operand piece (slot j ^ ((r / 2) % 8): see lds_off for the 64 banks).
__device__ __forceinline__ uint32_t skinny_off(uint32_t r, uint32_t j) {
  return 128u * r + 16u * (j ^ ((r >> 1) & 7u));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int MT, int NT, int kSets, bool kBf16Out>
__global__ __launch_bounds__(64 * kSkinnyWaves) void mx_gemm_skinny_kernel(GemmArgs g) {
  constexpr int kP = MT + NT;
  constexpr int kOps = kSkinnyWaves * kP * 4096;                  // operand pieces
  constexpr int kRed = kSkinnyWaves * 64 * MT * NT * 64;          // partial tiles
  // per wave: the pieces of the step being multiplied; afterwards the same
  // memory holds the partial tiles of all waves
  __shared__ __attribute__((aligned(16))) uint8_t smem[kOps > kRed ? kOps : kRed];
  const SkinnyTile tile = skinny_tile(blockIdx.x, (g.m + 32 * MT - 1) / (32 * MT));
  const int32_t n0 = tile.x * 32 * NT, m0 = tile.y * 32 * MT;
  if (n0 >= g.n) return;  // padding of the grid to whole XCD rounds
  const int32_t rows_a = min(32 * MT, g.m - m0), rows_b = min(32 * NT, g.n - n0);
  const rsrc_t ra = make_rsrc(g.a + (int64_t)m0 * g.ld_a, (uint32_t)(rows_a * g.ld_a));
  const rsrc_t rsa = scale_rsrc(g.sa, g.ld_sa, g.sg_a, m0, rows_a);
  const rsrc_t rb = make_rsrc(g.b + (int64_t)n0 * g.ld_b, (uint32_t)(rows_b * g.ld_b));
  const rsrc_t rsb = scale_rsrc(g.sb, g.ld_sb, g.sg_b, n0, rows_b);
  const uint32_t lane = threadIdx.x & 63u, r = lane & 31u, h = lane >> 5;
  const int32_t w = (int32_t)(threadIdx.x >> 6);
  uint8_t* const lw = smem + kP * 4096u * (uint32_t)w;
  const uint32_t kbytes = (uint32_t)g.k / 2u, nblk = (uint32_t)g.k / 32u;
  const int32_t steps = (g.k + 255) / 256;
  const int32_t cnt = steps > w ? (steps - w + kSkinnyWaves - 1) / kSkinnyWaves : 0;

  // loads of the wave's i-th super-step s = w + 8 i (i >= cnt or past K:
  // offsets out of range, which read zeros without touching memory)
  auto load = [&](int32_t i, SkinnyStep<MT, NT>& t) {
    const int32_t s = w + kSkinnyWaves * i;
    const bool live = i < cnt;
    const uint32_t off = 128u * (uint32_t)s + 16u * (lane & 7u);
    const bool ok = live && off < kbytes;
    // blk is a multiple of 4 below nblk <= k / 32: the dword stays inside
    // the row; bytes past K are cleared before use
    const uint32_t blk = 8u * (uint32_t)s + 4u * h;
    const bool oks = live && blk < nblk;
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      const bool pa = p < MT;
      const uint32_t base = 32u * (uint32_t)(pa ? p : p - MT);
      const uint32_t ld = (uint32_t)(pa ? g.ld_a : g.ld_b);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t row = base + 8u * c + (lane >> 3);
        t.v[p][c] = __builtin_amdgcn_raw_buffer_load_b128(pa ? ra : rb,
                                                          ok ? row * ld + off : kOob, 0, 0);
      }
      const uint32_t lds_ = (uint32_t)(pa ? g.ld_sa : g.ld_sb);
      const uint32_t so = scale_dword_off(base + r, blk, lds_, pa ? g.sg_a : g.sg_b);
      t.s[p] = __builtin_amdgcn_raw_buffer_load_b32(pa ? rsa : rsb, oks ? so : kOob, 0, 0);
    }
  };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mma = [&](int32_t i, const SkinnyStep<MT, NT>& t) {
    const int32_t s = w + kSkinnyWaves * i;
    const uint32_t blk = 8u * (uint32_t)s + 4u * h;
    const uint32_t keep = blk + 4u <= nblk ? 0xFFFFFFFFu
                          : blk >= nblk   ? 0u
                                          : (1u << (8u * (nblk - blk))) - 1u;
    // through the wave's LDS buffer into the MFMA layout (the previous
    // step's reads are done first)
    wave_sync();
#pragma unroll
    for (int p = 0; p < kP; ++p)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4_t*>(lw + 4096u * p + skinny_off(8u * c + (lane >> 3), lane & 7u)) =
            t.v[p][c];
    wave_sync();
    // MFMA c of every tile pair takes chunk c of each piece: operands are
    // read from LDS per chunk (each one a whole 8-register MFMA operand)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      i32x8_t va[MT], vb[NT];
#pragma unroll
      for (int p = 0; p < kP; ++p) {
        const u32x4_t f =
            *reinterpret_cast<const u32x4_t*>(lw + 4096u * p + skinny_off(r, 4u * h + c));
        const i32x8_t v{(int32_t)f.x, (int32_t)f.y, (int32_t)f.z, (int32_t)f.w, 0, 0, 0, 0};
        if (p < MT) va[p] = v;
        else vb[p - MT] = v;
      }
#pragma unroll
      for (int ti = 0; ti < MT; ++ti)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[ti][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              va[ti], vb[j], acc[ti][j], 4, 4, 0,
              (int32_t)(((t.s[ti] & keep) >> (8 * c)) & 0xFFu), 0,
              (int32_t)(((t.s[MT + j] & keep) >> (8 * c)) & 0xFFu));
    }
  };
  SkinnyStep<MT, NT> t[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) load(j, t[j]);
  int32_t i = 0;
  for (; i + kSets - 1 < cnt; i += kSets) {
#pragma unroll
    for (int j = 0; j < kSets; ++j) {
      mma(i + j, t[j]);
      load(i + j + kSets, t[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kSets - 1; ++j)
    if (i + j < cnt) mma(i + j, t[j]);

  // Partial tiles to LDS, four accumulator elements (one row group) per
  // 16-byte slot, lanes contiguous; then wave w adds up the items (tile, row
  // group) w, w + 8, ... over the waves in order 0..7 (deterministic) and
  // writes them. Lane (n, h) of a tile holds column n, rows 8 (e / 4) + 4 h +
  // e % 4.
  constexpr int kT = MT * NT;
  __syncthreads();  // every wave is done with its operand buffers
  f32x4_t* part = reinterpret_cast<f32x4_t*>(smem);  // [kSkinnyWaves][kT][4][64]
#pragma unroll
  for (int ti = 0; ti < MT; ++ti)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part[64 * ((w * kT + ti * NT + j) * 4 + q) + lane] =
            f32x4_t{acc[ti][j][4 * q], acc[ti][j][4 * q + 1], acc[ti][j][4 * q + 2],
                    acc[ti][j][4 * q + 3]};
  __syncthreads();
  for (int item = w; item < kT * 4; item += kSkinnyWaves) {
    f32x4_t sum = part[64 * item + lane];
#pragma unroll
    for (int v = 1; v < kSkinnyWaves; ++v) {
      const f32x4_t p = part[64 * (v * kT * 4 + item) + lane];
      sum.x += p.x;
      sum.y += p.y;
      sum.z += p.z;
      sum.w += p.w;
    }
    const int32_t tq = item / 4, q = item % 4;
    const int32_t col = n0 + 32 * (tq % NT) + (int32_t)r;
    const int32_t row0 = m0 + 32 * (tq / NT) + 8 * q + 4 * (int32_t)h;
    if (col >= g.n) continue;
    const float vals[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int32_t row = row0 + e;
      if (row >= g.m) continue;
      if constexpr (kBf16Out) {
        const uint32_t pk = pack_bf16x2(vals[e], 0.0f);
        static_cast<uint16_t*>(g.c)[(int64_t)row * g.ld_c + col] = (uint16_t)(pk & 0xFFFFu);
      } else {
        static_cast<float*>(g.c)[(int64_t)row * g.ld_c + col] = vals[e];
      }
    }
  }
}

template <int MT, int NT, int kSets>
void launch_skinny(const GemmArgs& g, bool bf16_out, hipStream_t st) {
  const unsigned grid =
      skinny_grid((g.n + 32 * NT - 1) / (32 * NT), (g.m + 32 * MT - 1) / (32 * MT));
  if (bf16_out)
    hipLaunchKernelGGL((mx_gemm_skinny_kernel<MT, NT, kSets, true>), dim3(grid),
                       dim3(64 * kSkinnyWaves), 0, st, g);
  else
    hipLaunchKernelGGL((mx_gemm_skinny_kernel<MT, NT, kSets, false>), dim3(grid),
                       dim3(64 * kSkinnyWaves), 0, st, g);
}

template <int WM, int WN, int VM, int VN, int KB, int kSets>
void launch_tiles(const GemmArgs& g, bool bf16_out, hipStream_t st) {
  constexpr int BM = 32 * WM * VM, BN = 32 * WN * VN;
  const int64_t tiles = (((int64_t)g.m + BM - 1) / BM) * (((int64_t)g.n + BN - 1) / BN);
  if (bf16_out)
    hipLaunchKernelGGL((mx_gemm_kernel<WM, WN, VM, VN, KB, kSets, true>), dim3((unsigned)tiles),
                       dim3(64 * VM * VN), 0, st, g);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<WM, WN, VM, VN, KB, kSets, false>), dim3((unsigned)tiles),
                       dim3(64 * VM * VN), 0, st, g);
}

}  // namespace

void launch_mx_gemm(int64_t m, int64_t n, int64_t k, const void* a, int64_t ld_a, const void* sa,
                    int64_t ld_sa, const void* b, int64_t ld_b, const void* sb, int64_t ld_sb,
                    void* c, int64_t ld_c, bool bf16_out, bool sg_a, bool sg_b,
                    hipStream_t st) {
  GemmArgs g{static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(sa),
             static_cast<const uint8_t*>(b), static_cast<const uint8_t*>(sb), c,
             ld_a, ld_sa, ld_b, ld_sb, ld_c, (int32_t)m, (int32_t)n, (int32_t)k, sg_a, sg_b};
  // split-K tiles: two super-steps in flight per wave for 1 x 1 (7.6 us at
  // 16 x 8192 x 8192 against 9.8 with four), one for the wider tiles (their
  // larger steps already fill the caches' queues; two measured no faster)
  const SkinnyShape sh = skinny_shape(m, n, device_info().cus, kSkinnyMaxM, 8);
  if (sh.mt == 1 && sh.nt == 1) return launch_skinny<1, 1, 2>(g, bf16_out, st);
  if (sh.mt == 1 && sh.nt == 2) return launch_skinny<1, 2, 1>(g, bf16_out, st);
  if (sh.mt == 2 && sh.nt == 2) return launch_skinny<2, 2, 1>(g, bf16_out, st);
  // large products: 256 x 256 tiles halve the operand traffic per flop;
  // smaller ones keep 128 x 128 for more work-groups
  // 256 x 256: eight waves (2 x 4) of 4 x 2 MFMA tiles, two per SIMD, so one
  // wave's MFMAs overlap the other's LDS reads and barrier (the accumulators
  // take half the register file). Measured against four waves of 4 x 4
  // tiles (one per SIMD, accumulators in AGPRs): 4-20% faster on the layer
  // shapes, bit-identical results. Stages of 256 K (whole 128-byte lines of
  // each row; 136 KB of LDS), the next stage in registers while one is
  // multiplied: up to 8% faster again than 128-K stages with two in flight.
  // Loading the stages straight into LDS (buffer loads with the LDS as
  // destination, four 128-K stages in flight, one barrier per stage or per
  // two) gave the same results 20-40% slower on the layer shapes.
  if (m >= 2048 && n >= 2048)
    launch_tiles<4, 2, 2, 4, 256, 1>(g, bf16_out, st);
  else
    launch_tiles<2, 2, 2, 2, 128, 3>(g, bf16_out, st);
}

}  // namespace fp4
