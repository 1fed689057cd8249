// gemm_nv.hip -- C = s_a s_b (A B^T) with NVFP4 operands, optionally RaZeR
// (and, for the weights B, RaZeR's weight variant), on the bf16 matrix cores.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping", technical summary sec. 2.3: GEMM kernels that take the
// quantized weights and activations, the special value rebuilt from the
// scale's metadata bit. A is [M, K], B is [N, K], each as fp4_quantize writes
// NVFP4: codes [rows, K/2], E4M3 scale bytes [rows, K/16] (RaZeR: selector in
// bit 7) and an fp32 tensor scale s.
//
// gfx950's block-scaled FP4 matrix instructions take E8M0 scales per 32
// elements; NVFP4's are E4M3 per 16, so they cannot be fed to it. Instead
// each element is decoded exactly: an E2M1 value (or the block's +-5, +-2.5)
// has at most 3 significant bits and an E4M3 or E3M3 scale 4, so value x
// scale has at most 7 and is a bf16, between 2^-10 and 2688. The work-group decodes each stage
// once, on its way into LDS, and the waves run v_mfma_f32_32x32x16_bf16 on the
// decoded tiles (products of bf16 are exact in fp32); the tensor scales
// multiply once in the epilogue. RaZeR needs no second pass: code 0x8 simply
// decodes to the block's special value.
//
// Tiling as in the MXFP4 GEMM: VM x VN waves, a (32 WM VM) x (32 WN VN)
// work-group tile, WM x WN MFMA tiles of 32 x 32 per wave; K advances 64 elements per
// stage (32 code bytes and 4 scale bytes of each row), decoded into one of two
// LDS buffers of bf16 rows (128 bytes per row, 16-byte chunks XOR-swizzled by
// row) while the waves multiply out of the other.
#include <type_traits>

#include "fp4_device.hpp"
#include "launch.hpp"
#include "split_k.hpp"

namespace fp4 {

namespace {

typedef __bf16 nbf16x8_t __attribute__((ext_vector_type(8)));
typedef float nf32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;         // K elements per stage
constexpr int kRowB = 2 * kBK;  // bf16 bytes per row per stage in LDS

// LDS byte offset of 16-byte chunk c (0..7, eight elements) of row r: slot
// c ^ ((r / 2) % 8). gfx950's LDS has 64 four-byte banks, two 128-byte rows
// per bank cycle, so the lane reads of one chunk of 16 consecutive rows fall
// on 16 different 16-byte bank groups (both row parities, eight slots).
__device__ __forceinline__ uint32_t nv_lds_off(uint32_t r, uint32_t c) {
  return r * kRowB + 16u * (c ^ ((r >> 1) & 7u));
}

struct NvGemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  const float* ta;
  const float* tb;
  void* c;
  int64_t ld_a, ld_sa, ld_b, ld_sb, ld_c;
  int32_t m, n, k;
};

struct NvRsrc {
  rsrc_t a, sa, b, sb;
};

// One operand chunk: 16 code bytes (32 elements, two NVFP4 blocks) and the
// blocks' two scale bytes; lane t of the kT-thread work-group takes chunk
// t + kT i of the stage, i.e. row (t + kT i) / 2, half (t + kT i) % 2 of its
// 64 elements.
template <int kRows, int kT>
struct NvOperand {
  static constexpr int kChunks = kRows * 2 / kT;
  static_assert(kChunks * kT == kRows * 2, "the stage divides evenly over the lanes");
  u32x4_t w[kChunks];
  uint32_t s[kChunks];

  __device__ __forceinline__ void load(rsrc_t q, rsrc_t qs, int64_t ld, int64_t ld_s, int32_t k0,
                                       int32_t k) {
    const uint32_t t = threadIdx.x, kb0 = (uint32_t)k0 / 2u, kbytes = (uint32_t)k / 2u;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk >> 1, half = chunk & 1u;
      const bool in_k = kb0 + 16u * half < kbytes;  // k is a multiple of 32: whole chunks
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(
          q, in_k ? row * (uint32_t)ld + kb0 + 16u * half : kOob, 0, 0);
      s[i] = __builtin_amdgcn_raw_buffer_load_b16(
          qs, in_k ? row * (uint32_t)ld_s + (uint32_t)k0 / 16u + 2u * half : kOob, 0, 0);
    }
  }

  // decode to bf16 and write the chunk's four 16-byte LDS chunks; kMode 0
  // plain, 1 RaZeR (E4M3 scale, +-5), 2 RaZeR for weights (E3M3 scale,
  // {+5, -5, +2.5, -2.5})
  template <int kMode>
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const uint32_t t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t chunk = t + (uint32_t)kT * i, row = chunk >> 1, half = chunk & 1u;
      const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // eight elements: block j / 2 of the chunk
        const uint32_t sbyte = (s[i] >> (8 * (j / 2))) & 0xFFu;
        const float sc =
            kMode == 2 ? e3m3_decode(sbyte) : e4m3_decode(kMode ? (sbyte & 0x7Fu) : sbyte);
        const float special =
            kMode == 2 ? weight_special(sbyte) : (sbyte & 0x80u) ? -5.0f : 5.0f;
        float v[8];
#define FP4_NV_DEC2(sel)                                                              \
  {                                                                                   \
    const float2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[j], 1.0f, sel);    \
    v[2 * sel] = p.x;                                                                 \
    v[2 * sel + 1] = p.y;                                                             \
  }
        FP4_NV_DEC2(0) FP4_NV_DEC2(1) FP4_NV_DEC2(2) FP4_NV_DEC2(3)
#undef FP4_NV_DEC2
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // RaZeR: code 0x8, the only code that decodes to -0.0, is the special
          if (kMode && __float_as_uint(v[e]) == 0x80000000u) v[e] = special;
          v[e] *= sc;  // exact: at most 7 significant bits
        }
        const u32x4_t o{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
        *reinterpret_cast<u32x4_t*>(lds + nv_lds_off(row, 4u * half + (uint32_t)j)) = o;
      }
    }
  }
};

template <int WM, int WN, int VM, int VN, int kModeA, int kModeB, bool kBf16Out>
__global__ __launch_bounds__(64 * VM * VN) void nv_gemm_kernel(NvGemmArgs g) {
  constexpr int BM = 32 * WM * VM, BN = 32 * WN * VN, kT = 64 * VM * VN;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kRowB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kRowB];

  const int32_t tiles_n = (g.n + BN - 1) / BN;
  const int32_t bm = blockIdx.x / tiles_n, bn = blockIdx.x - bm * tiles_n;
  const int32_t m0 = bm * BM, n0 = bn * BN;
  const int32_t rows_a = min(BM, g.m - m0), rows_b = min(BN, g.n - n0);
  NvRsrc q;
  q.a = make_rsrc(g.a + (int64_t)m0 * g.ld_a, (uint32_t)(rows_a * g.ld_a));
  q.b = make_rsrc(g.b + (int64_t)n0 * g.ld_b, (uint32_t)(rows_b * g.ld_b));
  q.sa = make_rsrc(g.sa + (int64_t)m0 * g.ld_sa, (uint32_t)(rows_a * g.ld_sa));
  q.sb = make_rsrc(g.sb + (int64_t)n0 * g.ld_sb, (uint32_t)(rows_b * g.ld_sb));

  const uint32_t lane = threadIdx.x & 63u, r = lane & 31u, h = lane >> 5;
  const uint32_t w = threadIdx.x >> 6, wm = w / VN, wn = w % VN;

  nf32x16_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // multiply out the stage in LDS buffer buf: four 16-element K steps; lane
  // (r, h) supplies elements 8h .. 8h + 7 of the step (chunk 2 ks + h)
  auto mma = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t c = 2u * ks + h;
      nbf16x8_t fa[WM], fb[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        fa[i] = *reinterpret_cast<const nbf16x8_t*>(
            lds_a[buf] + nv_lds_off(32u * WM * wm + 32u * i + r, c));
#pragma unroll
      for (int j = 0; j < WN; ++j)
        fb[j] = *reinterpret_cast<const nbf16x8_t*>(
            lds_b[buf] + nv_lds_off(32u * WN * wn + 32u * j + r, c));
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // two stages of loads in flight, as in the MXFP4 GEMM; loads past K read
  // zeros (code 0 decodes to +0 whatever the scale byte)
  const int32_t stages = (g.k + kBK - 1) / kBK;
  NvOperand<BM, kT> a0, a1;
  NvOperand<BN, kT> b0, b1;
  a0.load(q.a, q.sa, g.ld_a, g.ld_sa, 0, g.k);
  b0.load(q.b, q.sb, g.ld_b, g.ld_sb, 0, g.k);
  a1.load(q.a, q.sa, g.ld_a, g.ld_sa, kBK, g.k);
  b1.load(q.b, q.sb, g.ld_b, g.ld_sb, kBK, g.k);
  a0.template store<kModeA>(lds_a[0]);
  b0.template store<kModeB>(lds_b[0]);
  __syncthreads();
  int32_t s = 0;
  for (; s + 1 < stages; s += 2) {
    a0.load(q.a, q.sa, g.ld_a, g.ld_sa, (s + 2) * kBK, g.k);
    b0.load(q.b, q.sb, g.ld_b, g.ld_sb, (s + 2) * kBK, g.k);
    mma(0);
    a1.template store<kModeA>(lds_a[1]);
    b1.template store<kModeB>(lds_b[1]);
    __syncthreads();
    a1.load(q.a, q.sa, g.ld_a, g.ld_sa, (s + 3) * kBK, g.k);
    b1.load(q.b, q.sb, g.ld_b, g.ld_sb, (s + 3) * kBK, g.k);
    mma(1);
    a0.template store<kModeA>(lds_a[0]);
    b0.template store<kModeB>(lds_b[0]);
    __syncthreads();
  }
  if (s < stages) mma(0);

  const float ts = *g.ta * *g.tb;
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
        const float v = acc[i][j][e] * ts;
        if constexpr (kBf16Out) {
          const uint32_t p = pack_bf16x2(v, 0.0f);
          static_cast<uint16_t*>(g.c)[(int64_t)row * g.ld_c + col] = (uint16_t)(p & 0xFFFFu);
        } else {
          static_cast<float*>(g.c)[(int64_t)row * g.ld_c + col] = v;
        }
      }
    }
}

// Split-K products, as the MXFP4 split-K kernel: a work-group of eight
// waves computes MT x NT tiles of 32 x 32 of C, wave w takes the 256-K
// super-steps w, w + 8, ...; each operand piece (32 rows x 128 code bytes)
// is loaded with eight consecutive lanes per 128-byte row piece and passed
// through the wave's XOR-swizzled LDS buffer, so that lane (r, h) holds the
// 128 elements 128 h .. 128 h + 127 of row r of the step (16 dwords) and
// their 8 scale bytes. MFMA q (0..15) of a tile pair takes dword q, eight
// elements, from both operands in both lane halves (the same K values of A
// and B in every lane), decoded exactly to bf16 with the block scale of that
// dword (byte q / 2); each decoded dword serves every tile pair it belongs
// to. Partial tiles are added in LDS in wave order.
constexpr int kNvSkinnyWaves = 8;
constexpr int kNvSkinnyMaxM = 256;  // larger m always takes the 128 x 128 or 256 x 256 tiles

template <int MT, int NT>
struct NvSkinnyStep {
  u32x4_t v[MT + NT][4];  // row 8 c + lane / 8 of the piece, 16-byte chunk lane % 8
  uint32_t s[MT + NT][2];  // row lane % 32 of the piece: scale bytes 8 h .. 8 h + 7 of the step
};

__device__ __forceinline__ uint32_t nv_skinny_off(uint32_t r, uint32_t j) {
  return 128u * r + 16u * (j ^ ((r >> 1) & 7u));  // as nv_lds_off
}

__device__ __forceinline__ void nv_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight E2M1 codes of one dword, decoded with scale byte sbyte (kMode as for
// NvOperand::store), as four bf16 pairs.
template <int kMode>
__device__ __forceinline__ nbf16x8_t nv_decode8(uint32_t wd, uint32_t sbyte) {
  const float sc = kMode == 2 ? e3m3_decode(sbyte) : e4m3_decode(kMode ? (sbyte & 0x7Fu) : sbyte);
  const float special = kMode == 2 ? weight_special(sbyte) : (sbyte & 0x80u) ? -5.0f : 5.0f;
  float v[8];
#define FP4_NV_DEC2(sel)                                                          \
  {                                                                               \
    const float2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, sel);   \
    v[2 * sel] = p.x;                                                             \
    v[2 * sel + 1] = p.y;                                                         \
  }
  FP4_NV_DEC2(0) FP4_NV_DEC2(1) FP4_NV_DEC2(2) FP4_NV_DEC2(3)
#undef FP4_NV_DEC2
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (kMode && __float_as_uint(v[e]) == 0x80000000u) v[e] = special;
    v[e] *= sc;  // exact: at most 7 significant bits
  }
  const u32x4_t o{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
  return __builtin_bit_cast(nbf16x8_t, o);
}

template <int MT, int NT, int kSets, int kModeA, int kModeB, bool kBf16Out>
__global__ __launch_bounds__(64 * kNvSkinnyWaves) void nv_gemm_skinny_kernel(NvGemmArgs g) {
  constexpr int kP = MT + NT, kT = MT * NT;
  constexpr int kOps = kNvSkinnyWaves * kP * 4096;   // operand pieces
  constexpr int kRed = kNvSkinnyWaves * 64 * kT * 64;  // partial tiles
  __shared__ __attribute__((aligned(16))) uint8_t smem[kOps > kRed ? kOps : kRed];
  const SkinnyTile tile = skinny_tile(blockIdx.x, (g.m + 32 * MT - 1) / (32 * MT));
  const int32_t n0 = tile.x * 32 * NT, m0 = tile.y * 32 * MT;
  if (n0 >= g.n) return;  // padding of the grid to whole XCD rounds
  const int32_t rows_a = min(32 * MT, g.m - m0), rows_b = min(32 * NT, g.n - n0);
  const rsrc_t ra = make_rsrc(g.a + (int64_t)m0 * g.ld_a, (uint32_t)(rows_a * g.ld_a));
  const rsrc_t rsa = make_rsrc(g.sa + (int64_t)m0 * g.ld_sa, (uint32_t)(rows_a * g.ld_sa));
  const rsrc_t rb = make_rsrc(g.b + (int64_t)n0 * g.ld_b, (uint32_t)(rows_b * g.ld_b));
  const rsrc_t rsb = make_rsrc(g.sb + (int64_t)n0 * g.ld_sb, (uint32_t)(rows_b * g.ld_sb));
  const uint32_t lane = threadIdx.x & 63u, r = lane & 31u, h = lane >> 5;
  const int32_t w = (int32_t)(threadIdx.x >> 6);
  uint8_t* const lw = smem + kP * 4096u * (uint32_t)w;
  const uint32_t kbytes = (uint32_t)g.k / 2u, nblk = (uint32_t)g.k / 16u;
  const int32_t steps = (g.k + 255) / 256;
  const int32_t cnt = steps > w ? (steps - w + kNvSkinnyWaves - 1) / kNvSkinnyWaves : 0;

  // loads of the wave's i-th super-step (past the list or past K: offsets out
  // of range, which read zeros without touching memory; code 0 decodes to +0
  // whatever the scale byte)
  auto load = [&](int32_t i, NvSkinnyStep<MT, NT>& t) __attribute__((always_inline)) {
    const int32_t s = w + kNvSkinnyWaves * i;
    const bool live = i < cnt;
    const uint32_t off = 128u * (uint32_t)s + 16u * (lane & 7u);
    const bool ok = live && off < kbytes;
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
      // scale bytes in 16-bit pieces (rows are 2-byte aligned); an even block
      // index below nblk (even, as k % 32 == 0) covers both of its blocks
      const uint32_t lds_ = (uint32_t)(pa ? g.ld_sa : g.ld_sb);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t blk = 16u * (uint32_t)s + 8u * h + 2u * q;
        const bool oks = live && blk < nblk;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(
            pa ? rsa : rsb, oks ? (base + r) * lds_ + blk : kOob, 0, 0);
        if (q % 2 == 0) t.s[p][q / 2] = v;
        else t.s[p][q / 2] |= v << 16;
      }
    }
  };

  nf32x16_t acc[MT][NT];
#pragma unroll
  for (int ti = 0; ti < MT; ++ti)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ti][j][e] = 0.0f;
  auto mma = [&](const NvSkinnyStep<MT, NT>& t) __attribute__((always_inline)) {
    nv_wave_sync();  // the previous step's reads of the buffer are done
#pragma unroll
    for (int p = 0; p < kP; ++p)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<u32x4_t*>(lw + 4096u * p +
                                    nv_skinny_off(8u * c + (lane >> 3), lane & 7u)) = t.v[p][c];
    nv_wave_sync();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4_t f[kP];
#pragma unroll
      for (int p = 0; p < kP; ++p)
        f[p] = *reinterpret_cast<const u32x4_t*>(lw + 4096u * p + nv_skinny_off(r, 4u * h + c));
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int q = 4 * c + d;
        nbf16x8_t da[MT], db[NT];
#pragma unroll
        for (int ti = 0; ti < MT; ++ti)
          da[ti] = nv_decode8<kModeA>(f[ti][d], (t.s[ti][q / 8] >> (8 * ((q / 2) % 4))) & 0xFFu);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          db[j] = nv_decode8<kModeB>(f[MT + j][d],
                                     (t.s[MT + j][q / 8] >> (8 * ((q / 2) % 4))) & 0xFFu);
#pragma unroll
        for (int ti = 0; ti < MT; ++ti)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[ti][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ti], db[j], acc[ti][j], 0, 0, 0);
      }
    }
  };
  NvSkinnyStep<MT, NT> t[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) load(j, t[j]);
  int32_t i = 0;
  for (; i + kSets - 1 < cnt; i += kSets) {
#pragma unroll
    for (int j = 0; j < kSets; ++j) {
      mma(t[j]);
      load(i + j + kSets, t[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < kSets - 1; ++j)
    if (i + j < cnt) mma(t[j]);

  // Partial tiles to LDS, four accumulator elements (one row group) per
  // 16-byte slot, lanes contiguous; then wave w adds up the items (tile, row
  // group) w, w + 8, ... over the waves in order 0..7 (deterministic), scales
  // them by the two tensor scales and writes them. Lane (n, h) of a tile
  // holds column n, rows 8 (e / 4) + 4 h + e % 4.
  __syncthreads();  // every wave is done with its operand buffers
  f32x4_t* part = reinterpret_cast<f32x4_t*>(smem);  // [kNvSkinnyWaves][kT][4][64]
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
  const float ts = *g.ta * *g.tb;
  for (int item = w; item < kT * 4; item += kNvSkinnyWaves) {
    f32x4_t sum = part[64 * item + lane];
#pragma unroll
    for (int v = 1; v < kNvSkinnyWaves; ++v) {
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
    const float vals[4] = {sum.x * ts, sum.y * ts, sum.z * ts, sum.w * ts};
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

template <int MT, int NT, int kSets, int kMa, int kMb>
void nv_launch_skinny(const NvGemmArgs& g, bool bf16_out, hipStream_t st) {
  const unsigned grid =
      skinny_grid((g.n + 32 * NT - 1) / (32 * NT), (g.m + 32 * MT - 1) / (32 * MT));
  if (bf16_out)
    hipLaunchKernelGGL((nv_gemm_skinny_kernel<MT, NT, kSets, kMa, kMb, true>), dim3(grid),
                       dim3(64 * kNvSkinnyWaves), 0, st, g);
  else
    hipLaunchKernelGGL((nv_gemm_skinny_kernel<MT, NT, kSets, kMa, kMb, false>), dim3(grid),
                       dim3(64 * kNvSkinnyWaves), 0, st, g);
}

template <int WM, int WN, int VM, int VN, int kMa, int kMb>
void nv_launch(const NvGemmArgs& g, bool bf16_out, hipStream_t st) {
  constexpr int BM = 32 * WM * VM, BN = 32 * WN * VN;
  const int64_t tiles = (((int64_t)g.m + BM - 1) / BM) * (((int64_t)g.n + BN - 1) / BN);
  if (bf16_out)
    hipLaunchKernelGGL((nv_gemm_kernel<WM, WN, VM, VN, kMa, kMb, true>), dim3((unsigned)tiles),
                       dim3(64 * VM * VN), 0, st, g);
  else
    hipLaunchKernelGGL((nv_gemm_kernel<WM, WN, VM, VN, kMa, kMb, false>), dim3((unsigned)tiles),
                       dim3(64 * VM * VN), 0, st, g);
}

template <int kMa, int kMb>
void nv_tiles(const NvGemmArgs& g, bool bf16_out, hipStream_t st) {
  const SkinnyShape sh = skinny_shape(g.m, g.n, device_info().cus, kNvSkinnyMaxM, 10);
  if (sh.mt == 1 && sh.nt == 1) return nv_launch_skinny<1, 1, 2, kMa, kMb>(g, bf16_out, st);
  if (sh.mt == 1 && sh.nt == 2) return nv_launch_skinny<1, 2, 1, kMa, kMb>(g, bf16_out, st);
  if (sh.mt == 2 && sh.nt == 2) return nv_launch_skinny<2, 2, 1, kMa, kMb>(g, bf16_out, st);
  // 256 x 256 from eight waves (two per SIMD) of 4 x 2 MFMA tiles: 17-24%
  // faster than four waves of 4 x 4 on the layer shapes, bit-identical
  if (g.m >= 2048 && g.n >= 2048)
    nv_launch<4, 2, 2, 4, kMa, kMb>(g, bf16_out, st);
  else
    nv_launch<2, 2, 2, 2, kMa, kMb>(g, bf16_out, st);
}

template <int kMa>
void nv_modes_b(const NvGemmArgs& g, int mode_b, bool bf16_out, hipStream_t st) {
  if (mode_b == 2) nv_tiles<kMa, 2>(g, bf16_out, st);
  else if (mode_b == 1) nv_tiles<kMa, 1>(g, bf16_out, st);
  else nv_tiles<kMa, 0>(g, bf16_out, st);
}

}  // namespace

void launch_nv_gemm(int64_t m, int64_t n, int64_t k, const void* a, int64_t ld_a, const void* sa,
                    int64_t ld_sa, const float* ta, int mode_a, const void* b, int64_t ld_b,
                    const void* sb, int64_t ld_sb, const float* tb, int mode_b, void* c,
                    int64_t ld_c, bool bf16_out, hipStream_t st) {
  NvGemmArgs g{static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(sa),
               static_cast<const uint8_t*>(b), static_cast<const uint8_t*>(sb), ta, tb, c,
               ld_a, ld_sa, ld_b, ld_sb, ld_c, (int32_t)m, (int32_t)n, (int32_t)k};
  if (mode_a == 1) nv_modes_b<1>(g, mode_b, bf16_out, st);
  else nv_modes_b<0>(g, mode_b, bf16_out, st);
}

}  // namespace fp4
