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
// Tiling: a work-group of four waves computes a 128 x 128 tile of C; wave
// (wm, wn) owns the 64 x 64 quarter (wm, wn) as 2 x 2 MFMA tiles. K advances
// 128 elements per stage: the work-group copies the stage's 128 rows x 64
// code bytes of A and of B, and their 4 scale bytes per row, into one of two
// LDS buffers (rows padded to 80 bytes so the 16-byte lane reads of 32
// consecutive rows spread over all banks), while the waves multiply out of
// the other. Loads past M, N or K read zeros through buffer-resource range
// checks (code 0 is +0), so any K that is a multiple of 32 works.
#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {

namespace {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128;        // C tile of a work-group
constexpr int kBK = 128;                   // K elements per stage
constexpr int kRowBytes = kBK / 2;         // code bytes per row per stage
constexpr int kLdsRow = kRowBytes + 16;    // padded LDS row
constexpr int kTileBytes = kBM * kLdsRow;  // one operand, one stage

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* sa;
  const uint8_t* b;
  const uint8_t* sb;
  void* c;
  int64_t ld_a, ld_sa, ld_b, ld_sb, ld_c;  // bytes (codes, scales), elements (C)
  int32_t m, n, k;
};

// One operand's share of a stage, in flight in registers: two 16-byte code
// chunks per lane, and (lanes 0..127 for A, 128..255 for B) one row's four
// scale bytes.
struct StageRegs {
  u32x4_t a[2], b[2];
  uint32_t s;
};

struct OperandRsrc {
  rsrc_t a, sa, b, sb;
};

__device__ __forceinline__ void load_stage(const OperandRsrc& q, const GemmArgs& g, int32_t k0,
                                           StageRegs& r) {
  const uint32_t t = threadIdx.x;
  const uint32_t kb0 = (uint32_t)k0 / 2u, kbytes = (uint32_t)g.k / 2u;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t chunk = t + 256u * i, row = chunk >> 2, col = 16u * (chunk & 3u);
    const bool in_k = kb0 + col < kbytes;
    r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(
        q.a, in_k ? row * (uint32_t)g.ld_a + kb0 + col : kOob, 0, 0);
    r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(
        q.b, in_k ? row * (uint32_t)g.ld_b + kb0 + col : kOob, 0, 0);
  }
  // scales: waves 0-1 read the rows of A, waves 2-3 those of B (lane t reads
  // row t % 128); the choice is uniform per wave, so the resource stays scalar
  const bool is_a = __builtin_amdgcn_readfirstlane(t >> 6) < 2u;
  const rsrc_t rs = is_a ? q.sa : q.sb;
  const uint32_t row = t & 127u, blk0 = (uint32_t)k0 / 32u, nblk = (uint32_t)g.k / 32u;
  const uint32_t base = row * (uint32_t)(is_a ? g.ld_sa : g.ld_sb);
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t off = blk0 + j < nblk ? base + blk0 + j : kOob;
    s |= ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, 0) & 0xFFu) << (8 * j);
  }
  r.s = s;
}

__device__ __forceinline__ void store_stage(uint8_t* lds_a, uint8_t* lds_b, uint32_t* lds_s,
                                            const StageRegs& r) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t chunk = t + 256u * i, row = chunk >> 2, col = 16u * (chunk & 3u);
    *reinterpret_cast<u32x4_t*>(lds_a + row * kLdsRow + col) = r.a[i];
    *reinterpret_cast<u32x4_t*>(lds_b + row * kLdsRow + col) = r.b[i];
  }
  lds_s[t] = r.s;  // A rows 0..127, then B rows 0..127
}

template <bool kBf16Out>
__global__ __launch_bounds__(256, 2) void mx_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kTileBytes];
  __shared__ uint32_t lds_s[2][256];

  const int32_t tiles_n = (g.n + kBN - 1) / kBN;
  const int32_t bm = blockIdx.x / tiles_n, bn = blockIdx.x - bm * tiles_n;
  const int32_t m0 = bm * kBM, n0 = bn * kBN;
  const int32_t rows_a = min(kBM, g.m - m0), rows_b = min(kBN, g.n - n0);
  OperandRsrc q;
  q.a = make_rsrc(g.a + (int64_t)m0 * g.ld_a, (uint32_t)(rows_a * g.ld_a));
  q.b = make_rsrc(g.b + (int64_t)n0 * g.ld_b, (uint32_t)(rows_b * g.ld_b));
  q.sa = make_rsrc(g.sa + (int64_t)m0 * g.ld_sa, (uint32_t)(rows_a * g.ld_sa));
  q.sb = make_rsrc(g.sb + (int64_t)n0 * g.ld_sb, (uint32_t)(rows_b * g.ld_sb));

  const uint32_t lane = threadIdx.x & 63u, r = lane & 31u, h = lane >> 5;
  const uint32_t w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1u;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int32_t stages = (g.k + kBK - 1) / kBK;
  StageRegs st;
  load_stage(q, g, 0, st);
  store_stage(lds_a[0], lds_b[0], lds_s[0], st);
  __syncthreads();

  for (int32_t s = 0; s < stages; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < stages;
    if (more) load_stage(q, g, (s + 1) * kBK, st);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // two 64-element K steps per stage
      i32x8_t fa[2], fb[2];
      int32_t sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ra = 64u * wm + 32u * i + r, rb = 64u * wn + 32u * i + r;
        const u32x4_t va =
            *reinterpret_cast<const u32x4_t*>(lds_a[buf] + ra * kLdsRow + 32u * ks + 16u * h);
        const u32x4_t vb =
            *reinterpret_cast<const u32x4_t*>(lds_b[buf] + rb * kLdsRow + 32u * ks + 16u * h);
        fa[i] = i32x8_t{(int32_t)va.x, (int32_t)va.y, (int32_t)va.z, (int32_t)va.w, 0, 0, 0, 0};
        fb[i] = i32x8_t{(int32_t)vb.x, (int32_t)vb.y, (int32_t)vb.z, (int32_t)vb.w, 0, 0, 0, 0};
        sa[i] = (int32_t)((lds_s[buf][ra] >> (8u * (2u * ks + h))) & 0xFFu);
        sb[i] = (int32_t)((lds_s[buf][128u + rb] >> (8u * (2u * ks + h))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    }
    if (more) store_stage(lds_a[buf ^ 1], lds_b[buf ^ 1], lds_s[buf ^ 1], st);
    __syncthreads();
  }

  // epilogue: lane (n, h) of tile (i, j) holds column n, rows 8 (e / 4) + 4 h + e % 4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int32_t col = n0 + 64 * (int32_t)wn + 32 * j + (int32_t)r;
      if (col >= g.n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t row = m0 + 64 * (int32_t)wm + 32 * i + 8 * (e / 4) + 4 * (int32_t)h + e % 4;
        if (row >= g.m) continue;
        if constexpr (kBf16Out) {
          const uint32_t p = pack_bf16x2(acc[i][j][e], 0.0f);
          static_cast<uint16_t*>(g.c)[(int64_t)row * g.ld_c + col] = (uint16_t)(p & 0xFFFFu);
        } else {
          static_cast<float*>(g.c)[(int64_t)row * g.ld_c + col] = acc[i][j][e];
        }
      }
    }
}

}  // namespace

void launch_mx_gemm(int64_t m, int64_t n, int64_t k, const void* a, int64_t ld_a, const void* sa,
                    int64_t ld_sa, const void* b, int64_t ld_b, const void* sb, int64_t ld_sb,
                    void* c, int64_t ld_c, bool bf16_out, hipStream_t st) {
  GemmArgs g{static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(sa),
             static_cast<const uint8_t*>(b), static_cast<const uint8_t*>(sb), c,
             ld_a, ld_sa, ld_b, ld_sb, ld_c, (int32_t)m, (int32_t)n, (int32_t)k};
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  if (bf16_out)
    hipLaunchKernelGGL(mx_gemm_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(mx_gemm_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, st, g);
}

}  // namespace fp4
