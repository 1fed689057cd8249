// launch.hpp -- internal interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

// Largest row length that the forward permuting kernels stage in LDS (their
// gather offsets are 16-bit byte offsets into the row), and that the inverse
// permutation and the Givens-layer kernels stage (row + indices, 4 bytes per
// column).
constexpr int64_t kMaxPermCols = 32768;
constexpr int64_t kMaxUnpermCols = 16384;
// Work-groups of the row-at-a-time (LDS-staged) kernels.
#ifndef FP4_PERM_GRID
#define FP4_PERM_GRID 1024
#endif
constexpr int kPermGrid = FP4_PERM_GRID;

// Compute units and LDS bytes per CU of the current device.
struct DeviceInfo {
  int cus, lds;
};
DeviceInfo device_info();

struct Shape {
  int64_t rows, cols;
  int64_t ld_x;  // bf16 input (or output, for dequantize) row stride, elements
  int64_t ld_c;  // code row stride, bytes
  int64_t ld_s;  // scale row stride, bytes (GEMM order: 32-row group stride)
  bool s_gemm = false;  // MXFP4 scale bytes in the GEMM order (FP4_FLAG_SCALES_GEMM)
};

// MXFP4, or MXINT4 with mxint.
void launch_mx_quant(const Shape& s, bool floor_rule, bool mxint, const void* x, void* codes,
                     void* scales, hipStream_t st);
// Writes s_t; uses the code buffer as scratch for per-work-group partial maxima.
// top: 2688 (E4M3 scales) or 180 (E3M3 scales of RaZeR for weights).
void launch_nv_tensor_scale(const Shape& s, const void* x, void* codes, float top, float* ts,
                            hipStream_t st);
// s_t from nparts amax partials, partial i in the code slot of chunk i (row-major
// chunks of 8 elements, 4 code bytes each).
void launch_nv_scale_from_partials(const Shape& s, void* codes, uint32_t nparts, float* ts,
                                   hipStream_t st);
// mode: 0 plain, 1 RaZeR, 2 RaZeR for weights (E3M3 scale, four specials).
void launch_nv_quant(const Shape& s, int mode, const void* x, void* codes, void* scales,
                     const float* ts, hipStream_t st);
void launch_dequant(const Shape& s, int format, int mode, const void* codes, const void* scales,
                    const float* ts, void* out, hipStream_t st);
// MXFP4, or MXINT4 with mxint.
void launch_mx_rotate_quant(const Shape& s, const int32_t* perm, int hadamard, bool floor_rule,
                            bool mxint, const void* x, void* codes, void* scales, float* rot,
                            int64_t ld_rot, hipStream_t st);
// NVFP4 (block 16) after the two-level rotation with the 16-point Hadamard;
// with !scale_given, s_t is computed from the rotated tensor first (the code
// buffer holds the amax partials meanwhile). Requires cols % 32 == 0.
void launch_nv_rotate_quant(const Shape& s, const int32_t* perm, int hadamard, bool razer,
                            bool scale_given, const void* x, void* codes, void* scales,
                            float* ts, float* rot, int64_t ld_rot, hipStream_t st);
void launch_mx_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard, bool mxint,
                                const void* codes, const void* scales, void* out, hipStream_t st);
// NVFP4 decode followed by the inverse rotation (16-point Hadamard, then the
// inverse permutation). Requires cols % 32 == 0.
void launch_nv_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard, bool razer,
                                const void* codes, const void* scales, const float* ts, void* out,
                                hipStream_t st);
// C = A B^T, MXFP4 operands (codes [rows, K/2], E8M0 scales [rows, K/32], or
// in the GEMM order with sg_a / sg_b); fp32 or bf16 output.
void launch_mx_gemm(int64_t m, int64_t n, int64_t k, const void* a, int64_t ld_a, const void* sa,
                    int64_t ld_sa, const void* b, int64_t ld_b, const void* sb, int64_t ld_sb,
                    void* c, int64_t ld_c, bool bf16_out, bool sg_a, bool sg_b, hipStream_t st);
// C = ta tb (A B^T), NVFP4 operands (codes [rows, K/2], E4M3 scales
// [rows, K/16], RaZeR per operand), decoded exactly to bf16 for the MFMA.
// mode_a: 0 plain or 1 RaZeR; mode_b: 0, 1 or 2 (RaZeR for weights).
void launch_nv_gemm(int64_t m, int64_t n, int64_t k, const void* a, int64_t ld_a, const void* sa,
                    int64_t ld_sa, const float* ta, int mode_a, const void* b, int64_t ld_b,
                    const void* sb, int64_t ld_sb, const float* tb, int mode_b, void* c,
                    int64_t ld_c, bool bf16_out, hipStream_t st);
// MXFP4 after the permutation and a learned 32x32 block matrix (rmat, device,
// row-major fp32) in place of the Hadamard; and the inverse on decode
// (rmat^T, then the inverse permutation). perm must be given.
void launch_mx_matrix_rotate_quant(const Shape& s, const int32_t* perm, const float* rmat,
                                   const void* x, void* codes, void* scales, float* rot,
                                   int64_t ld_rot, hipStream_t st);
void launch_mx_matrix_dequant_unrotate(const Shape& s, const int32_t* perm, const float* rmat,
                                       const void* codes, const void* scales, void* out,
                                       hipStream_t st);
void launch_channel_energy(int64_t rows, int64_t cols, int64_t ld_x, const void* x, float* energy,
                           hipStream_t st);

// Rows of bf16: permutation (perm may be NULL), then n_layers layers of
// disjoint Givens rotations (layer L = rotations layer_start[L] ..
// layer_start[L + 1] - 1), in fp32, rounded to bf16 once. out may be x.
void launch_givens_rows(int64_t rows, int64_t cols, const void* x, int64_t ld_x,
                        const int32_t* perm, const int32_t* pairs, const float* cs,
                        const int32_t* layer_start, int n_layers, int n_rot, void* out,
                        int64_t ld_out, hipStream_t st);

}  // namespace fp4
