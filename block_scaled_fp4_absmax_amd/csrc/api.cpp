// api.cpp -- C ABI of libfp4.so: argument checks, then kernel launches on the
// caller's stream. Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include "../../include/fp4.h"
#include "launch.hpp"

using fp4::Shape;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int block_of(int format) { return format == FP4_NVFP4 ? 16 : 32; }

bool known_format(int format) {
  return format == FP4_MXFP4 || format == FP4_NVFP4 || format == FP4_MXINT4;
}

// Stride check of an MXFP4 scale array in the GEMM order (FP4_FLAG_SCALES_GEMM):
// ld is the 32-row group stride, whole 256-byte steps covering `len` elements.
bool gemm_scale_ld_ok(int64_t ld, int64_t len) {
  return ld % 256 == 0 && ld >= 256 * ((len + 255) / 256);
}

// Checks shared by the quantizing entry points.
int check_quant_args(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int format,
                     int block, int mode, uint32_t flags, const void* codes, int64_t ld_codes,
                     const void* scales, int64_t ld_scales, const float* tensor_scale) {
  if (!known_format(format)) return FP4_ERR_UNSUPPORTED;
  if (block != block_of(format)) return FP4_ERR_UNSUPPORTED;
  if (mode != FP4_PLAIN && mode != FP4_RAZER && mode != FP4_RAZER_W) return FP4_ERR_UNSUPPORTED;
  if (mode != FP4_PLAIN && format != FP4_NVFP4) return FP4_ERR_UNSUPPORTED;  // E8M0 has no free bit
  if (flags & ~(FP4_FLAG_TENSOR_SCALE_GIVEN | FP4_FLAG_SCALE_OCP_FLOOR | FP4_FLAG_SCALES_GEMM))
    return FP4_ERR_UNSUPPORTED;
  if ((flags & FP4_FLAG_TENSOR_SCALE_GIVEN) && format != FP4_NVFP4) return FP4_ERR_UNSUPPORTED;
  if ((flags & FP4_FLAG_SCALE_OCP_FLOOR) && format == FP4_NVFP4) return FP4_ERR_UNSUPPORTED;
  const bool s_gemm = (flags & FP4_FLAG_SCALES_GEMM) != 0;
  if (s_gemm && format != FP4_MXFP4) return FP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % block != 0) return FP4_ERR_SHAPE;
  if (ld_x < cols || ld_codes < cols / 2) return FP4_ERR_SHAPE;
  if (s_gemm ? !gemm_scale_ld_ok(ld_scales, cols) : ld_scales < cols / block) return FP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && rows * cols / 8 >= (int64_t)1 << 31) return FP4_ERR_UNSUPPORTED;
  if (format == FP4_NVFP4 && !tensor_scale) return FP4_ERR_NULL;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x || !codes || !scales) return FP4_ERR_NULL;
  if (!aligned(x, 16) || ld_x % 8 != 0) return FP4_ERR_ALIGN;
  if (!aligned(codes, 4) || ld_codes % 4 != 0) return FP4_ERR_ALIGN;
  if (format == FP4_NVFP4 && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace

extern "C" {

int fp4_version(void) { return FP4_VERSION; }

const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_SHAPE: return "invalid shape or row stride";
    case FP4_ERR_ALIGN: return "pointer or row stride not aligned";
    case FP4_ERR_UNSUPPORTED: return "unsupported format, mode, flag, block or size";
    case FP4_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int fp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, int format,
                 int block, int mode, uint32_t flags, void* codes, int64_t ld_codes,
                 void* scales, int64_t ld_scales, float* tensor_scale, void* stream) {
  int rc = check_quant_args(x_bf16, rows, cols, ld_x, format, block, mode, flags, codes, ld_codes,
                            scales, ld_scales, tensor_scale);
  if (rc != FP4_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Shape s{rows, cols, ld_x, ld_codes, ld_scales, (flags & FP4_FLAG_SCALES_GEMM) != 0};
  const bool empty = rows == 0 || cols == 0;
  const bool need_scale = format == FP4_NVFP4 && !(flags & FP4_FLAG_TENSOR_SCALE_GIVEN);
  if (empty && !need_scale) return FP4_OK;  // nothing to enqueue
  (void)hipGetLastError();  // clear a stale error so the status below is this call's
  if (format != FP4_NVFP4) {
    if (!empty)
      fp4::launch_mx_quant(s, (flags & FP4_FLAG_SCALE_OCP_FLOOR) != 0, format == FP4_MXINT4, x_bf16,
                           codes, scales, st);
  } else {
    if (need_scale)
      fp4::launch_nv_tensor_scale(s, x_bf16, codes, mode == FP4_RAZER_W ? 180.0f : 2688.0f,
                                  tensor_scale, st);
    if (!empty) fp4::launch_nv_quant(s, mode, x_bf16, codes, scales, tensor_scale, st);
  }
  return launch_status();
}

int fp4_dequantize(const void* codes, int64_t ld_codes, const void* scales, int64_t ld_scales,
                   const float* tensor_scale, int64_t rows, int64_t cols, int format, int block,
                   int mode, const int32_t* perm, int hadamard, void* out_bf16, int64_t ld_out,
                   void* stream) {
  if (!known_format(format)) return FP4_ERR_UNSUPPORTED;
  if (block != block_of(format)) return FP4_ERR_UNSUPPORTED;
  if (mode != FP4_PLAIN && mode != FP4_RAZER && mode != FP4_RAZER_W) return FP4_ERR_UNSUPPORTED;
  if (mode != FP4_PLAIN && format != FP4_NVFP4) return FP4_ERR_UNSUPPORTED;
  if (hadamard != 0 && hadamard != block) return FP4_ERR_UNSUPPORTED;
  if (mode == FP4_RAZER_W && (hadamard || perm)) return FP4_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || cols % block != 0) return FP4_ERR_SHAPE;
  if ((hadamard || perm) && cols % 32 != 0) return FP4_ERR_SHAPE;  // 32-element segments
  if (ld_out < cols || ld_codes < cols / 2 || ld_scales < cols / block) return FP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && rows * cols / 8 >= (int64_t)1 << 31) return FP4_ERR_UNSUPPORTED;
  if (perm && cols > fp4::kMaxUnpermCols) return FP4_ERR_UNSUPPORTED;
  if (format == FP4_NVFP4 && !tensor_scale) return FP4_ERR_NULL;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales || !out_bf16) return FP4_ERR_NULL;
  if (!aligned(out_bf16, 16) || ld_out % 8 != 0) return FP4_ERR_ALIGN;
  if (!aligned(codes, 4) || ld_codes % 4 != 0) return FP4_ERR_ALIGN;
  if (format == FP4_NVFP4 && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  if (perm && !aligned(perm, 4)) return FP4_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Shape s{rows, cols, ld_out, ld_codes, ld_scales};
  (void)hipGetLastError();
  if ((hadamard || perm) && format != FP4_NVFP4)
    fp4::launch_mx_dequant_unrotate(s, perm, hadamard, format == FP4_MXINT4, codes, scales,
                                    out_bf16, st);
  else if (hadamard || perm)
    fp4::launch_nv_dequant_unrotate(s, perm, hadamard, mode == FP4_RAZER, codes, scales,
                                    tensor_scale, out_bf16, st);
  else
    fp4::launch_dequant(s, format, mode, codes, scales, tensor_scale, out_bf16, st);
  return launch_status();
}

int fp4_rotate_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                        const int32_t* perm, int hadamard, int format, int block, int mode,
                        uint32_t flags, void* codes, int64_t ld_codes, void* scales,
                        int64_t ld_scales, float* tensor_scale, float* rotated_out,
                        int64_t ld_rot, void* stream) {
  int rc = check_quant_args(x_bf16, rows, cols, ld_x, format, block, mode, flags, codes, ld_codes,
                            scales, ld_scales, tensor_scale);
  if (rc != FP4_OK) return rc;
  if (mode == FP4_RAZER_W) return FP4_ERR_UNSUPPORTED;  // a weight format; rotation is online
  if (hadamard != 0 && hadamard != block) return FP4_ERR_UNSUPPORTED;
  if (cols % 32 != 0) return FP4_ERR_SHAPE;  // the kernels work on 32-element segments
  if (perm && cols > fp4::kMaxPermCols) return FP4_ERR_UNSUPPORTED;
  if (rotated_out && ld_rot < cols) return FP4_ERR_SHAPE;
  const bool need_scale = format == FP4_NVFP4 && !(flags & FP4_FLAG_TENSOR_SCALE_GIVEN);
  const bool empty = rows == 0 || cols == 0;
  if (empty && !need_scale) return FP4_OK;
  if (!empty && perm && !aligned(perm, 4)) return FP4_ERR_ALIGN;
  if (!empty && rotated_out && (!aligned(rotated_out, 16) || ld_rot % 4 != 0)) return FP4_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Shape s{rows, cols, ld_x, ld_codes, ld_scales, (flags & FP4_FLAG_SCALES_GEMM) != 0};
  (void)hipGetLastError();
  if (format != FP4_NVFP4)
    fp4::launch_mx_rotate_quant(s, perm, hadamard, (flags & FP4_FLAG_SCALE_OCP_FLOOR) != 0,
                                format == FP4_MXINT4, x_bf16, codes, scales, rotated_out, ld_rot,
                                st);
  else
    fp4::launch_nv_rotate_quant(s, perm, hadamard, mode == FP4_RAZER, !need_scale, x_bf16, codes,
                                scales, tensor_scale, rotated_out, ld_rot, st);
  return launch_status();
}

int fp4_rotate_quantize_r(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                          const int32_t* perm, const float* rotation, void* codes,
                          int64_t ld_codes, void* scales, int64_t ld_scales, float* rotated_out,
                          int64_t ld_rot, void* stream) {
  int rc = check_quant_args(x_bf16, rows, cols, ld_x, FP4_MXFP4, 32, FP4_PLAIN, 0, codes, ld_codes,
                            scales, ld_scales, nullptr);
  if (rc != FP4_OK) return rc;
  if (cols > fp4::kMaxPermCols) return FP4_ERR_UNSUPPORTED;
  if (rotated_out && ld_rot < cols) return FP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!perm || !rotation) return FP4_ERR_NULL;
  if (!aligned(perm, 4) || !aligned(rotation, 4)) return FP4_ERR_ALIGN;
  if (rotated_out && (!aligned(rotated_out, 16) || ld_rot % 4 != 0)) return FP4_ERR_ALIGN;
  (void)hipGetLastError();
  fp4::launch_mx_matrix_rotate_quant(Shape{rows, cols, ld_x, ld_codes, ld_scales}, perm, rotation,
                                     x_bf16, codes, scales, rotated_out, ld_rot,
                                     static_cast<hipStream_t>(stream));
  return launch_status();
}

int fp4_dequantize_r(const void* codes, int64_t ld_codes, const void* scales, int64_t ld_scales,
                     int64_t rows, int64_t cols, const int32_t* perm, const float* rotation,
                     void* out_bf16, int64_t ld_out, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return FP4_ERR_SHAPE;
  if (ld_out < cols || ld_codes < cols / 2 || ld_scales < cols / 32) return FP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && rows * cols / 8 >= (int64_t)1 << 31) return FP4_ERR_UNSUPPORTED;
  if (cols > fp4::kMaxUnpermCols) return FP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales || !out_bf16 || !perm || !rotation) return FP4_ERR_NULL;
  if (!aligned(out_bf16, 16) || ld_out % 8 != 0) return FP4_ERR_ALIGN;
  if (!aligned(codes, 4) || ld_codes % 4 != 0) return FP4_ERR_ALIGN;
  if (!aligned(perm, 4) || !aligned(rotation, 4)) return FP4_ERR_ALIGN;
  (void)hipGetLastError();
  fp4::launch_mx_matrix_dequant_unrotate(Shape{rows, cols, ld_out, ld_codes, ld_scales}, perm,
                                         rotation, codes, scales, out_bf16,
                                         static_cast<hipStream_t>(stream));
  return launch_status();
}

int fp4_apply_channel_rotation(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               const int32_t* perm, const int32_t* pairs, const float* cs,
                               const int32_t* layer_start, int n_layers, int n_rot,
                               void* out_bf16, int64_t ld_out, void* stream) {
  if (rows < 0 || cols < 0 || cols % 8 != 0 || ld_x < cols || ld_out < cols) return FP4_ERR_SHAPE;
  if (n_layers < 0 || n_rot < 0) return FP4_ERR_SHAPE;
  if (cols > fp4::kMaxUnpermCols || rows >= ((int64_t)1 << 31)) return FP4_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return FP4_OK;
  if (!x_bf16 || !out_bf16) return FP4_ERR_NULL;
  if (n_layers > 0 && !layer_start) return FP4_ERR_NULL;
  if (n_rot > 0 && (!pairs || !cs || n_layers == 0)) return FP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || ld_x % 8 != 0 || !aligned(out_bf16, 16) || ld_out % 8 != 0)
    return FP4_ERR_ALIGN;
  if ((perm && !aligned(perm, 4)) || (pairs && !aligned(pairs, 4)) || (cs && !aligned(cs, 4)) ||
      (layer_start && !aligned(layer_start, 4)))
    return FP4_ERR_ALIGN;
  if (x_bf16 == out_bf16 && ld_x != ld_out) return FP4_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  fp4::launch_givens_rows(rows, cols, x_bf16, ld_x, perm, pairs, cs, layer_start, n_layers,
                          n_rot, out_bf16, ld_out, static_cast<hipStream_t>(stream));
  return launch_status();
}

int fp4_gemm(const void* a_codes, int64_t ld_a, const void* a_scales, int64_t ld_sa,
             const float* a_ts, int mode_a, const void* b_codes, int64_t ld_b,
             const void* b_scales, int64_t ld_sb, const float* b_ts, int mode_b, int64_t m,
             int64_t n, int64_t k, int format, int out_dtype, void* c, int64_t ld_c,
             void* stream) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_UNSUPPORTED;
  if (out_dtype != FP4_OUT_F32 && out_dtype != FP4_OUT_BF16) return FP4_ERR_UNSUPPORTED;
  // MXFP4 scale order per operand: row-major, or the GEMM order
  const bool sg_a = format == FP4_MXFP4 && (mode_a & (int)FP4_FLAG_SCALES_GEMM) != 0;
  const bool sg_b = format == FP4_MXFP4 && (mode_b & (int)FP4_FLAG_SCALES_GEMM) != 0;
  if (sg_a) mode_a &= ~(int)FP4_FLAG_SCALES_GEMM;
  if (sg_b) mode_b &= ~(int)FP4_FLAG_SCALES_GEMM;
  if (mode_a != FP4_PLAIN && mode_a != FP4_RAZER) return FP4_ERR_UNSUPPORTED;
  if (mode_b != FP4_PLAIN && mode_b != FP4_RAZER && mode_b != FP4_RAZER_W)
    return FP4_ERR_UNSUPPORTED;
  if (format == FP4_MXFP4 && (mode_a != FP4_PLAIN || mode_b != FP4_PLAIN))
    return FP4_ERR_UNSUPPORTED;
  const int blk = block_of(format);
  if (m < 0 || n < 0 || k < 0 || k % 32 != 0) return FP4_ERR_SHAPE;
  if (m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31) || k >= ((int64_t)1 << 31))
    return FP4_ERR_UNSUPPORTED;
  if (ld_a < k / 2 || ld_b < k / 2 || ld_c < n) return FP4_ERR_SHAPE;
  if (sg_a ? !gemm_scale_ld_ok(ld_sa, k) : ld_sa < k / blk) return FP4_ERR_SHAPE;
  if (sg_b ? !gemm_scale_ld_ok(ld_sb, k) : ld_sb < k / blk) return FP4_ERR_SHAPE;
  const int64_t lim = ((int64_t)1 << 31) / 256;
  if (ld_a >= lim || ld_b >= lim || ld_sa >= lim || ld_sb >= lim) return FP4_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return FP4_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4_ERR_NULL;
  if (format == FP4_NVFP4 && (!a_ts || !b_ts)) return FP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || ld_a % 16 != 0 || ld_b % 16 != 0)
    return FP4_ERR_ALIGN;
  // scale rows are read as dwords (MXFP4) or 16-bit pairs (NVFP4)
  const int sal = format == FP4_MXFP4 ? 4 : 2;
  if (!aligned(a_scales, sal) || !aligned(b_scales, sal) || ld_sa % sal != 0 || ld_sb % sal != 0)
    return FP4_ERR_ALIGN;
  if (format == FP4_NVFP4 && (!aligned(a_ts, 4) || !aligned(b_ts, 4))) return FP4_ERR_ALIGN;
  if (!aligned(c, out_dtype == FP4_OUT_F32 ? 4 : 2)) return FP4_ERR_ALIGN;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (format == FP4_MXFP4)
    fp4::launch_mx_gemm(m, n, k, a_codes, ld_a, a_scales, ld_sa, b_codes, ld_b, b_scales, ld_sb,
                        c, ld_c, out_dtype == FP4_OUT_BF16, sg_a, sg_b, st);
  else
    fp4::launch_nv_gemm(m, n, k, a_codes, ld_a, a_scales, ld_sa, a_ts, mode_a, b_codes, ld_b,
                        b_scales, ld_sb, b_ts, mode_b, c, ld_c,
                        out_dtype == FP4_OUT_BF16, st);
  return launch_status();
}

int fp4_channel_energy(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                       float* energy, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0 || ld_x < cols) return FP4_ERR_SHAPE;
  if (cols == 0) return FP4_OK;
  if (!x_bf16 || !energy) return FP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || ld_x % 8 != 0 || !aligned(energy, 4)) return FP4_ERR_ALIGN;
  if (cols / 32 >= (int64_t)1 << 31) return FP4_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  fp4::launch_channel_energy(rows, cols, ld_x, x_bf16, energy, static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"
