/*
 * fp4_oracle.h -- plain, slow CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path never
 * calls it and shares no code, header, table or helper with it.
 *
 * Every function computes its result by definition: brute-force nearest search
 * over the code book, exact comparisons in double precision, and dense 32x32
 * matrix products for the rotation. See fp4_oracle.c for the page citations.
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int orc_version(void);
void orc_set_threads(int n);
int orc_get_threads(void);

/* element and scale formats */
double orc_e2m1_value(int code);
int orc_e2m1_nearest(double y);
int orc_e2m1_nearest_razer(double y, double special);
double orc_e4m3_value(int code);
int orc_e4m3_encode(double v);
double orc_e8m0_value(int byte);
int orc_e8m0_scale(double amax, int floor_rule);
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);

/* MXFP4: 32-element blocks, E8M0 scale */
void orc_mx_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                         int floor_rule, uint8_t* codes, int64_t ld_codes,
                         uint8_t* scales, int64_t ld_scales);
void orc_mx_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          int floor_rule, uint8_t* codes, int64_t ld_codes,
                          uint8_t* scales, int64_t ld_scales);

/* MXINT4: 32-element blocks, E8M0 scale, two's complement k / 4 elements */
double orc_int4_value(int code);
int orc_int4_nearest(double y);
int orc_mxint4_scale(double amax, int floor_rule);
void orc_mxint4_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                             int floor_rule, uint8_t* codes, int64_t ld_codes,
                             uint8_t* scales, int64_t ld_scales);
void orc_mxint4_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              int floor_rule, uint8_t* codes, int64_t ld_codes,
                              uint8_t* scales, int64_t ld_scales);

/* NVFP4: 16-element blocks, E4M3 block scale, fp32 tensor scale; RaZeR option */
float orc_nv_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x);
float orc_nv_tensor_scale(float amax);
void orc_nv_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          int razer, float tensor_scale, uint8_t* codes, int64_t ld_codes,
                          uint8_t* scales, int64_t ld_scales);
void orc_nv_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int razer,
                         float tensor_scale, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                         int64_t ld_scales);
float orc_nv_tensor_amax_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x);
int orc_razer_block(const float* y, int n, uint8_t* codes, double* sse_chosen,
                    double* sse_plain);

/* RaZeR for weights: E3M3 block scale, selector over {+5, -5, +p, -p} */
double orc_e3m3_value(int code);
int orc_e3m3_encode(double v);
float orc_nvw_tensor_scale(float amax);
int orc_razer_block_set(const float* y, int n, const double* specials, int ns, uint8_t* codes);
void orc_nvw_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                           float tensor_scale, double p, uint8_t* codes, int64_t ld_codes,
                           uint8_t* scales, int64_t ld_scales);
double orc_nvw_value(int code, int byte, double p);

/* dequantization; format 0 = MXFP4, 1 = NVFP4, 2 = MXINT4; razer 2 = the
 * weight variant (second special pair +-p) */
void orc_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                    int64_t ld_scales, float tensor_scale, int64_t rows, int64_t cols,
                    int format, int razer, double p, uint16_t* out, int64_t ld_out);
void orc_dequantize_f64(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                        int64_t ld_scales, float tensor_scale, int64_t rows, int64_t cols,
                        int format, int razer, double p, double* out, int64_t ld_out);

/* two-level rotation: permutation across blocks, Hadamard inside each block */
void orc_rotate(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                const int32_t* perm, int hadamard, float* out, int64_t ld_out);
void orc_unrotate_f64(const double* y, int64_t rows, int64_t cols, int64_t ld_y,
                      const int32_t* perm, int hadamard, double* out, int64_t ld_out);
void orc_rotate_r(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                  const int32_t* perm, const double* R, float* out, int64_t ld_out);
void orc_unrotate_r_f64(const double* y, int64_t rows, int64_t cols, int64_t ld_y,
                        const int32_t* perm, const double* R, double* out, int64_t ld_out);
void orc_apply_givens(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                      const int32_t* perm, int64_t n, const int32_t* pairs, const double* cs,
                      double* out, int64_t ld_out);
double orc_occupancy(const float* y, int64_t rows, int64_t cols, int64_t ld, double* hist);
void orc_channel_energy(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                        double* energy);
void orc_build_perm(const float* energy, int64_t cols, int block, int group, int32_t* perm);
double orc_hadamard_entry(int n, int i, int j);

#ifdef __cplusplus
}
#endif
#endif
