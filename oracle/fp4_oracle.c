/*
 * fp4_oracle.c -- plain, slow CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path. It shares no
 * code with the HIP kernels.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no FMA contraction, no fast-math, SSE float arithmetic: every float
 * expression below is one IEEE binary32 operation rounded to nearest-even).
 *
 * Sources (web pages explaining the papers; cited by title and section):
 *  [RaZeR]  "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
 *           Remapping", technical summary sec. 1 (E2M1 value set, the +0/-0
 *           redundancy, the always-positive E4M3 block scale whose sign bit is
 *           unused) and sec. 2.2 (a freed bit selects a special value that
 *           replaces the redundant zero code; the block picks the candidate of
 *           lowest mean squared quantization error; the activation pair is +-5,
 *           a multiple of 0.5 filling the gap between 4 and 6).
 *  [TORQ]   "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
 *           technical summary sec. 1 (32-element blocks sharing one exponent),
 *           sec. 2(a) (orthogonal transform that equalises the block variances),
 *           sec. 2(b) (intra-block rotation; the S-step maps each block's
 *           largest magnitude onto the largest MXFP4 code).
 * Where the pages are silent the reading used is stated at the function.
 *
 * Parity status of each function is recorded in oracle/__init__.py.
 */
#include "fp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

int orc_version(void) { return 1; }

void orc_set_threads(int n) { g_threads = n > 0 ? n : 1; }

int orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------------ */
/* Element format: FP4 E2M1, sign-magnitude.                                  */
/* [RaZeR] sec. 1 prints the value set {+-0, +-0.5, +-1, +-1.5, +-2, +-3,    */
/* +-4, +-6}. Code = sign << 3 | magnitude index, magnitudes in ascending    */
/* order (the usual E2M1 bit layout: 2 exponent bits, 1 mantissa bit).       */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double m = E2M1_MAG[code & 7];
  return (code & 8) ? -m : m;
}

/* Index of the magnitude nearest to a >= 0. Reading (pages silent): ties go
 * to the even index, i.e. round-half-to-even on the E2M1 mantissa bit; values
 * above 6 saturate to 6 because 6 is then the nearest magnitude. For a <= 6
 * that arises from an fp32 value times a power of two, every distance that
 * decides a near-tie is exact in double. */
static int nearest_mag(double a) {
  /* Every a > 6 is nearest to 6; stated directly because for very large a
   * the double distances below round to equal values. */
  if (a > 6.0) return 7;
  int best = 0;
  double bestd = fabs(a - E2M1_MAG[0]);
  for (int k = 1; k < 8; ++k) {
    double d = fabs(a - E2M1_MAG[k]);
    if (d < bestd || (d == bestd && (k % 2 == 0) && (best % 2 != 0))) {
      best = k;
      bestd = d;
    }
  }
  return best;
}

/* Plain E2M1 code of a scaled value y. Reading: the sign is kept even when
 * the magnitude rounds to zero (both zeros exist, [RaZeR] sec. 1), so a
 * negative value that rounds to zero gets code 0x8. */
int orc_e2m1_nearest(double y) {
  int s = signbit(y) ? 1 : 0;
  return (s << 3) | nearest_mag(fabs(y));
}

/* RaZeR code book: the fifteen standard values (zero only as +0, code 0x0)
 * plus the special value at the freed code 0x8 ([RaZeR] sec. 2.2). The
 * nearest entry wins; the special value wins only when strictly closer than
 * every standard value (reading: ties keep the standard code). */
int orc_e2m1_nearest_razer(double y, double special) {
  int idx = nearest_mag(fabs(y));
  double v_std = idx == 0 ? 0.0 : (signbit(y) ? -E2M1_MAG[idx] : E2M1_MAG[idx]);
  int code_std = idx == 0 ? 0 : (((signbit(y) ? 1 : 0) << 3) | idx);
  if (fabs(y - special) < fabs(y - v_std)) return 8;
  return code_std;
}

/* ------------------------------------------------------------------------ */
/* Block scale formats.                                                       */
/* ------------------------------------------------------------------------ */

/* FP8 E4M3 as used for the NVFP4 block scale ([RaZeR] sec. 1 names the
 * format). Reading: the OCP "E4M3FN" encoding -- bias 7, subnormals m*2^-9,
 * largest finite 448, S.1111.111 is NaN, no infinities. */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest non-negative finite E4M3 value to v >= 0 by exhaustive search over
 * the 127 codes 0x00..0x7E; ties go to the even code (round-half-to-even),
 * values above 448 saturate to 448 (code 0x7E) because it is then nearest. */
int orc_e4m3_encode(double v) {
  /* stated directly: for very large v the double distances round to equal */
  if (v > 448.0) return 0x7E;
  int best = 0;
  double bestd = fabs(v - orc_e4m3_value(0));
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(v - orc_e4m3_value(c));
    if (d < bestd || (d == bestd && (c % 2 == 0) && (best % 2 != 0))) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

/* E8M0: a bare power of two 2^(byte-127); byte 0xFF is NaN. */
double orc_e8m0_value(int byte) {
  if ((byte & 0xFF) == 0xFF) return NAN;
  return ldexp(1.0, (byte & 0xFF) - 127);
}

/* MXFP4 shared exponent of a block with largest magnitude amax.
 * Default rule ([TORQ] sec. 2(b), S-step: the block maximum maps onto the top
 * code, 6): the smallest e in [-127, 127] with amax <= 6 * 2^e, found by
 * trying every e in ascending order, so no element is clipped. amax == 0 gives
 * e = -127. A block holding Inf or NaN gets the NaN byte 0xFF.
 * floor_rule != 0 selects the alternative e = floor(log2 amax) - 2, clamped to
 * [-127, 127], under which magnitudes above 6 * 2^e saturate to 6. */
int orc_e8m0_scale(double amax, int floor_rule) {
  if (!isfinite(amax)) return 0xFF;
  if (floor_rule) {
    if (amax == 0.0) return 0;
    int k;
    frexp(amax, &k); /* amax = f * 2^k, f in [0.5, 1): floor(log2) = k - 1 */
    int e = (k - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
  }
  for (int e = -127; e <= 127; ++e)
    if (amax <= ldexp(6.0, e)) return e + 127;
  return 254;
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round-to-nearest-even binary32 -> bfloat16, NaN kept as a quiet NaN,
 * overflow to +-Inf. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void put_nibble(uint8_t* row_codes, int64_t j, int code) {
  uint8_t* b = row_codes + (j >> 1);
  if (j & 1)
    *b = (uint8_t)((*b & 0x0F) | ((code & 15) << 4));
  else
    *b = (uint8_t)((*b & 0xF0) | (code & 15));
}

static int get_nibble(const uint8_t* row_codes, int64_t j) {
  uint8_t b = row_codes[j >> 1];
  return (j & 1) ? (b >> 4) : (b & 15);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 quantization: blocks of 32 consecutive elements of a row ([TORQ]    */
/* sec. 1), one E8M0 byte per block, element 2i in the low nibble and 2i+1   */
/* in the high nibble of byte i (reading: pages silent on packing order).    */
/* ------------------------------------------------------------------------ */
static void mx_block(const float* v, int floor_rule, uint8_t* row_codes, int64_t j0,
                     uint8_t* scale_out) {
  double amax = 0.0;
  int nonfinite = 0;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(v[i])) nonfinite = 1;
    double a = fabs((double)v[i]);
    if (a > amax) amax = a;
  }
  if (nonfinite) {
    *scale_out = 0xFF;
    for (int i = 0; i < 32; ++i) put_nibble(row_codes, j0 + i, 0);
    return;
  }
  int byte = orc_e8m0_scale(amax, floor_rule);
  *scale_out = (uint8_t)byte;
  int e = byte - 127;
  for (int i = 0; i < 32; ++i) {
    double y = ldexp((double)v[i], -e); /* exact: a power-of-two rescale */
    put_nibble(row_codes, j0 + i, orc_e2m1_nearest(y));
  }
}

void orc_mx_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                         int floor_rule, uint8_t* codes, int64_t ld_codes,
                         uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 32; ++b)
      mx_block(x + r * ld_x + 32 * b, floor_rule, codes + r * ld_codes, 32 * b,
               scales + r * ld_scales + b);
}

void orc_mx_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          int floor_rule, uint8_t* codes, int64_t ld_codes,
                          uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    float v[32];
    for (int64_t b = 0; b < cols / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = orc_bf16_to_f32(x[r * ld_x + 32 * b + i]);
      mx_block(v, floor_rule, codes + r * ld_codes, 32 * b, scales + r * ld_scales + b);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* MXINT4: [TORQ] (the generalisation remark of its results) reports the     */
/* rotation with an MXINT4 grid as well; the pages name the format only.     */
/* Reading: the microscaling integer element of the OCP MX family at 4 bits: */
/* a two's complement integer k in [-8, 7] read as fixed point with two      */
/* fraction bits (value k / 4, largest power of two 1, the 4-bit analogue of */
/* MXINT8's k / 64), 32-element blocks, one E8M0 byte per block.             */
/* Encoding: nearest grid value, ties to even k, clamped to k in [-7, 7] so  */
/* the grid is symmetric (k = -8 only decodes). Scale rule, as for MXFP4:    */
/* the smallest e with amax <= 1.75 * 2^e (the top symmetric code), so no    */
/* element is clipped (e is capped at 127, so a magnitude above 1.75 * 2^127 */
/* saturates); the floor rule takes e = floor(log2 amax), the element        */
/* format's largest power of two being 1, and saturates at 1.75.             */
/* ------------------------------------------------------------------------ */
double orc_int4_value(int code) {
  int k = code & 15;
  if (k >= 8) k -= 16;
  return k / 4.0;
}

/* Nearest k / 4 (|k| <= 7) to y by brute force; ties to the even k. */
int orc_int4_nearest(double y) {
  int best = 0;
  double bd = INFINITY;
  for (int k = -7; k <= 7; ++k) {
    double d = fabs(y - k / 4.0);
    if (d < bd || (d == bd && (k & 1) == 0)) {
      bd = d;
      best = k;
    }
  }
  return best & 15;
}

int orc_mxint4_scale(double amax, int floor_rule) {
  if (!isfinite(amax)) return 0xFF;
  if (floor_rule) {
    if (amax == 0.0) return 0;
    int k;
    frexp(amax, &k); /* floor(log2 amax) = k - 1 */
    int e = k - 1;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
  }
  for (int e = -127; e <= 127; ++e)
    if (amax <= ldexp(1.75, e)) return e + 127;
  return 254;
}

static void mxint_block(const float* v, int floor_rule, uint8_t* row_codes, int64_t j0,
                        uint8_t* scale_out) {
  double amax = 0.0;
  int nonfinite = 0;
  for (int i = 0; i < 32; ++i) {
    if (!isfinite(v[i])) nonfinite = 1;
    double a = fabs((double)v[i]);
    if (a > amax) amax = a;
  }
  if (nonfinite) { /* as for MXFP4: the NaN scale byte, codes 0 */
    *scale_out = 0xFF;
    for (int i = 0; i < 32; ++i) put_nibble(row_codes, j0 + i, 0);
    return;
  }
  int byte = orc_mxint4_scale(amax, floor_rule);
  *scale_out = (uint8_t)byte;
  for (int i = 0; i < 32; ++i)
    put_nibble(row_codes, j0 + i, orc_int4_nearest(ldexp((double)v[i], 127 - byte)));
}

void orc_mxint4_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x,
                             int floor_rule, uint8_t* codes, int64_t ld_codes,
                             uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 32; ++b)
      mxint_block(x + r * ld_x + 32 * b, floor_rule, codes + r * ld_codes, 32 * b,
                  scales + r * ld_scales + b);
}

void orc_mxint4_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              int floor_rule, uint8_t* codes, int64_t ld_codes,
                              uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    float v[32];
    for (int64_t b = 0; b < cols / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = orc_bf16_to_f32(x[r * ld_x + 32 * b + i]);
      mxint_block(v, floor_rule, codes + r * ld_codes, 32 * b, scales + r * ld_scales + b);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* NVFP4: blocks of 16, E4M3 block scale, fp32 per-tensor scale s_t.          */
/* The scale is derived from the block absmax and is therefore positive, so  */
/* its sign bit is free ([RaZeR] sec. 1). Readings where the pages are       */
/* silent: s_t = amax_t / (6 * 448) so the largest block product reaches     */
/* 6 * 448; s_raw = amax_b / (6 * s_t); the E4M3 byte is the nearest value;  */
/* the element scale is s_eff = e4m3(s_b) * s_t and elements are multiplied  */
/* by the rounded reciprocal of s_eff. Each step is one fp32 operation.      */
/* ------------------------------------------------------------------------ */
float orc_nv_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x) {
  float amax = 0.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) {
      float a = fabsf(orc_bf16_to_f32(x[r * ld_x + j]));
      if (a > amax) amax = a;
    }
  return amax;
}

float orc_nv_tensor_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / 2688.0f; /* 2688 = 6 * 448 */
}

/* [RaZeR] sec. 2.2: per block, pick from the pair {+5, -5} the special value
 * of least squared quantization error; the selector is stored in the block
 * scale's free sign bit (reading: bit 0 -> +5, bit 1 -> -5; equal error ->
 * bit 0). codes[] receives n unpacked codes for the chosen candidate.
 *
 * The two candidate code vectors differ only where the nearest entry changes;
 * elsewhere both squared errors are the same double, so their difference is
 * exactly zero. Where they differ, y lies in (4.5, 5.5), a binade in which
 * fp32 values are multiples of 2^-21, so each squared error and each
 * difference is exact in double and so is the sum. SSE(+5) - SSE(-5) is
 * therefore computed without rounding error and the comparison is exact.
 * Returns the selector bit. */
int orc_razer_block(const float* y, int n, uint8_t* codes, double* sse_chosen,
                    double* sse_plain) {
  uint8_t cp[64], cm[64];
  double diff = 0.0, ssp = 0.0, ssm = 0.0, ss0 = 0.0;
  for (int i = 0; i < n; ++i) {
    double v = (double)y[i];
    cp[i] = (uint8_t)orc_e2m1_nearest_razer(v, 5.0);
    cm[i] = (uint8_t)orc_e2m1_nearest_razer(v, -5.0);
    double vp = cp[i] == 8 ? 5.0 : orc_e2m1_value(cp[i]);
    double vm = cm[i] == 8 ? -5.0 : orc_e2m1_value(cm[i]);
    double ep = (v - vp) * (v - vp), em = (v - vm) * (v - vm);
    diff += ep - em;
    ssp += ep;
    ssm += em;
    double v0 = orc_e2m1_value(orc_e2m1_nearest(v));
    ss0 += (v - v0) * (v - v0);
  }
  int sel = diff > 0.0 ? 1 : 0;
  for (int i = 0; i < n; ++i) codes[i] = sel ? cm[i] : cp[i];
  if (sse_chosen) *sse_chosen = sel ? ssm : ssp;
  if (sse_plain) *sse_plain = ss0;
  return sel;
}

/* One NVFP4 block of 16 values (already widened to fp32): [RaZeR] sec. 1 with
 * the arithmetic of the NVFP4 section comment above:
 * s_raw = RN(amax / RN(6 s_t)), s_b = E4M3(s_raw), s_eff = RN(e4m3(s_b) s_t),
 * y = RN(x * RN(1 / s_eff)), then the nearest code (RaZeR: sec. 2.2). */
static void nv_block(const float* xv, int razer, float s_t, uint8_t* rc, int64_t b,
                     uint8_t* scale) {
  const float d = 6.0f * s_t;
  float y[16];
  float amax = 0.0f;
  for (int i = 0; i < 16; ++i)
    if (fabsf(xv[i]) > amax) amax = fabsf(xv[i]);
  float s_raw = amax / d;
  int sb = orc_e4m3_encode((double)s_raw);
  if (sb == 0) { /* scale rounds to zero: the block is stored as zeros */
    for (int i = 0; i < 16; ++i) put_nibble(rc, 16 * b + i, 0);
    *scale = 0;
    return;
  }
  float s_eff = (float)orc_e4m3_value(sb) * s_t;
  float rcp = 1.0f / s_eff;
  for (int i = 0; i < 16; ++i) y[i] = xv[i] * rcp;
  if (razer) {
    uint8_t c[16];
    int sel = orc_razer_block(y, 16, c, NULL, NULL);
    for (int i = 0; i < 16; ++i) put_nibble(rc, 16 * b + i, c[i]);
    *scale = (uint8_t)(sb | (sel << 7));
  } else {
    for (int i = 0; i < 16; ++i) put_nibble(rc, 16 * b + i, orc_e2m1_nearest((double)y[i]));
    *scale = (uint8_t)sb;
  }
}

void orc_nv_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                          int razer, float tensor_scale, uint8_t* codes, int64_t ld_codes,
                          uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      float xv[16];
      for (int i = 0; i < 16; ++i) xv[i] = orc_bf16_to_f32(x[r * ld_x + 16 * b + i]);
      nv_block(xv, razer, tensor_scale, codes + r * ld_codes, b, scales + r * ld_scales + b);
    }
  }
}

/* The same quantizer on fp32 values (for instance the rotated values of the
 * two-level rotation, which are not bf16). */
void orc_nv_quantize_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x, int razer,
                         float tensor_scale, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                         int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 16; ++b)
      nv_block(x + r * ld_x + 16 * b, razer, tensor_scale, codes + r * ld_codes, b,
               scales + r * ld_scales + b);
}

/* Largest |x| over an fp32 tensor. */
float orc_nv_tensor_amax_f32(const float* x, int64_t rows, int64_t cols, int64_t ld_x) {
  float m = 0.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      float v = fabsf(x[r * ld_x + c]);
      if (v > m) m = v;
    }
  return m;
}

/* ------------------------------------------------------------------------ */
/* RaZeR for weights ([RaZeR] sec. 2.1 and 2.2): weights tolerate a coarser  */
/* block scale, E3M3 (6 bits) instead of E4M3, which frees 2 bits per block; */
/* they select one of four special values, two +- pairs computed offline,    */
/* for the redundant code 0x8, the block taking the one of least squared     */
/* error. Readings where the pages are silent: E3M3 "fn"-style, bias 3,      */
/* subnormals m 2^-5, largest 30, no Inf or NaN; the tensor scale maps the   */
/* largest block onto 6 * 30, s_t = amax_t / 180; selector i picks           */
/* {+5, -5, +p, -p}[i] (the pages give +-5; p is the second pair); the scale  */
/* byte is e3m3 | i << 6. Ties: the lowest selector; an element takes the    */
/* special code only when strictly closer to it than to every standard value.*/
/* ------------------------------------------------------------------------ */
double orc_e3m3_value(int code) {
  int e = (code >> 3) & 7, m = code & 7;
  if (e == 0) return ldexp((double)m, -5);
  return ldexp(1.0 + m / 8.0, e - 3);
}

int orc_e3m3_encode(double v) {
  if (v > 30.0) return 63;
  int best = 0;
  double bestd = fabs(v - orc_e3m3_value(0));
  for (int c = 1; c < 64; ++c) {
    double d = fabs(v - orc_e3m3_value(c));
    if (d < bestd || (d == bestd && (c % 2 == 0) && (best % 2 != 0))) {
      best = c;
      bestd = d;
    }
  }
  return best;
}

float orc_nvw_tensor_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  return amax / 180.0f;
}

/* Index of the special value (of ns) whose code book gives the least squared
 * error on y[0..n): the error of an element differs between candidates only
 * where it takes code 0x8, so the candidates are ranked by their total gain
 * over plain E2M1, exact in double (see orc_razer_block). */
int orc_razer_block_set(const float* y, int n, const double* specials, int ns, uint8_t* codes) {
  double best_gain = -1.0;
  int best = 0;
  for (int i = 0; i < ns; ++i) {
    double gain = 0.0;
    for (int j = 0; j < n; ++j) {
      double v = (double)y[j];
      int c = orc_e2m1_nearest_razer(v, specials[i]);
      if (c == 8) {
        double vs = orc_e2m1_value(orc_e2m1_nearest(v));
        gain += (v - vs) * (v - vs) - (v - specials[i]) * (v - specials[i]);
      }
    }
    if (gain > best_gain) {
      best_gain = gain;
      best = i;
    }
  }
  for (int j = 0; j < n; ++j) codes[j] = (uint8_t)orc_e2m1_nearest_razer((double)y[j], specials[best]);
  return best;
}

static void nvw_block(const float* xv, float s_t, double p, uint8_t* rc, int64_t b,
                      uint8_t* scale) {
  const double specials[4] = {5.0, -5.0, p, -p};
  const float d = 6.0f * s_t;
  float amax = 0.0f;
  for (int i = 0; i < 16; ++i)
    if (fabsf(xv[i]) > amax) amax = fabsf(xv[i]);
  float s_raw = amax / d;
  int sb = orc_e3m3_encode((double)s_raw);
  if (sb == 0) {
    for (int i = 0; i < 16; ++i) put_nibble(rc, 16 * b + i, 0);
    *scale = 0;
    return;
  }
  float s_eff = (float)orc_e3m3_value(sb) * s_t;
  float rcp = 1.0f / s_eff;
  float y[16];
  uint8_t c[16];
  for (int i = 0; i < 16; ++i) y[i] = xv[i] * rcp;
  int sel = orc_razer_block_set(y, 16, specials, 4, c);
  for (int i = 0; i < 16; ++i) put_nibble(rc, 16 * b + i, c[i]);
  *scale = (uint8_t)(sb | (sel << 6));
}

void orc_nvw_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                           float tensor_scale, double p, uint8_t* codes, int64_t ld_codes,
                           uint8_t* scales, int64_t ld_scales) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      float xv[16];
      for (int i = 0; i < 16; ++i) xv[i] = orc_bf16_to_f32(x[r * ld_x + 16 * b + i]);
      nvw_block(xv, tensor_scale, p, codes + r * ld_codes, b, scales + r * ld_scales + b);
    }
  }
}

/* Value of a weight-RaZeR element before the tensor scale: e2m1 or special,
 * times e3m3(scale). */
double orc_nvw_value(int code, int byte, double p) {
  const double specials[4] = {5.0, -5.0, p, -p};
  double v = code == 8 ? specials[(byte >> 6) & 3] : orc_e2m1_value(code);
  return v * orc_e3m3_value(byte & 63);
}

/* ------------------------------------------------------------------------ */
/* Dequantization. MXFP4 and MXINT4: value * 2^e, exact before the final   */
/* rounding.                                                                 */
/* NVFP4: fp32 product value * s_eff. RaZeR: code 0x8 decodes to the block's */
/* special value, +5 or -5 by the scale's top bit ([RaZeR] sec. 2.2 and 2.3: */
/* the decoder rebuilds the special value from the metadata bits).           */
/* A NaN E8M0 byte decodes every element of its block to NaN.                */
/* ------------------------------------------------------------------------ */
static double dq_value(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                       int64_t ld_scales, float s_t, int64_t r, int64_t j, int format,
                       int razer, double p) {
  int c = get_nibble(codes + r * ld_codes, j);
  if (format == 0 || format == 2) {
    int byte = scales[r * ld_scales + j / 32];
    if (byte == 0xFF) return NAN;
    return ldexp(format == 0 ? orc_e2m1_value(c) : orc_int4_value(c), byte - 127);
  }
  int byte = scales[r * ld_scales + j / 16];
  double v;
  float s_eff;
  if (razer == 2) { /* weights: E3M3 scale, four specials */
    const double specials[4] = {5.0, -5.0, p, -p};
    s_eff = (float)orc_e3m3_value(byte & 63) * s_t;
    v = (c == 8) ? specials[(byte >> 6) & 3] : orc_e2m1_value(c);
  } else if (razer) {
    s_eff = (float)orc_e4m3_value(byte & 0x7F) * s_t;
    v = (c == 8) ? ((byte & 0x80) ? -5.0 : 5.0) : orc_e2m1_value(c);
  } else {
    s_eff = (float)orc_e4m3_value(byte) * s_t;
    v = orc_e2m1_value(c);
  }
  float prod = (float)v * s_eff;
  return (double)prod;
}

void orc_dequantize_f64(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                        int64_t ld_scales, float tensor_scale, int64_t rows, int64_t cols,
                        int format, int razer, double p, double* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j)
      out[r * ld_out + j] =
          dq_value(codes, ld_codes, scales, ld_scales, tensor_scale, r, j, format, razer, p);
}

void orc_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                    int64_t ld_scales, float tensor_scale, int64_t rows, int64_t cols,
                    int format, int razer, double p, uint16_t* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) {
      double v = dq_value(codes, ld_codes, scales, ld_scales, tensor_scale, r, j, format, razer, p);
      out[r * ld_out + j] = orc_f32_to_bf16((float)v); /* exact or already fp32 */
    }
}

/* ------------------------------------------------------------------------ */
/* Two-level rotation ([TORQ] sec. 2(a) and 2(b)).                            */
/* Level 1: a channel permutation pi, x'[j] = x[pi(j)], chosen offline so    */
/* that every 32-block receives the same mix of high- and low-energy         */
/* channels (an orthogonal transform that evens out the block variances).    */
/* Level 2: the orthonormal Sylvester-Hadamard matrix inside each block,     */
/* H[i][j] = (-1)^popcount(i & j) / sqrt(n), applied as a dense product in   */
/* double and rounded once to fp32.                                          */
/* ------------------------------------------------------------------------ */
double orc_hadamard_entry(int n, int i, int j) {
  int p = __builtin_popcount((unsigned)(i & j)) & 1;
  return (p ? -1.0 : 1.0) / sqrt((double)n);
}

void orc_rotate(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                const int32_t* perm, int hadamard, float* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    double xp[64];
    for (int64_t b0 = 0; b0 < cols; b0 += (hadamard ? hadamard : cols)) {
      int64_t n = hadamard ? hadamard : cols;
      for (int64_t j = 0; j < n; ++j) {
        int64_t src = perm ? perm[b0 + j] : b0 + j;
        double v = (double)orc_bf16_to_f32(x[r * ld_x + src]);
        if (hadamard)
          xp[j] = v;
        else
          out[r * ld_out + b0 + j] = (float)v;
      }
      if (!hadamard) break;
      for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j) acc += orc_hadamard_entry((int)n, i, j) * xp[j];
        out[r * ld_out + b0 + i] = (float)acc;
      }
    }
  }
}

/* Inverse of orc_rotate in double: H is symmetric and orthonormal, so its
 * inverse is H itself; the permutation is undone by scattering to pi(j). */
void orc_unrotate_f64(const double* y, int64_t rows, int64_t cols, int64_t ld_y,
                      const int32_t* perm, int hadamard, double* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    int64_t n = hadamard ? hadamard : 1;
    for (int64_t b0 = 0; b0 < cols; b0 += n) {
      for (int64_t j = 0; j < n; ++j) {
        double acc;
        if (hadamard) {
          acc = 0.0;
          for (int64_t i = 0; i < n; ++i)
            acc += orc_hadamard_entry((int)n, (int)i, (int)j) * y[r * ld_y + b0 + i];
        } else {
          acc = y[r * ld_y + b0 + j];
        }
        int64_t dst = perm ? perm[b0 + j] : b0 + j;
        out[r * ld_out + dst] = acc;
      }
    }
  }
}

/* A general orthogonal rotation inside each 32-block ([TORQ] sec. 2(b): the
 * intra-block rotation is learned): y_b = R x'_b with R [32][32] row-major,
 * as a dense product in double rounded once to fp32; x' is the permuted row. */
void orc_rotate_r(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                  const int32_t* perm, const double* R, float* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    double xp[32];
    for (int64_t b0 = 0; b0 < cols; b0 += 32) {
      for (int j = 0; j < 32; ++j) {
        int64_t src = perm ? perm[b0 + j] : b0 + j;
        xp[j] = (double)orc_bf16_to_f32(x[r * ld_x + src]);
      }
      for (int i = 0; i < 32; ++i) {
        double acc = 0.0;
        for (int j = 0; j < 32; ++j) acc += R[32 * i + j] * xp[j];
        out[r * ld_out + b0 + i] = (float)acc;
      }
    }
  }
}

/* Inverse: x'_b = R^T y_b, then element j of the row goes to column perm[j]. */
void orc_unrotate_r_f64(const double* y, int64_t rows, int64_t cols, int64_t ld_y,
                        const int32_t* perm, const double* R, double* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r)
    for (int64_t b0 = 0; b0 < cols; b0 += 32)
      for (int j = 0; j < 32; ++j) {
        double acc = 0.0;
        for (int i = 0; i < 32; ++i) acc += R[32 * i + j] * y[r * ld_y + b0 + i];
        out[r * ld_out + (perm ? perm[b0 + j] : b0 + j)] = acc;
      }
}

/* Code-book occupancy ([TORQ] sec. 2(b), the occupancy-equilibrium loss):
 * quantize every 32-block of y to MXFP4 (default scale rule) and count the
 * elements per E2M1 magnitude index 0..7; hist receives the 8 fractions.
 * The loss is their squared distance from the uniform 1/8 (returned). */
double orc_occupancy(const float* y, int64_t rows, int64_t cols, int64_t ld, double* hist) {
  double cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b0 = 0; b0 < cols; b0 += 32) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        double a = fabs((double)y[r * ld + b0 + i]);
        if (a > amax) amax = a;
      }
      int e = orc_e8m0_scale(amax, 0) - 127;
      for (int i = 0; i < 32; ++i)
        cnt[nearest_mag(fabs(ldexp((double)y[r * ld + b0 + i], -e)))] += 1.0;
    }
  double n = (double)(rows * (cols / 32) * 32), loss = 0.0;
  for (int c = 0; c < 8; ++c) {
    hist[c] = n > 0 ? cnt[c] / n : 0.0;
    loss += (hist[c] - 0.125) * (hist[c] - 0.125);
  }
  return loss;
}

/* [TORQ] sec. 2(a): the inter-block transform built from Givens rotations.
 * x'[j] = x[perm[j]] (perm NULL: identity), then for k = 0 .. n-1 in order,
 * with (i, j) = pairs[2k], pairs[2k+1] and (c, s) = cs[2k], cs[2k+1]:
 *   (x'_i, x'_j) <- (c x'_i - s x'_j, s x'_i + c x'_j).
 * fp64 throughout (the written definition, one rotation after another). */
void orc_apply_givens(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                      const int32_t* perm, int64_t n, const int32_t* pairs, const double* cs,
                      double* out, int64_t ld_out) {
  int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (r = 0; r < rows; ++r) {
    double* z = out + r * ld_out;
    for (int64_t j = 0; j < cols; ++j)
      z[j] = (double)orc_bf16_to_f32(x[r * ld_x + (perm ? perm[j] : j)]);
    for (int64_t k = 0; k < n; ++k) {
      const int32_t i = pairs[2 * k], j = pairs[2 * k + 1];
      const double c = cs[2 * k], s = cs[2 * k + 1];
      const double zi = z[i], zj = z[j];
      z[i] = c * zi - s * zj;
      z[j] = s * zi + c * zj;
    }
  }
}

/* Per-channel energy E_c = sum over rows of x_rc^2, in double, row order.
 * It is the diagonal of the (uncentred) activation second-moment matrix whose
 * 32x32 diagonal blocks carry the block variances in [TORQ] sec. 2(a). */
void orc_channel_energy(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                        double* energy) {
  for (int64_t j = 0; j < cols; ++j) energy[j] = 0.0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) {
      double v = (double)orc_bf16_to_f32(x[r * ld_x + j]);
      energy[j] += v * v;
    }
}

static const double* g_sort_energy;

static int by_energy_desc(const void* a, const void* b) {
  int32_t ia = *(const int32_t*)a, ib = *(const int32_t*)b;
  double ea = g_sort_energy[ia], eb = g_sort_energy[ib];
  if (ea > eb) return -1;
  if (ea < eb) return 1;
  return ia < ib ? -1 : (ia > ib ? 1 : 0);
}

/* Magnitude-balancing permutation (reading of [TORQ] sec. 2(a) -- an
 * orthogonal transform that makes the block variances equal -- restricted to
 * permutations; the pages build their macro rotation from Givens rotations).
 * The unit moved is an aligned run of `group` channels (1 = single channels;
 * 2, 4 or 8 keep neighbouring channels together), with energy the sum of its
 * channels' energies in double, in channel order. Units are taken largest
 * energy first (equal energies: lower index first); each goes to the block
 * whose accumulated energy is smallest among the blocks that still have a
 * free unit slot (equal loads: lower block index), in the block's next free
 * slot, keeping its channels in order. Loads are summed in double. perm[j] is
 * the source channel of position j. Not thread-safe (qsort comparator state). */
void orc_build_perm(const float* energy, int64_t cols, int block, int group, int32_t* perm) {
  int64_t B = cols / block, nu = cols / group, slots = block / group;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)nu);
  double* ue = (double*)malloc(sizeof(double) * (size_t)nu);
  double* load = (double*)calloc((size_t)B, sizeof(double));
  int64_t* fill = (int64_t*)calloc((size_t)B, sizeof(int64_t));
  for (int64_t u = 0; u < nu; ++u) {
    order[u] = (int32_t)u;
    ue[u] = 0.0;
    for (int i = 0; i < group; ++i) ue[u] += (double)energy[u * group + i];
  }
  g_sort_energy = ue;
  qsort(order, (size_t)nu, sizeof(int32_t), by_energy_desc);
  for (int64_t t = 0; t < nu; ++t) {
    int64_t best = -1;
    for (int64_t b = 0; b < B; ++b) {
      if (fill[b] == slots) continue;
      if (best < 0 || load[b] < load[best]) best = b;
    }
    int32_t u = order[t];
    for (int i = 0; i < group; ++i)
      perm[best * block + fill[best] * group + i] = u * group + i;
    fill[best] += 1;
    load[best] += ue[u];
  }
  free(order);
  free(ue);
  free(load);
  free(fill);
}
