/*
 * fp4.h -- block-scaled 4-bit (MXFP4 / NVFP4 / MXINT4) quantization on AMD Instinct
 * MI355X (gfx950): C ABI of libfp4.so.
 *
 * Sources (web pages explaining the papers; cited by title and section):
 *  [RaZeR] "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
 *          Remapping", technical summary sec. 1 (FP4 E2M1 value set with both
 *          zeros; E4M3 block scale that is always positive, so its sign bit is
 *          free) and sec. 2.2 (the freed bit selects a special value, +5 or -5,
 *          that replaces the redundant zero code; chosen per block by least
 *          squared error).
 *  [TORQ]  "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
 *          technical summary sec. 1 (32-element blocks sharing one exponent)
 *          and sec. 2 (an inter-block transform that evens out block variances,
 *          then a rotation inside each block; the scale maps the block maximum
 *          onto the largest code) and the generalisation remark of its results
 *          (the rotation with NVFP4 and with an MXINT4 grid).
 *
 * Conventions shared by every entry point
 *  - Matrices are row-major. A block is `block` consecutive elements of one
 *    row (32 for MXFP4 and MXINT4, 16 for NVFP4). `ld_*` is the row stride in elements
 *    of that array (bytes for the uint8 code and scale arrays).
 *  - codes: uint8 [rows, ld_codes], element 2i of a row in the low nibble of
 *    byte i and element 2i+1 in the high nibble. FP4 E2M1 code =
 *    sign << 3 | magnitude index, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *    MXINT4 code: a two's complement nibble k in [-8, 7], value k / 4 (the
 *    4-bit microscaling integer element: two fraction bits; reading, the
 *    pages name the format only).
 *  - scales: uint8 [rows, ld_scales], one byte per block. MXFP4, MXINT4: E8M0 byte,
 *    scale 2^(byte-127), 0xFF = NaN. NVFP4: E4M3 (OCP "fn") byte; in RaZeR
 *    mode bit 7 holds the selector (0: code 0x8 means +5, 1: -5) and bits 0-6
 *    the positive scale.
 *  - tensor_scale (NVFP4 only): one fp32 in device memory; element scale of a
 *    block = e4m3(scale byte) * tensor_scale.
 *  - Ownership: every pointer except those marked "host" is device memory
 *    owned by the caller. The library allocates nothing and keeps no handle
 *    between calls. Work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and the call returns without waiting: outputs are valid
 *    once the stream has reached this point.
 *  - Errors: arguments are checked before anything is enqueued; on failure
 *    nothing is enqueued and a negative fp4_status is returned. FP4_ERR_HIP
 *    means a launch failed after the arguments were accepted.
 *  - Rounding (readings where the pages are silent): nearest E2M1 value with
 *    ties to the even code, saturating at 6; the sign of an element that
 *    rounds to zero is kept (code 0x8) except in RaZeR mode, where zero is
 *    always 0x0.
 */
#ifndef FP4_H
#define FP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4_VERSION 1

enum fp4_format { FP4_MXFP4 = 0, FP4_NVFP4 = 1, FP4_MXINT4 = 2 };
enum fp4_mode { FP4_PLAIN = 0, FP4_RAZER = 1, FP4_RAZER_W = 2 };

/* NVFP4: read tensor_scale as an input instead of computing it. */
#define FP4_FLAG_TENSOR_SCALE_GIVEN 1u
/* MXFP4: shared exponent floor(log2 amax) - 2 (elements above 6 * 2^e
 * saturate) instead of the default smallest e with amax <= 6 * 2^e.
 * MXINT4: floor(log2 amax) (elements above 1.75 * 2^e saturate) instead of the
 * default smallest e with amax <= 1.75 * 2^e. */
#define FP4_FLAG_SCALE_OCP_FLOOR 2u
/* MXFP4 only: scale bytes in the GEMM's order instead of [rows, ld_scales]
 * (the scale layout that fp4_gemm reads fastest; [RaZeR] sec. 2.3, GEMM
 * kernels fed by the quantizer's own output). Rows form groups of 32, and a
 * group's scales are kept in steps of 256 elements of the row (8 blocks):
 * the byte of row r, block b sits at
 *     (r / 32) * ld_scales + (b / 8) * 256 + (r % 32) * 8 + b % 8,
 * so each 256-element step of a 32-row group is 256 contiguous bytes. Here
 * ld_scales is the stride between row groups: a multiple of 256, at least
 * 256 * ceil(cols / 256); the array holds ceil(rows / 32) * ld_scales bytes.
 * Bytes of rows past `rows` and of blocks past cols / 32 are never written
 * and do not affect fp4_gemm's results. Taken by fp4_quantize and
 * fp4_rotate_quantize in `flags`, and by fp4_gemm OR-ed into mode_a or
 * mode_b (per operand). fp4_dequantize reads [rows, ld_scales] only. */
#define FP4_FLAG_SCALES_GEMM 0x100u

enum fp4_status {
  FP4_OK = 0,
  FP4_ERR_NULL = -1,        /* a required pointer is NULL */
  FP4_ERR_SHAPE = -2,       /* negative size, cols % block != 0, ld too small */
  FP4_ERR_ALIGN = -3,       /* pointer or row stride not aligned as stated */
  FP4_ERR_UNSUPPORTED = -4, /* unknown enum/flag, bad combination, size limit */
  FP4_ERR_HIP = -5          /* a kernel launch failed */
};

/* Library version (FP4_VERSION of the build). */
int fp4_version(void);

/* Static description of a status code; never NULL. */
const char* fp4_status_string(int status);

/*
 * fp4_quantize -- block absmax -> scale -> round to E2M1 -> pack.
 *
 * MXFP4 ([TORQ] sec. 1 and the S-step of sec. 2(b)): block 32; the E8M0
 * exponent is the smallest e in [-127, 127] with amax <= 6 * 2^e (so the block
 * maximum maps onto the top code 6 without clipping; amax = 0 gives e = -127),
 * or floor(log2 amax) - 2 with FP4_FLAG_SCALE_OCP_FLOOR. Elements are
 * x * 2^-e exactly. A block holding Inf or NaN gets scale byte 0xFF and codes 0.
 *
 * MXINT4 ([TORQ] results, generalisation remark; the format as read in the
 * header conventions): block 32, E8M0 exponent the smallest e in [-127, 127]
 * with amax <= 1.75 * 2^e (capped at 127), or floor(log2 amax) with
 * FP4_FLAG_SCALE_OCP_FLOOR; k = the integer nearest 4 x 2^-e, ties to even,
 * clamped to [-7, 7] (-8 is never produced). Non-finite blocks as for MXFP4.
 *
 * NVFP4 ([RaZeR] sec. 1): block 16. Each step is one fp32 operation rounded to
 * nearest-even: s_t = amax_tensor / 2688 (2688 = 6 * 448; 1.0 if the tensor is
 * all zero) unless FP4_FLAG_TENSOR_SCALE_GIVEN; s_b = E4M3 nearest to
 * amax_block / (6 * s_t), saturating at 448 (a block whose s_b is 0 is stored
 * as scale 0, codes 0); s_eff = e4m3(s_b) * s_t; y = x * (1 / s_eff).
 * Non-finite NVFP4 inputs give unspecified codes.
 *
 * RaZeR mode ([RaZeR] sec. 2.2; NVFP4 only): per block, the code book is the
 * fifteen values other than -0 plus one special value at code 0x8, +5 or -5;
 * the block takes the one with the smaller sum of squared errors in y (equal:
 * +5), an element takes the special code only when strictly closer to it.
 *
 * RaZeR for weights (FP4_RAZER_W; [RaZeR] sec. 2.1 and 2.2; NVFP4 only):
 * the block scale is E3M3 (6 bits: bias 3, subnormals m 2^-5, largest 30,
 * no Inf/NaN; reading, the pages give the width only), s_t = amax / 180 (6 *
 * 30) unless given, and the two freed bits (scale byte bits 6-7) select code
 * 0x8's value among {+5, -5, +2.5, -2.5}; +-2.5, the second pair, is not on
 * the pages and was chosen offline as the best multiple of 0.5 on synthetic
 * LLM weights. The block takes the special of least squared error (ties: the
 * lower selector). Not available with rotation.
 *
 *  x_bf16       device, bf16 [rows, ld_x]; 16-byte aligned, ld_x % 8 == 0
 *  rows, cols   rows >= 0, cols >= 0, cols % block == 0; rows * cols / 8 < 2^31
 *  format       FP4_MXFP4, FP4_NVFP4 or FP4_MXINT4
 *  block        32 for MXFP4 and MXINT4, 16 for NVFP4
 *  mode         FP4_PLAIN, or FP4_RAZER / FP4_RAZER_W with NVFP4
 *  flags        FP4_FLAG_* bits valid for the format
 *  codes        device, uint8 [rows, ld_codes]; 4-byte aligned, ld_codes % 4 == 0,
 *               ld_codes >= cols / 2
 *  scales       device, uint8 [rows, ld_scales], ld_scales >= cols / block;
 *               with FP4_FLAG_SCALES_GEMM the GEMM order above (MXFP4)
 *  tensor_scale NVFP4: device fp32[1], written (or read with the flag);
 *               MXFP4, MXINT4: ignored, may be NULL
 *  stream       hipStream_t
 * Returns FP4_OK or an fp4_status. With NVFP4 and a computed s_t, three
 * kernels are enqueued (tensor amax, s_t, quantize) and the codes array also
 * carries the amax pass's per-work-group partial maxima until the quantize
 * kernel overwrites it; otherwise one kernel is enqueued.
 */
int fp4_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, int format,
                 int block, int mode, uint32_t flags, void* codes, int64_t ld_codes,
                 void* scales, int64_t ld_scales, float* tensor_scale, void* stream);

/*
 * fp4_dequantize -- decode codes and scales back to bf16.
 *
 * MXFP4, MXINT4: bf16(value * 2^e) (exact unless it overflows to Inf; scale
 * 0xFF gives NaN). NVFP4: bf16_rne(fp32(value * s_eff)); RaZeR mode decodes code
 * 0x8 to the block's special value, the decoder rebuilding it from the scale
 * byte's top bit ([RaZeR] sec. 2.3).
 * Optional inverse rotation so the result lies in the original basis: with
 * hadamard == block the block Hadamard is applied again (it is its own
 * inverse), then with perm != NULL element j is written to column perm[j].
 * The inverse-rotated values are computed in fp32 and rounded once to bf16:
 * the transform of the decoded grid values is exact, and the block scale
 * (MXFP4 2^e, NVFP4 s_eff) multiplies once, after it.
 * FP4_RAZER_W: s_eff = e3m3(byte & 63) * s_t and code 0x8 decodes to
 * {+5, -5, +2.5, -2.5}[byte >> 6] (no inverse rotation).
 *
 *  codes, scales, tensor_scale  as produced by fp4_quantize / fp4_rotate_quantize
 *  rows, cols, format, block, mode  as for fp4_quantize
 *  perm         NULL or device int32[cols], a permutation of 0..cols-1;
 *               requires cols <= 16384
 *  hadamard     0, or the block size (32 MXFP4/MXINT4, 16 NVFP4); with a
 *               rotation (perm or hadamard) cols % 32 == 0
 *  out_bf16     device, bf16 [rows, ld_out]; 16-byte aligned, ld_out % 8 == 0
 */
int fp4_dequantize(const void* codes, int64_t ld_codes, const void* scales, int64_t ld_scales,
                   const float* tensor_scale, int64_t rows, int64_t cols, int format,
                   int block, int mode, const int32_t* perm, int hadamard, void* out_bf16,
                   int64_t ld_out, void* stream);

/*
 * fp4_rotate_quantize -- two-level rotation fused with FP4 quantize + pack
 * ([TORQ] sec. 2(a) and 2(b); NVFP4: the generalisation remark of its results).
 *
 * Level 1: channel permutation x'[r, j] = x[r, perm[j]] (perm computed offline,
 * e.g. by fp4_build_permutation from fp4_channel_energy, so that every block
 * receives a balanced share of channel energy). Level 2: the orthonormal
 * Sylvester-Hadamard matrix H[i][j] = (-1)^popcount(i & j) / sqrt(n) inside
 * each n-block (n = block: 32 for MXFP4 and MXINT4, 16 for NVFP4), y = H x'
 * in fp32.
 * Then quantization of y exactly as in fp4_quantize, with every amax taken
 * over the fp32 y: the MX formats' shared exponent; NVFP4's block scales, RaZeR
 * choice and (unless FP4_FLAG_TENSOR_SCALE_GIVEN) s_t = amax(y) / 2688. With
 * a computed s_t three kernels are enqueued (rotation + amax partials held in
 * the code array, s_t, rotation + quantize); otherwise one.
 *
 *  perm         NULL (identity) or device int32[cols], a permutation of
 *               0..cols-1 (entries are clamped to cols-1); requires
 *               cols <= 32768 (rows up to 16384 wide are staged through
 *               registers, wider ones straight into LDS, one work-group per
 *               CU). A permutation made of aligned runs of 2, 4 or 8
 *               consecutive channels (fp4_build_permutation with group > 1)
 *               is detected and gathered with 4-, 8- or 16-byte LDS reads
 *  hadamard     the block size (32 MXFP4/MXINT4, 16 NVFP4) or 0 (none)
 *  format       FP4_MXFP4, FP4_MXINT4, or FP4_NVFP4 with mode FP4_PLAIN or
 *               FP4_RAZER
 *  cols         cols % 32 == 0
 *  rotated_out  NULL, or device fp32 [rows, ld_rot] receiving y; 16-byte
 *               aligned, ld_rot % 4 == 0 (for parity checks)
 *  others       as for fp4_quantize
 */
int fp4_rotate_quantize(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                        const int32_t* perm, int hadamard, int format, int block, int mode,
                        uint32_t flags, void* codes, int64_t ld_codes, void* scales,
                        int64_t ld_scales, float* tensor_scale, float* rotated_out,
                        int64_t ld_rot, void* stream);

/*
 * fp4_rotate_quantize_r -- the two-level rotation with a learned block matrix
 * in place of the Hadamard, fused with MXFP4 quantize + pack ([TORQ] sec.
 * 2(b): the rotation inside each block is learned, see
 * fp4_calibrate_block_rotation).
 *
 * x'[r, j] = x[r, perm[j]], then y = R x' on every 32-element block of x',
 * R the same 32x32 matrix for all blocks (fp32, products exact, sums in fp32),
 * then MXFP4 quantization of y as in fp4_quantize (default scale rule).
 *
 *  perm         device int32[cols], a permutation of 0..cols-1 (entries
 *               clamped to cols-1); required: pass the identity for none;
 *               cols <= 32768
 *  rotation     device fp32[32 * 32], R row-major (R[i][j] at 32 i + j),
 *               4-byte aligned; read once per work-group. Any matrix is
 *               accepted; fp4_dequantize_r inverts it only if orthogonal
 *  rotated_out  NULL, or device fp32 [rows, ld_rot] receiving y; 16-byte
 *               aligned, ld_rot % 4 == 0 (for parity checks)
 *  others       as for fp4_quantize with format FP4_MXFP4 (cols % 32 == 0)
 */
int fp4_rotate_quantize_r(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                          const int32_t* perm, const float* rotation, void* codes,
                          int64_t ld_codes, void* scales, int64_t ld_scales, float* rotated_out,
                          int64_t ld_rot, void* stream);

/*
 * fp4_dequantize_r -- inverse of fp4_rotate_quantize_r: MXFP4 decode (exact
 * in bf16), x' = R^T y per 32-element block (fp32 sums), then
 * out[r, perm[j]] = x'[r, j], rounded to bf16 (RNE). Arguments as for
 * fp4_dequantize with format FP4_MXFP4 and as for fp4_rotate_quantize_r.
 */
int fp4_dequantize_r(const void* codes, int64_t ld_codes, const void* scales, int64_t ld_scales,
                     int64_t rows, int64_t cols, const int32_t* perm, const float* rotation,
                     void* out_bf16, int64_t ld_out, void* stream);

/*
 * fp4_gemm -- C = A B^T on the quantized operands, the consumer of the path
 * ([RaZeR] sec. 2.3: GEMM kernels that take quantized weights and
 * activations, the special value rebuilt from the scale's metadata bit).
 *
 * A is [m, k] (e.g. activations) and B is [n, k] (e.g. weights, one row per
 * output channel), each exactly as fp4_quantize / fp4_rotate_quantize write
 * it: codes [rows, ld] (element 2i in the low nibble of byte i) and scale
 * bytes [rows, ld_s], one per block of k.
 *  - MXFP4: gfx950's scaled FP4 matrix instructions; every product of two
 *    elements is exact, the block scales 2^(e_a + e_b) apply per 32-element
 *    block pair, sums accumulate in fp32 (64 k at a time). A scale byte 0xFF
 *    (NaN) gives NaN in every output it reaches.
 *  - NVFP4 (mode_a / mode_b FP4_PLAIN or FP4_RAZER per operand): each element
 *    e2m1(code) * e4m3(scale) (RaZeR code 0x8: +-5 by the scale's bit 7) is
 *    decoded exactly to bf16 and multiplied on the bf16 matrix instructions
 *    (exact products, fp32 sums 16 k at a time); C = (ts_a ts_b) * sum, one
 *    fp32 rounding of the tensor-scale product and one of the result.
 *
 *  a_codes, b_codes     device, uint8; 16-byte aligned, ld % 16 == 0,
 *                       ld >= k / 2, 256 * ld < 2^31
 *  a_scales, b_scales   device, uint8; ld_s >= k / block, 256 * ld_s < 2^31;
 *                       MXFP4: 4-byte aligned, ld_s % 4 == 0; NVFP4: 2-byte
 *                       aligned, ld_s % 2 == 0 (bytes past k / block unused).
 *                       MXFP4 with FP4_FLAG_SCALES_GEMM in the operand's mode:
 *                       the GEMM order (ld_s the 32-row group stride, a
 *                       multiple of 256, >= 256 * ceil(k / 256)); each step of
 *                       256 k then reads 256 contiguous bytes per 32 rows
 *                       instead of 8 bytes from each of 32 rows
 *  a_ts, b_ts           NVFP4: device fp32[1] tensor scales; MXFP4: ignored
 *  mode_a, mode_b       FP4_PLAIN, or (NVFP4 only) FP4_RAZER; mode_b may also
 *                       be FP4_RAZER_W (E3M3 scale, four specials: weights);
 *                       MXFP4: FP4_PLAIN, optionally | FP4_FLAG_SCALES_GEMM
 *  m, n, k              >= 0, < 2^31; k % 32 == 0 (m or n zero: no work;
 *                       k zero: C = 0)
 *  format               FP4_MXFP4 or FP4_NVFP4
 *  out_dtype            FP4_OUT_F32 (c fp32) or FP4_OUT_BF16 (c bf16, RNE)
 *  c, ld_c              device, [m, ld_c], ld_c >= n, aligned to its element
 */
enum fp4_out_dtype { FP4_OUT_F32 = 0, FP4_OUT_BF16 = 1 };
int fp4_gemm(const void* a_codes, int64_t ld_a, const void* a_scales, int64_t ld_sa,
             const float* a_ts, int mode_a, const void* b_codes, int64_t ld_b,
             const void* b_scales, int64_t ld_sb, const float* b_ts, int mode_b, int64_t m,
             int64_t n, int64_t k, int format, int out_dtype, void* c, int64_t ld_c,
             void* stream);

/*
 * fp4_channel_energy -- calibration statistic for the permutation: energy[c] =
 * sum over rows of x[r, c]^2, accumulated in fp64 in a fixed order (the result
 * is deterministic) and rounded to fp32. It is the diagonal of the activation
 * second-moment matrix whose diagonal blocks hold the block variances that
 * [TORQ] sec. 2(a) equalises.
 *
 *  x_bf16   device, bf16 [rows, ld_x]; 16-byte aligned, ld_x % 8 == 0
 *  cols     cols % 32 == 0
 *  energy   device fp32[cols], 4-byte aligned (overwritten)
 */
int fp4_channel_energy(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                       float* energy, void* stream);

/*
 * fp4_build_permutation -- host-side, synchronous. Magnitude-balancing
 * permutation from channel energies (reading of [TORQ] sec. 2(a) as a
 * permutation). The unit moved is an aligned run of `group` channels with
 * energy the fp64 sum of its channels'. Units are taken in order of decreasing
 * energy (equal energies: lower index first); each goes to the next free slot
 * of the block whose accumulated energy (summed in fp64) is smallest among
 * blocks with a free slot (equal loads: lower block index), its channels kept
 * in order. group 1 balances single channels best; 2, 4 or 8 keep runs of
 * neighbouring channels together, which fp4_rotate_quantize gathers with one
 * 4-, 8- or 16-byte LDS read per run.
 *
 *  energy_host  host fp32[cols]
 *  cols         cols > 0, cols % block == 0
 *  block        32 (MXFP4) or 16 (NVFP4)
 *  group        1, 2, 4 or 8
 *  perm_host    host int32[cols]; perm[j] = source channel of column j
 */
int fp4_build_permutation(const float* energy_host, int64_t cols, int block, int group,
                          int32_t* perm_host);

/*
 * fp4_calibrate_block_rotation -- host-side, synchronous. Learns the 32x32
 * block matrix R of fp4_rotate_quantize_r on a calibration sample ([TORQ]
 * sec. 2(b)): alternating coordinate descent on the code-book occupancy
 * equilibrium loss L(R) = sum over the 8 E2M1 magnitudes c of
 * (p_c - 1/8)^2, p_c the fraction of elements of R x' (every block of every
 * row) that round to magnitude c under their block's MXFP4 scale.
 *  - start: R = H / sqrt(32), the orthonormal Sylvester-Hadamard matrix;
 *  - S-step: every block's shared exponent by the default MXFP4 rule, so the
 *    block maximum lands in the top binade of the code book;
 *  - R-step: one Givens rotation of output coordinates (i, j), i the
 *    coordinate whose own occupancy is farthest from uniform (largest sum of
 *    squared deviations), j the most complementary partner (smallest dot
 *    product of the two deviation vectors; ties: lowest index); the angle is
 *    the best of theta = k pi / (2 angles), k = 1 .. angles - 1 (the loss is
 *    piecewise constant in theta); taken only if it lowers the loss, else the
 *    pair is barred until the next accepted step.
 * `iters` R-steps are tried (fewer if every pair is barred). The result is
 * orthogonal up to fp64 rounding, then stored as fp32; the sample is
 * evaluated in fp64 (bf16 inputs are exact). Cost: about iters * angles *
 * rows * cols / 32 block evaluations on one host thread (30 steps of 32
 * angles on a 256 x 8192 sample take a few seconds), so calibrate on a
 * sample of rows.
 *
 *  x_host       host bf16 [rows, ld_x]; rows * cols <= 2^26
 *  cols         cols % 32 == 0
 *  perm_host    NULL (identity) or host int32[cols], the permutation that
 *               will be used online
 *  iters        >= 0 R-steps
 *  angles       2 .. 4096
 *  rotation_out host fp32[32 * 32], R row-major
 *  loss_out     NULL or host double[2]: L(H / sqrt(32)) and L(R)
 */
int fp4_calibrate_block_rotation(const uint16_t* x_host, int64_t rows, int64_t cols,
                                 int64_t ld_x, const int32_t* perm_host, int iters, int angles,
                                 float* rotation_out, double* loss_out);

/*
 * fp4_calibrate_macro_rotation -- host-side, synchronous. The inter-block
 * transform of [TORQ] sec. 2(a): an orthogonal transform, built from Givens
 * rotations, after which every block has the same variance. Readings: the
 * variance of a block is the sum over its channels of the second moment
 * sum_r x[r, j]^2 of the sample (after perm); the start is the permutation
 * (e.g. fp4_build_permutation's, which already balances most of it).
 * Each step takes the block p of largest and q of smallest variance
 * (ties: lowest index), moves t = min(V_p - mean, mean - V_q) from p to q with
 * one rotation (x_i, x_j) <- (c x_i - s x_j, s x_i + c x_j) of the channel i
 * of p with the largest second moment and the channel j of q with the
 * smallest (both not yet used in the current layer; ties: lowest index),
 * angle from the exact transfer equation with the pair's cross moment (the
 * whole of t, or as much as the pair can move). The sample is kept rotated in
 * fp64, so every step sees exact moments. Stops once
 * (max V - min V) <= tol * mean V, or after max_rot rotations. A full step
 * brings a block to the mean, so blocks - 1 steps suffice when no pair is
 * too weak. Rotations are grouped in layers of disjoint channel pairs.
 *
 *  x_host           host bf16 [rows, ld_x]; rows * cols <= 2^26
 *  perm_host        NULL (identity) or host int32[cols]
 *  block            32 or 16; cols % block == 0
 *  tol              >= 0, relative spread to reach
 *  max_rot          >= 0
 *  pairs_out        host int32[2 * max_rot]: (i, j) per rotation, in order
 *  cs_out           host fp32[2 * max_rot]: (cos, sin) per rotation
 *  layer_start_out  host int32[max_rot + 1]: layer L = rotations
 *                   layer_start[L] .. layer_start[L + 1] - 1
 *  n_rot_out, n_layers_out  host: counts written
 *  spread_out       NULL or host double[2]: (max V - min V) / mean V before,
 *                   and after the returned (fp32) rotations
 */
int fp4_calibrate_macro_rotation(const uint16_t* x_host, int64_t rows, int64_t cols,
                                 int64_t ld_x, const int32_t* perm_host, int block, double tol,
                                 int max_rot, int32_t* pairs_out, float* cs_out,
                                 int32_t* layer_start_out, int* n_rot_out, int* n_layers_out,
                                 double* spread_out);

/*
 * fp4_apply_channel_rotation -- the inter-block transform on every row of a
 * bf16 matrix ([TORQ] sec. 2(a)): z = x[r, perm[.]] in fp32, then each layer
 * of Givens rotations (x_i, x_j) <- (c x_i - s x_j, s x_i + c x_j), then
 * out[r, .] = bf16(z) (RNE). Rotations within a layer must touch disjoint
 * channels (as fp4_calibrate_macro_rotation writes them); they run in
 * parallel. For activations this yields the input of fp4_rotate_quantize /
 * fp4_rotate_quantize_r with perm = identity; for a consumer's weights W
 * [n, cols] (one row per output) the same call gives W' with W' z = W x, the
 * offline folding the pages describe.
 *
 *  x_bf16, out_bf16  device bf16 [rows, ld]; 16-byte aligned, ld % 8 == 0;
 *                    out may be x (in place) when ld_out == ld_x
 *  cols              cols % 8 == 0, cols <= 16384
 *  perm              NULL or device int32[cols] (entries clamped into the row)
 *  pairs, cs         device int32[2 n_rot], fp32[2 n_rot] (indices clamped)
 *  layer_start       device int32[n_layers + 1] (clamped to 0 .. n_rot)
 */
int fp4_apply_channel_rotation(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                               const int32_t* perm, const int32_t* pairs, const float* cs,
                               const int32_t* layer_start, int n_layers, int n_rot,
                               void* out_bf16, int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4_H */
