// rotate_mx.hip -- MXFP4 after the two-level rotation (kernels in
// rotate_kernels.hpp; MXINT4 in rotate_int.hip).
#include "rotate_kernels.hpp"

namespace fp4 {

void launch_mx_rotate_quant(const Shape& s, const int32_t* perm, int hadamard, bool floor_rule,
                            bool mxint, const void* x, void* codes, void* scales, float* rot,
                            int64_t ld_rot, hipStream_t st) {
  RotGeom g = rot_geom(s, ld_rot);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / 32 &&
                    !s.s_gemm && (!rot || ld_rot == s.cols);
  if (mxint)
    mxint_rotate_quant(s, perm, hadamard != 0, floor_rule, xp, cp, sp, rot, g, flat, st);
  else
    mx_rotq_variants<false>(s, perm, hadamard != 0, floor_rule, xp, cp, sp, rot, g, flat, st);
}

}  // namespace fp4
