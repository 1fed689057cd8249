// rotate_mat.hip -- MXFP4 after the permutation and a learned 32x32 block
// matrix ("TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
// technical summary sec. 2(b): the intra-block rotation is learned), kernels
// in rotate_kernels.hpp.
#include "rotate_kernels.hpp"

namespace fp4 {

void launch_mx_matrix_rotate_quant(const Shape& s, const int32_t* perm, const float* rmat,
                                   const void* x, void* codes, void* scales, float* rot,
                                   int64_t ld_rot, hipStream_t st) {
  const RotGeom g = rot_geom(s, ld_rot);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  if (rot)
    (void)perm_dispatch<kFmtMxMat, true, false, true>(s, perm, xp, cp, sp, rmat, rot, g, st);
  else
    (void)perm_dispatch<kFmtMxMat, true, false, false>(s, perm, xp, cp, sp, rmat, rot, g, st);
}

}  // namespace fp4
