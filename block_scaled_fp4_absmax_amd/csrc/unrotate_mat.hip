// unrotate_mat.hip -- MXFP4 dequantization with the inverse of the learned
// block matrix and of the permutation (kernel in unrotate_kernels.hpp).
#include "unrotate_kernels.hpp"

namespace fp4 {

void launch_mx_matrix_dequant_unrotate(const Shape& s, const int32_t* perm, const float* rmat,
                                       const void* codes, const void* scales, void* out,
                                       hipStream_t st) {
  unrot_dispatch<3, false, true, true>(s, perm, static_cast<const uint8_t*>(codes),
                                       static_cast<const uint8_t*>(scales), rmat,
                                       static_cast<uint16_t*>(out), rot_geom(s, 0), st);
}

}  // namespace fp4
