// rotate_int.hip -- MXINT4 after the two-level rotation (kernels in
// rotate_kernels.hpp).
#include "rotate_kernels.hpp"

namespace fp4 {

void mxint_rotate_quant(const Shape& s, const int32_t* perm, bool had, bool floor_rule,
                        const uint16_t* x, uint8_t* codes, uint8_t* scales, float* rot,
                        const RotGeom& g, bool flat, hipStream_t st) {
  mx_rotq_variants<true>(s, perm, had, floor_rule, x, codes, scales, rot, g, flat, st);
}

}  // namespace fp4
