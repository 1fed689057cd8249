// unrotate_int.hip -- MXINT4 dequantization with the inverse rotation (kernel
// in unrotate_kernels.hpp).
#include "unrotate_kernels.hpp"

namespace fp4 {

void mxint_dequant_unrotate(const Shape& s, const int32_t* perm, bool hadamard,
                            const uint8_t* codes, const uint8_t* scales, uint16_t* out,
                            const RotGeom& g, hipStream_t st) {
  unrot_variants<2, false>(s, perm, hadamard, codes, scales, nullptr, out, g, st);
}

}  // namespace fp4
