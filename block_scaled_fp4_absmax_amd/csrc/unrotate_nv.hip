// unrotate_nv.hip -- NVFP4 (+RaZeR) dequantization with the inverse rotation
// (16-point Hadamard; kernel in unrotate_kernels.hpp).
#include "unrotate_kernels.hpp"

namespace fp4 {

void launch_nv_dequant_unrotate(const Shape& s, const int32_t* perm, int hadamard, bool razer,
                                const void* codes, const void* scales, const float* ts, void* out,
                                hipStream_t st) {
  const RotGeom g = rot_geom(s, 0, 16);
  auto c = static_cast<const uint8_t*>(codes);
  auto sc = static_cast<const uint8_t*>(scales);
  auto o = static_cast<uint16_t*>(out);
  if (razer) unrot_variants<1, true>(s, perm, hadamard != 0, c, sc, ts, o, g, st);
  else unrot_variants<1, false>(s, perm, hadamard != 0, c, sc, ts, o, g, st);
}

}  // namespace fp4
