// rotate_nv.hip -- NVFP4 (+RaZeR) after the two-level rotation with the
// 16-point Hadamard (kernels in rotate_kernels.hpp).
#include "rotate_kernels.hpp"

namespace fp4 {

template <bool kHad, bool kRazer, bool kRot, bool kAmax>
static int nv_stream_launch(const uint16_t* x, uint8_t* c, uint8_t* sc, const float* ts,
                            float* rot, const RotGeom& g, bool flat, hipStream_t st) {
  const uint64_t tiles = ((uint64_t)g.nblk + 31) / 32;
  const int grid = (int)((tiles + kWaves * kTiles - 1) / (kWaves * kTiles));
  if (flat)
    hipLaunchKernelGGL((nv_rotq_stream_kernel<true, kHad, kRazer, kRot, kAmax>), dim3(grid),
                       dim3(kThreads), 0, st, x, c, sc, ts, rot, g);
  else
    hipLaunchKernelGGL((nv_rotq_stream_kernel<false, kHad, kRazer, kRot, kAmax>), dim3(grid),
                       dim3(kThreads), 0, st, x, c, sc, ts, rot, g);
  return grid;
}

template <bool kHad, bool kRazer, bool kRot>
static void nv_rotq(const Shape& s, const int32_t* perm, bool scale_given, const uint16_t* x,
                    uint8_t* c, uint8_t* sc, float* ts, float* rot, const RotGeom& g, bool flat,
                    hipStream_t st) {
  if (!scale_given) {  // s_t from the largest rotated magnitude
    const int nparts = perm ? perm_dispatch<kFmtNvAmax, kHad, false, false>(s, perm, x, c, sc,
                                                                             nullptr, nullptr, g, st)
                            : nv_stream_launch<kHad, false, false, true>(x, c, sc, nullptr,
                                                                        nullptr, g, flat, st);
    launch_nv_scale_from_partials(s, c, (uint32_t)nparts, ts, st);
  }
  if (perm)
    (void)perm_dispatch<kFmtNv, kHad, kRazer, kRot>(s, perm, x, c, sc, ts, rot, g, st);
  else
    (void)nv_stream_launch<kHad, kRazer, kRot, false>(x, c, sc, ts, rot, g, flat, st);
}

void launch_nv_rotate_quant(const Shape& s, const int32_t* perm, int hadamard, bool razer,
                            bool scale_given, const void* x, void* codes, void* scales,
                            float* ts, float* rot, int64_t ld_rot, hipStream_t st) {
  if (s.rows == 0 || s.cols == 0) {  // nothing to quantize; a computed s_t is 1
    if (!scale_given) launch_nv_scale_from_partials(s, codes, 0, ts, st);
    return;
  }
  RotGeom g = rot_geom(s, ld_rot, 16);
  auto xp = static_cast<const uint16_t*>(x);
  auto cp = static_cast<uint8_t*>(codes);
  auto sp = static_cast<uint8_t*>(scales);
  const bool had = hadamard != 0, r = rot != nullptr;
  const bool flat = s.ld_x == s.cols && s.ld_c == s.cols / 2 && s.ld_s == s.cols / 16 &&
                    (!r || ld_rot == s.cols);
  if (had && razer && r) nv_rotq<true, true, true>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (had && razer && !r) nv_rotq<true, true, false>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (had && !razer && r) nv_rotq<true, false, true>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (had && !razer && !r) nv_rotq<true, false, false>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (!had && razer && r) nv_rotq<false, true, true>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (!had && razer && !r) nv_rotq<false, true, false>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (!had && !razer && r) nv_rotq<false, false, true>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
  if (!had && !razer && !r) nv_rotq<false, false, false>(s, perm, scale_given, xp, cp, sp, ts, rot, g, flat, st);
}

}  // namespace fp4
