// split_k.hpp -- work-group tiles of the split-K GEMM kernels (MXFP4 and
// NVFP4): the XCD-aware work-group -> tile map and the per-product choice of
// tile shape.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace fp4 {

// Work-group -> (column tile x, row tile y) of a skinny product with gx x gy
// tiles of 32 x 32 on a grid of skinny_grid(gx, gy) work-groups. Work-groups
// are dealt to the 8 XCDs in turn, so the ids of one column tile are made
// congruent mod 8: all row tiles of a column tile run on one XCD and read
// their shared B rows through one L2. x >= gx marks a padding work-group.
struct SkinnyTile {
  int32_t x, y;
};
__device__ __forceinline__ SkinnyTile skinny_tile(uint32_t id, int32_t gy) {
  const int32_t q = (int32_t)(id >> 3);
  return SkinnyTile{(q / gy) * 8 + (int32_t)(id & 7u), q % gy};
}
inline unsigned skinny_grid(int64_t gx, int64_t gy) {
  return (unsigned)(((gx + 7) / 8) * 8 * gy);
}

// Work-group tile of a split-K product: MT 32-row pieces of A by NT of B.
// {0, 0} selects the 128 x 128 tiles instead. The choice minimises the
// operand pieces (32 rows by K) each CU streams through its vector caches,
// which bound the MXFP4 products (about 30 GB/s per CU measured for both
// kernels) and, through the decode per piece, the NVFP4 ones: a work-group
// reads MT + NT pieces, a CU runs ceil(work-groups / CUs) of them; a 128 x 128
// tile counts as tile_pieces (8 pieces for MXFP4; 10 for NVFP4, whose
// four-wave tiles decode more slowly, as measured). Ties keep the earlier
// candidate.
struct SkinnyShape {
  int mt, nt;
};
inline SkinnyShape skinny_shape(int64_t m, int64_t n, int64_t cus, int64_t max_m,
                                int64_t tile_pieces) {
  if (m > max_m) return {0, 0};
  const auto per_cu = [&](int64_t wg) { return (wg + cus - 1) / cus; };
  SkinnyShape best{0, 0};
  int64_t best_cost = per_cu(((m + 127) / 128) * ((n + 127) / 128)) * tile_pieces;
  constexpr SkinnyShape kShapes[] = {{1, 1}, {1, 2}, {2, 2}};
  for (const SkinnyShape& s : kShapes) {
    const int64_t wg = ((m + 32 * s.mt - 1) / (32 * s.mt)) * ((n + 32 * s.nt - 1) / (32 * s.nt));
    const int64_t c = per_cu(wg) * (s.mt + s.nt);
    if (c < best_cost) {
      best = s;
      best_cost = c;
    }
  }
  return best;
}

}  // namespace fp4
