// perm.cpp -- host-side magnitude-balancing permutation (offline calibration).
//
// Reading of "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
// technical summary sec. 2(a) -- an orthogonal transform that makes every
// block's variance equal -- restricted to channel permutations: channels are
// placed largest energy first, each into the open block (fewer than `block`
// channels so far) of least accumulated energy. The unit placed is an aligned
// run of `group` channels (1, 2, 4 or 8): runs let the permuting kernel gather
// 2 * group bytes per LDS read. A binary heap keyed by (load, block index)
// finds that block in O(log B).
#include <stdint.h>

#include <algorithm>
#include <numeric>
#include <queue>
#include <vector>

#include "../../include/fp4.h"

extern "C" int fp4_build_permutation(const float* energy_host, int64_t cols, int block,
                                     int group, int32_t* perm_host) {
  if (!energy_host || !perm_host) return FP4_ERR_NULL;
  if (block != 16 && block != 32) return FP4_ERR_UNSUPPORTED;
  if (group != 1 && group != 2 && group != 4 && group != 8) return FP4_ERR_UNSUPPORTED;
  if (cols <= 0 || cols % block != 0) return FP4_ERR_SHAPE;
  if (cols > INT32_MAX) return FP4_ERR_UNSUPPORTED;
  const int64_t nblk = cols / block, nunit = cols / group, slots = block / group;

  // unit energy: the sum of its channels' energies in fp64, in channel order
  std::vector<double> ue(static_cast<size_t>(nunit), 0.0);
  for (int64_t u = 0; u < nunit; ++u)
    for (int i = 0; i < group; ++i) ue[u] += static_cast<double>(energy_host[u * group + i]);

  std::vector<int32_t> order(static_cast<size_t>(nunit));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return ue[a] > ue[b]; });  // ties keep index order

  struct Bin {
    double load;
    int64_t idx;
  };
  auto later = [](const Bin& a, const Bin& b) {  // min-heap on (load, idx)
    return a.load > b.load || (a.load == b.load && a.idx > b.idx);
  };
  std::priority_queue<Bin, std::vector<Bin>, decltype(later)> open(later);
  for (int64_t b = 0; b < nblk; ++b) open.push(Bin{0.0, b});
  std::vector<int64_t> fill(static_cast<size_t>(nblk), 0);

  for (int32_t u : order) {
    Bin top = open.top();
    open.pop();
    const int64_t pos = top.idx * block + fill[top.idx] * group;
    for (int i = 0; i < group; ++i) perm_host[pos + i] = static_cast<int32_t>(u * group + i);
    fill[top.idx] += 1;
    top.load += ue[u];
    if (fill[top.idx] < slots) open.push(top);
  }
  return FP4_OK;
}
