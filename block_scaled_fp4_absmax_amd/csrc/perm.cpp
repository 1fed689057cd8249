// perm.cpp -- host-side magnitude-balancing permutation (offline calibration).
//
// Reading of "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization",
// technical summary sec. 2(a) -- an orthogonal transform that makes every
// block's variance equal -- restricted to channel permutations: channels are
// placed largest energy first, each into the open block (fewer than `block`
// channels so far) of least accumulated energy. A binary heap keyed by
// (load, block index) finds that block in O(log B).
#include <stdint.h>

#include <algorithm>
#include <numeric>
#include <queue>
#include <vector>

#include "../../include/fp4.h"

extern "C" int fp4_build_permutation(const float* energy_host, int64_t cols, int block,
                                     int32_t* perm_host) {
  if (!energy_host || !perm_host) return FP4_ERR_NULL;
  if (block != 16 && block != 32) return FP4_ERR_UNSUPPORTED;
  if (cols <= 0 || cols % block != 0) return FP4_ERR_SHAPE;
  if (cols > INT32_MAX) return FP4_ERR_UNSUPPORTED;
  const int64_t nblk = cols / block;

  std::vector<int32_t> order(static_cast<size_t>(cols));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return energy_host[a] > energy_host[b];  // equal energies keep index order
  });

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

  for (int32_t c : order) {
    Bin top = open.top();
    open.pop();
    perm_host[top.idx * block + fill[top.idx]] = c;
    fill[top.idx] += 1;
    top.load += static_cast<double>(energy_host[c]);
    if (fill[top.idx] < block) open.push(top);
  }
  return FP4_OK;
}
