// calib.cpp -- host-side calibration of the learned intra-block rotation
// (offline).
//
// "TORQ: Two-Level Orthogonal Rotation for MXFP4 Quantization", technical
// summary sec. 2(b): the rotation inside each block is learned by alternating
// coordinate descent on a code-book occupancy-equilibrium loss, which measures
// how far the empirical use of the MXFP4 codes is from uniform. The S-step
// sets every block's scale so its largest magnitude maps onto the top code;
// the R-step updates the orthogonal block matrix with a Givens rotation of
// two coordinates, picked by a heuristic among badly balanced, statistically
// complementary pairs, at the angle that minimizes the loss over a finite set
// (the loss is piecewise constant in the angle).
//
// Readings where the summary is silent (stated again in the header): one
// matrix shared by all 32-element blocks, started from the orthonormal
// Hadamard; occupancy = fraction of elements per E2M1 magnitude index (8
// bins, nearest value, ties to the even index) after the MXFP4 scale rule;
// loss = sum over bins of (fraction - 1/8)^2; the pair is the coordinate
// whose own occupancy is farthest from uniform, with the partner whose
// deviation from uniform is most anti-correlated with it; angles k pi / (2A),
// k = 1 .. A - 1; a step that does not lower the loss is rejected and its
// pair is not tried again until a step succeeds.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/fp4.h"

namespace {

constexpr int kN = 32;

// E2M1 magnitude index nearest to a >= 0, ties to the even index.
inline int bin_of(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

// MXFP4 shared exponent: the smallest e in [-127, 127] with amax <= 6 * 2^e.
inline int e8m0_exp(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = ilogb(amax) - 2;
  if (amax > ldexp(6.0, e)) ++e;
  return std::min(127, std::max(-127, e));
}

inline float bf16_to_f32(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

struct State {
  int64_t nb = 0;                 // blocks in the sample
  std::vector<double> y;          // [nb][32] rotated values
  std::vector<int> e;             // [nb] block exponents
  std::vector<uint8_t> bin;       // [nb][32]
  double hist[8] = {0};           // total counts
  double coord[kN][8] = {{0}};    // counts per coordinate

  void rescan(int64_t b) {
    double amax = 0.0;
    for (int k = 0; k < kN; ++k) amax = std::max(amax, fabs(y[b * kN + k]));
    e[b] = e8m0_exp(amax);
    for (int k = 0; k < kN; ++k) bin[b * kN + k] = (uint8_t)bin_of(ldexp(fabs(y[b * kN + k]), -e[b]));
  }
  // y = R x' for every block, then the S-step and the counts
  void apply(const std::vector<double>& R, const std::vector<double>& xp) {
    y.assign(nb * kN, 0.0);
    for (int64_t b = 0; b < nb; ++b) {
      for (int i = 0; i < kN; ++i) {
        double acc = 0.0;
        for (int k = 0; k < kN; ++k) acc += R[i * kN + k] * xp[b * kN + k];
        y[b * kN + i] = acc;
      }
      rescan(b);
    }
    count();
  }
  void count() {
    std::fill(hist, hist + 8, 0.0);
    for (auto& c : coord) std::fill(c, c + 8, 0.0);
    for (int64_t b = 0; b < nb; ++b)
      for (int k = 0; k < kN; ++k) {
        hist[bin[b * kN + k]] += 1.0;
        coord[k][bin[b * kN + k]] += 1.0;
      }
  }
  double loss_of(const double* h) const {
    const double n = (double)(nb * kN);
    double l = 0.0;
    for (int c = 0; c < 8; ++c) l += (h[c] / n - 0.125) * (h[c] / n - 0.125);
    return l;
  }
};

// Loss after rotating coordinates i, j of every block by (c, s); omax[b] is
// the largest magnitude of the block's other coordinates.
double trial_loss(const State& st, int i, int j, double c, double s,
                  const std::vector<double>& omax) {
  double h[8];
  std::copy(st.hist, st.hist + 8, h);
  for (int64_t b = 0; b < st.nb; ++b) {
    const double* yb = &st.y[b * kN];
    const double ni = c * yb[i] - s * yb[j], nj = s * yb[i] + c * yb[j];
    const int e = e8m0_exp(std::max(omax[b], std::max(fabs(ni), fabs(nj))));
    const uint8_t* bb = &st.bin[b * kN];
    if (e == st.e[b]) {
      h[bb[i]] -= 1.0;
      h[bb[j]] -= 1.0;
      h[bin_of(ldexp(fabs(ni), -e))] += 1.0;
      h[bin_of(ldexp(fabs(nj), -e))] += 1.0;
    } else {
      for (int k = 0; k < kN; ++k) {
        h[bb[k]] -= 1.0;
        const double v = k == i ? ni : k == j ? nj : yb[k];
        h[bin_of(ldexp(fabs(v), -e))] += 1.0;
      }
    }
  }
  return st.loss_of(h);
}

}  // namespace

extern "C" int fp4_calibrate_block_rotation(const uint16_t* x_host, int64_t rows, int64_t cols,
                                            int64_t ld_x, const int32_t* perm_host, int iters,
                                            int angles, float* rotation_out, double* loss_out) {
  if (!x_host || !rotation_out) return FP4_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % kN != 0 || ld_x < cols) return FP4_ERR_SHAPE;
  if (iters < 0 || angles < 2 || angles > 4096) return FP4_ERR_UNSUPPORTED;
  if (rows * cols > ((int64_t)1 << 26)) return FP4_ERR_UNSUPPORTED;  // a sample, not a model

  // R = H / sqrt(32) rounded to fp32 (the form the kernels read), row-major
  std::vector<double> R(kN * kN);
  for (int i = 0; i < kN; ++i)
    for (int j = 0; j < kN; ++j)
      R[i * kN + j] = (double)(float)((__builtin_popcount((unsigned)(i & j)) & 1 ? -1.0 : 1.0) /
                                      sqrt(32.0));
  const std::vector<double> R0 = R;

  State st;
  st.nb = rows * (cols / kN);
  st.e.assign(st.nb, 0);
  st.bin.assign(st.nb * kN, 0);
  std::vector<double> xp(st.nb * kN);  // the permuted sample, block by block
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b0 = 0; b0 < cols; b0 += kN)
      for (int k = 0; k < kN; ++k) {
        const int64_t src = perm_host ? perm_host[b0 + k] : b0 + k;
        if (src < 0 || src >= cols) return FP4_ERR_SHAPE;
        xp[(r * (cols / kN) + b0 / kN) * kN + k] = (double)bf16_to_f32(x_host[r * ld_x + src]);
      }
  st.apply(R, xp);
  const double loss0 = st.loss_of(st.hist);
  double loss = loss0;
  if (loss_out) loss_out[0] = loss0;

  const double n = (double)st.nb;
  std::vector<uint8_t> tabu(kN * kN, 0);
  std::vector<double> omax(st.nb);
  for (int it = 0; it < iters; ++it) {
    // per-coordinate deviation from uniform occupancy
    double dev[kN][8], imb[kN];
    for (int k = 0; k < kN; ++k) {
      imb[k] = 0.0;
      for (int c = 0; c < 8; ++c) {
        dev[k][c] = st.coord[k][c] / n - 0.125;
        imb[k] += dev[k][c] * dev[k][c];
      }
    }
    int bi = -1, bj = -1;
    double best_imb = -1.0, best_dot = 0.0;
    for (int i = 0; i < kN; ++i) {
      for (int j = 0; j < kN; ++j) {
        if (j == i || tabu[i * kN + j]) continue;
        double dot = 0.0;
        for (int c = 0; c < 8; ++c) dot += dev[i][c] * dev[j][c];
        if (imb[i] > best_imb || (imb[i] == best_imb && dot < best_dot)) {
          best_imb = imb[i];
          best_dot = dot;
          bi = i;
          bj = j;
        }
      }
    }
    if (bi < 0) break;  // every pair tried without gain
    for (int64_t b = 0; b < st.nb; ++b) {
      double m = 0.0;
      for (int k = 0; k < kN; ++k)
        if (k != bi && k != bj) m = std::max(m, fabs(st.y[b * kN + k]));
      omax[b] = m;
    }
    double best_loss = loss, bc = 1.0, bs = 0.0;
    for (int a = 1; a < angles; ++a) {
      const double th = a * (M_PI / 2.0) / angles, c = cos(th), s = sin(th);
      const double l = trial_loss(st, bi, bj, c, s, omax);
      if (l < best_loss) {
        best_loss = l;
        bc = c;
        bs = s;
      }
    }
    if (!(best_loss < loss)) {
      tabu[bi * kN + bj] = tabu[bj * kN + bi] = 1;
      continue;
    }
    // accept: rotate rows bi, bj of R and coordinates bi, bj of every block
    for (int k = 0; k < kN; ++k) {
      const double ri = R[bi * kN + k], rj = R[bj * kN + k];
      R[bi * kN + k] = bc * ri - bs * rj;
      R[bj * kN + k] = bs * ri + bc * rj;
    }
    for (int64_t b = 0; b < st.nb; ++b) {
      double* yb = &st.y[b * kN];
      const double yi = yb[bi], yj = yb[bj];
      yb[bi] = bc * yi - bs * yj;
      yb[bj] = bs * yi + bc * yj;
      st.rescan(b);
    }
    st.count();
    loss = st.loss_of(st.hist);
    std::fill(tabu.begin(), tabu.end(), 0);
  }
  // the matrix returned is R rounded to fp32; its loss is evaluated afresh,
  // and the start is returned instead should the rounding have undone the gain
  for (int k = 0; k < kN * kN; ++k) R[k] = (double)(float)R[k];
  if (loss < loss0) {
    st.apply(R, xp);
    loss = st.loss_of(st.hist);
  }
  if (!(loss < loss0)) {
    R = R0;
    loss = loss0;
  }
  for (int k = 0; k < kN * kN; ++k) rotation_out[k] = (float)R[k];
  if (loss_out) loss_out[1] = loss;
  return FP4_OK;
}
