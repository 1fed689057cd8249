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
#include <thread>
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
    // the angles are independent: evaluated on several host threads (each
    // loss is a sum of integer counts, so the result does not depend on the
    // split), then the first strictly best one is taken in angle order
    std::vector<double> la(angles, 0.0);
    const int nth = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> pool;
    for (int t = 0; t < nth; ++t)
      pool.emplace_back([&, t]() {
        for (int a = 1 + t; a < angles; a += nth) {
          const double th = a * (M_PI / 2.0) / angles;
          la[a] = trial_loss(st, bi, bj, cos(th), sin(th), omax);
        }
      });
    for (auto& th : pool) th.join();
    double best_loss = loss, bc = 1.0, bs = 0.0;
    for (int a = 1; a < angles; ++a) {
      if (la[a] < best_loss) {
        const double th = a * (M_PI / 2.0) / angles;
        best_loss = la[a];
        bc = cos(th);
        bs = sin(th);
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

// ---------------------------------------------------------------------------
// Inter-block transform ("TORQ: Two-Level Orthogonal Rotation for MXFP4
// Quantization", technical summary sec. 2(a)): an orthogonal transform that
// makes every block's variance the same, built by iterated Givens rotations.
// Reading: block variance = sum over the block's channels of the second
// moment sum_r x[r, j]^2 on the sample (after the permutation). Each step
// takes the block p of largest and q of smallest variance and moves
// t = min(V_p - mean, mean - V_q) from p to q with one rotation of channel i
// (largest second moment in p) and channel j (smallest in q), whose angle
// solves the exact transfer equation with the pair's cross moment; a step
// that cannot move all of t (the pair is too weak) moves what it can. So each
// full step brings one block to the mean: at most (blocks - 1) full steps.
// Channels are used once per layer, so the rotations of one layer are
// disjoint and can be applied in parallel.
namespace {

struct Macro {
  int64_t rows, cols;
  int block;
  std::vector<double> X;  // [cols][rows], the permuted sample, column-major
  std::vector<double> E;  // [cols] second moments
  std::vector<double> V;  // [blocks]

  double* col(int64_t j) { return &X[j * rows]; }
  void moment(int64_t j) {
    const double* c = col(j);
    double e = 0.0;
    for (int64_t r = 0; r < rows; ++r) e += c[r] * c[r];
    E[j] = e;
  }
  void block_sum(int64_t b) {
    double v = 0.0;
    for (int k = 0; k < block; ++k) v += E[b * block + k];
    V[b] = v;
  }
  void rotate(int64_t i, int64_t j, double c, double s) {
    double* xi = col(i);
    double* xj = col(j);
    for (int64_t r = 0; r < rows; ++r) {
      const double a = xi[r], b = xj[r];
      xi[r] = c * a - s * b;
      xj[r] = s * a + c * b;
    }
    moment(i);
    moment(j);
  }
  double spread() const {
    double lo = V[0], hi = V[0], sum = 0.0;
    for (double v : V) {
      lo = std::min(lo, v);
      hi = std::max(hi, v);
      sum += v;
    }
    const double mean = sum / (double)V.size();
    return mean > 0.0 ? (hi - lo) / mean : 0.0;
  }
};

void load_sample(Macro& m, const uint16_t* x, int64_t ld_x, const int32_t* perm) {
  m.X.assign(m.cols * m.rows, 0.0);
  for (int64_t r = 0; r < m.rows; ++r)
    for (int64_t j = 0; j < m.cols; ++j)
      m.X[j * m.rows + r] = (double)bf16_to_f32(x[r * ld_x + (perm ? perm[j] : j)]);
  m.E.assign(m.cols, 0.0);
  for (int64_t j = 0; j < m.cols; ++j) m.moment(j);
  m.V.assign(m.cols / m.block, 0.0);
  for (int64_t b = 0; b < (int64_t)m.V.size(); ++b) m.block_sum(b);
}

}  // namespace

extern "C" int fp4_calibrate_macro_rotation(const uint16_t* x_host, int64_t rows, int64_t cols,
                                            int64_t ld_x, const int32_t* perm_host, int block,
                                            double tol, int max_rot, int32_t* pairs_out,
                                            float* cs_out, int32_t* layer_start_out,
                                            int* n_rot_out, int* n_layers_out,
                                            double* spread_out) {
  if (!x_host || !n_rot_out || !n_layers_out || !layer_start_out) return FP4_ERR_NULL;
  if (max_rot > 0 && (!pairs_out || !cs_out)) return FP4_ERR_NULL;
  if (block != 16 && block != 32) return FP4_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || cols % block != 0 || ld_x < cols) return FP4_ERR_SHAPE;
  if (max_rot < 0 || !(tol >= 0.0)) return FP4_ERR_UNSUPPORTED;
  if (rows * cols > ((int64_t)1 << 26)) return FP4_ERR_UNSUPPORTED;  // a sample, not a model
  if (perm_host)
    for (int64_t j = 0; j < cols; ++j)
      if (perm_host[j] < 0 || perm_host[j] >= cols) return FP4_ERR_SHAPE;

  Macro m;
  m.rows = rows;
  m.cols = cols;
  m.block = block;
  load_sample(m, x_host, ld_x, perm_host);
  const int64_t nb = cols / block;
  if (spread_out) spread_out[0] = m.spread();

  std::vector<uint8_t> used(cols, 0);
  int n = 0, layers = 0;
  layer_start_out[0] = 0;
  bool layer_open = false;
  while (n < max_rot && m.spread() > tol) {
    // the mean is taken afresh: the fp32 (cos, sin) kept below are orthogonal
    // only to about 2^-24, so the total moves a little with every step
    double total = 0.0;
    int64_t p = 0, q = 0;
    for (int64_t b = 0; b < nb; ++b) {
      total += m.V[b];
      if (m.V[b] > m.V[p]) p = b;
      if (m.V[b] < m.V[q]) q = b;
    }
    const double mean = total / (double)nb;
    const double t_want = std::min(m.V[p] - mean, mean - m.V[q]);
    // the pair: free channels of p (largest moment) and q (smallest); if
    // they cannot move all of t, or none is free, a new layer frees them all
    int64_t i = -1, j = -1;
    double C = 0.0, A = 0.0, rad = 0.0, t_max = 0.0;
    auto pick = [&]() {
      i = j = -1;
      for (int k = 0; k < block; ++k) {
        const int64_t a = p * block + k, b = q * block + k;
        if (!used[a] && (i < 0 || m.E[a] > m.E[i])) i = a;
        if (!used[b] && (j < 0 || m.E[b] < m.E[j])) j = b;
      }
      if (i < 0 || j < 0) return;
      // moment moved into j by the rotation of angle phi / 2:
      //   A (1 - cos phi) + C sin phi = A - rad cos(phi + beta),
      // A = (E_i - E_j) / 2, C = cross moment, rad = |(A, C)|, beta = atan2(C, A);
      // at most A + rad
      const double* xi = m.col(i);
      const double* xj = m.col(j);
      C = 0.0;
      for (int64_t r = 0; r < rows; ++r) C += xi[r] * xj[r];
      A = 0.5 * (m.E[i] - m.E[j]);
      rad = std::hypot(A, C);
      t_max = A + rad;
    };
    pick();
    if ((i < 0 || j < 0 || t_max < t_want) && layer_open && n > layer_start_out[layers]) {
      std::fill(used.begin(), used.end(), 0);
      layer_start_out[++layers] = n;
      pick();
    }
    if (i < 0 || j < 0 || !(t_max > 0.0)) break;  // no pair can move anything
    layer_open = true;
    const double t = std::min(t_want, t_max);
    const double beta = std::atan2(C, A);
    const double arg = std::max(-1.0, std::min(1.0, (A - t) / rad));
    const double phi = std::acos(arg) - beta;
    // the sample follows the rotation exactly as returned (fp32 cos, sin)
    const float c = (float)std::cos(0.5 * phi), s = (float)std::sin(0.5 * phi);
    m.rotate(i, j, (double)c, (double)s);
    m.block_sum(p);
    m.block_sum(q);
    used[i] = used[j] = 1;
    pairs_out[2 * n] = (int32_t)i;
    pairs_out[2 * n + 1] = (int32_t)j;
    cs_out[2 * n] = c;
    cs_out[2 * n + 1] = s;
    ++n;
  }
  if (layer_open && layer_start_out[layers] < n) ++layers;  // close the last, non-empty layer
  layer_start_out[layers] = n;
  *n_rot_out = n;
  *n_layers_out = layers;
  if (spread_out) {  // the spread the returned (fp32) rotations reach, evaluated afresh
    load_sample(m, x_host, ld_x, perm_host);
    for (int k = 0; k < n; ++k) {
      m.rotate(pairs_out[2 * k], pairs_out[2 * k + 1], (double)cs_out[2 * k],
               (double)cs_out[2 * k + 1]);
    }
    for (int64_t b = 0; b < nb; ++b) m.block_sum(b);
    spread_out[1] = m.spread();
  }
  return FP4_OK;
}
