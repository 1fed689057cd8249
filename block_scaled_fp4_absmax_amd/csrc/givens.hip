// givens.hip -- the inter-block transform on every row: permutation, then
// layers of disjoint Givens rotations of channel pairs ("TORQ: Two-Level
// Orthogonal Rotation for MXFP4 Quantization", technical summary sec. 2(a):
// an orthogonal transform built from Givens rotations that evens out the
// block variances). The same call folds the transform into the rows of a
// consumer's weight matrix.
#include <algorithm>

#include "fp4_device.hpp"
#include "launch.hpp"

namespace fp4 {
namespace {

__device__ __forceinline__ int clamp_index(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// Chunks of 8 bf16 (16 bytes) per thread: cols <= 16384 is 2048 chunks; and
// columns per thread.
constexpr int kMaxChunksPerThread = 2048 / kThreads;
constexpr int kMaxColsPerThread = 16384 / kThreads;

// Rotation tables staged in LDS: (i | j << 16) and (cos, sin) per rotation,
// then the layer starts.
struct Tables {
  uint32_t* ij;
  float2_t* cs;
  int32_t* ls;
};

// A work-group takes rows blockIdx.x, blockIdx.x + gridDim.x, ... The row is
// read with 16-byte loads (the next row's loads are issued before the current
// row is rotated, so they are in flight meanwhile), put in LDS (as bf16 when
// it is then gathered through the permutation), widened to an fp32 LDS row,
// rotated layer by layer (the pairs of a layer are disjoint: one thread per
// pair, a barrier between layers), and written back as bf16 (RNE) with
// 16-byte stores. With kStaged the rotation tables are copied to LDS once per
// work-group; otherwise they are read from memory in every layer. Every index
// read from memory is clamped into the row, every rotation number into
// 0 .. n_rot.
template <bool kPerm, bool kStaged>
__global__ __launch_bounds__(kThreads) void givens_rows_kernel(
    const uint16_t* x, int64_t ld_x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ pairs, const float* __restrict__ cs,
    const int32_t* __restrict__ layer_start, int n_layers, int n_rot, uint16_t* out,
    int64_t ld_out, int64_t rows, int cols) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* z = reinterpret_cast<float*>(smem);  // cols fp32
  uint8_t* rest = smem + 4 * (size_t)cols;
  uint16_t* raw = reinterpret_cast<uint16_t*>(rest);  // cols bf16 (kPerm)
  if (kPerm) rest += 2 * (size_t)cols;
  Tables t{reinterpret_cast<uint32_t*>(rest),
           reinterpret_cast<float2_t*>(rest + 4 * (size_t)n_rot + 4 * (n_rot & 1)),
           reinterpret_cast<int32_t*>(rest + 12 * (size_t)n_rot + 4 * (n_rot & 1))};
  if (kStaged) {
    for (int k = threadIdx.x; k < n_rot; k += kThreads) {
      t.ij[k] = (uint32_t)clamp_index(pairs[2 * k], cols) |
                ((uint32_t)clamp_index(pairs[2 * k + 1], cols) << 16);
      t.cs[k] = float2_t{cs[2 * k], cs[2 * k + 1]};
    }
    for (int L = threadIdx.x; L <= n_layers; L += kThreads)
      t.ls[L] = min(max(layer_start[L], 0), n_rot);
  }
  const int chunks = cols / 8;
  // the permutation entries of the thread's columns j = threadIdx.x + 256 u,
  // two 16-bit entries per register (read once; a load issued per row would
  // wait behind the next row's loads)
  uint32_t pj[kMaxColsPerThread / 2];
  if (kPerm) {
#pragma unroll
    for (int u = 0; u < kMaxColsPerThread; u += 2) {
      const int j0 = (int)threadIdx.x + u * kThreads, j1 = j0 + kThreads;
      const uint32_t a = j0 < cols ? (uint32_t)clamp_index(perm[j0], cols) : 0u;
      const uint32_t b = j1 < cols ? (uint32_t)clamp_index(perm[j1], cols) : 0u;
      pj[u / 2] = a | (b << 16);
    }
  }
  u32x4_t nxt[kMaxChunksPerThread];
  auto load_row = [&](int64_t r) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + r * ld_x);
#pragma unroll
    for (int u = 0; u < kMaxChunksPerThread; ++u) {
      const int c = (int)threadIdx.x + u * kThreads;
      if (c < chunks) nxt[u] = __builtin_nontemporal_load(src + c);
    }
  };
  if (blockIdx.x < rows) load_row(blockIdx.x);
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
#pragma unroll
    for (int u = 0; u < kMaxChunksPerThread; ++u) {
      const int c = (int)threadIdx.x + u * kThreads;
      if (c >= chunks) continue;
      const u32x4_t v = nxt[u];
      if (kPerm) {
        reinterpret_cast<u32x4_t*>(raw)[c] = v;
      } else {
        f32x4_t lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = __uint_as_float(e & 1 ? (v[e / 2] & 0xFFFF0000u) : (v[e / 2] << 16));
          hi[e] = __uint_as_float(e & 1 ? (v[2 + e / 2] & 0xFFFF0000u) : (v[2 + e / 2] << 16));
        }
        reinterpret_cast<f32x4_t*>(z)[2 * c] = lo;
        reinterpret_cast<f32x4_t*>(z)[2 * c + 1] = hi;
      }
    }
    if (r + gridDim.x < rows) load_row(r + gridDim.x);  // in flight during this row
    __syncthreads();
    if (kPerm) {
#pragma unroll
      for (int u = 0; u < kMaxColsPerThread; ++u) {
        const int j = (int)threadIdx.x + u * kThreads;
        if (j < cols) z[j] = __uint_as_float((uint32_t)raw[(pj[u / 2] >> (16 * (u & 1))) & 0xFFFFu] << 16);
      }
      __syncthreads();
    }
    for (int L = 0; L < n_layers; ++L) {
      int k0, k1;
      if (kStaged) {
        k0 = t.ls[L];
        k1 = max(t.ls[L + 1], k0);
      } else {
        k0 = min(max(layer_start[L], 0), n_rot);
        k1 = min(max(layer_start[L + 1], k0), n_rot);
      }
      for (int k = k0 + (int)threadIdx.x; k < k1; k += kThreads) {
        int i, j;
        float c, s;
        if (kStaged) {
          const uint32_t ij = t.ij[k];
          i = (int)(ij & 0xFFFFu);
          j = (int)(ij >> 16);
          const float2_t q = t.cs[k];
          c = q[0];
          s = q[1];
        } else {
          i = clamp_index(pairs[2 * k], cols);
          j = clamp_index(pairs[2 * k + 1], cols);
          c = cs[2 * k];
          s = cs[2 * k + 1];
        }
        const float zi = z[i], zj = z[j];
        z[i] = c * zi - s * zj;
        z[j] = s * zi + c * zj;
      }
      __syncthreads();
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + r * ld_out);
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
      const f32x4_t lo = reinterpret_cast<const f32x4_t*>(z)[2 * c];
      const f32x4_t hi = reinterpret_cast<const f32x4_t*>(z)[2 * c + 1];
      const u32x4_t w = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                         pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
      __builtin_nontemporal_store(w, dst + c);
    }
    __syncthreads();  // the LDS rows are reused by the next row
  }
}

// Wait for this wave's LDS operations and keep the compiler's memory accesses
// on their side: lanes of one wave then see each other's LDS writes (the LDS
// runs a wave's instructions in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// LDS bytes of givens_compact_kernel: two bf16 row buffers (4 cols bytes,
// which also hold the channel -> slot map while the tables are built), then
// per rotation 28 bytes (two fp32 slot values, (cos, sin), the slot pair, two
// 16-bit sources, two bf16 results) and the layer starts.
__host__ __device__ constexpr size_t compact_lds(int64_t cols, int n_rot, int n_layers) {
  return 4 * (size_t)cols + 28 * (size_t)n_rot + 4 * (size_t)(n_layers + 1);
}

// The permuted transform with the rotations on a compact copy of the
// channels they touch. A rotation touches two channels and a calibrated
// transform has at most blocks - 1 of them (510 of 8192 channels at 16384 x
// 8192), so every other output channel is a plain gather of the input row.
// At set-up each work-group gives every touched channel one slot (the lowest
// of 2k, 2k + 1 over the rotations k that touch it), rewrites the rotation
// table in slots, and records per slot the input position pi(channel) it
// starts from. Per row:
//   1. the row goes from registers into one of two LDS row buffers (bf16),
//      the next row's loads are issued, and the work-group meets;
//   2. wave 0 alone gathers the touched channels into the fp32 slots, runs the
//      layers on them (a layer's rotations are disjoint: one lane per
//      rotation, a wave-level wait between layers) and rounds them to bf16;
//      the work-group meets;
//   3. every thread writes its 16-byte output chunks, each value read from
//      the row buffer at pi(j) or, for a touched channel j, from its slot.
// Two barriers per row, against one per layer in givens_rows_kernel, and
// 4 bytes of LDS per column against 6. The arithmetic of every rotation is
// the same, in the same layer order, so the results equal givens_rows_kernel's
// (untouched channels bit for bit). The row buffer written in step 1 of row
// k + 1 was last read in step 3 of row k - 1, before the first barrier of row
// k; the bf16 slots written in step 2 were last read in step 3 of the row
// before, before this row's first barrier. Indices are clamped into the row.
constexpr int kRounds = 16;     // rotation rounds wave 0 can hold in registers
constexpr int kSlotRounds = 8;  // slot sources it can hold (512 slots)

template <int kCpt>  // 16-byte chunks per thread: cols <= 8 kCpt kThreads
__global__ __launch_bounds__(kThreads) void givens_compact_kernel(
    const uint16_t* x, int64_t ld_x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ pairs, const float* __restrict__ cs,
    const int32_t* __restrict__ layer_start, int n_layers, int n_rot, uint16_t* out,
    int64_t ld_out, int64_t rows, int cols) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int ns = 2 * n_rot;  // slots
  uint16_t* raw = reinterpret_cast<uint16_t*>(smem);      // [2][cols] bf16
  uint32_t* slot_of = reinterpret_cast<uint32_t*>(smem);  // [cols], set-up only
  uint8_t* p = smem + 4 * (size_t)cols;
  float* zs = reinterpret_cast<float*>(p);
  p += 4 * (size_t)ns;
  float2_t* tcs = reinterpret_cast<float2_t*>(p);  // 8-byte aligned: cols % 8 == 0
  p += 8 * (size_t)n_rot;
  uint32_t* tij = reinterpret_cast<uint32_t*>(p);
  p += 4 * (size_t)n_rot;
  int32_t* tls = reinterpret_cast<int32_t*>(p);
  p += 4 * (size_t)(n_layers + 1);
  uint16_t* src = reinterpret_cast<uint16_t*>(p);
  p += 2 * (size_t)ns;
  uint16_t* zb = reinterpret_cast<uint16_t*>(p);
  const int tid = (int)threadIdx.x;

  // ---- set-up: slots, slot tables, per-thread output sources ----
  for (int c = tid; c < cols; c += kThreads) slot_of[c] = 0xFFFFFFFFu;
  for (int s = tid; s < ns; s += kThreads) src[s] = 0xFFFFu;
  for (int L = tid; L <= n_layers; L += kThreads) tls[L] = min(max(layer_start[L], 0), n_rot);
  __syncthreads();
  for (int k = tid; k < n_rot; k += kThreads) {
    atomicMin(&slot_of[clamp_index(pairs[2 * k], cols)], (uint32_t)(2 * k));
    atomicMin(&slot_of[clamp_index(pairs[2 * k + 1], cols)], (uint32_t)(2 * k + 1));
    tcs[k] = float2_t{cs[2 * k], cs[2 * k + 1]};
  }
  __syncthreads();
  for (int k = tid; k < n_rot; k += kThreads) {
    const int i = clamp_index(pairs[2 * k], cols), j = clamp_index(pairs[2 * k + 1], cols);
    const uint32_t si = slot_of[i], sj = slot_of[j];
    tij[k] = si | (sj << 16);
    if (si == (uint32_t)(2 * k)) src[si] = (uint16_t)clamp_index(perm[i], cols);
    if (sj == (uint32_t)(2 * k + 1)) src[sj] = (uint16_t)clamp_index(perm[j], cols);
  }
  // output sources of the thread's chunks c = tid + kThreads u, two 16-bit
  // entries per register: 0x8000 | slot for a touched channel, else pi(j)
  const int chunks = cols / 8;
  uint32_t code[kCpt * 4];
#pragma unroll
  for (int u = 0; u < kCpt; ++u) {
    const int c = tid + u * kThreads;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t h[2] = {0u, 0u};
      if (c < chunks) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = 8 * c + e + q;
          const uint32_t so = slot_of[j];
          h[q] = so != 0xFFFFFFFFu ? 0x8000u | so : (uint32_t)clamp_index(perm[j], cols);
        }
      }
      code[u * 4 + e / 2] = h[0] | (h[1] << 16);
    }
  }
  __syncthreads();  // slot_of's bytes become row buffers

  u32x4_t nxt[kCpt];
  auto load_row = [&](int64_t r) {
    const u32x4_t* srcp = reinterpret_cast<const u32x4_t*>(x + r * ld_x);
#pragma unroll
    for (int u = 0; u < kCpt; ++u) {
      const int c = tid + u * kThreads;
      if (c < chunks) nxt[u] = __builtin_nontemporal_load(srcp + c);
    }
  };
  const uint32_t wave = (uint32_t)tid >> 6, lane = (uint32_t)tid & 63u;
  // Wave 0 keeps its rotations in registers when they fit: round t is up to
  // 64 rotations of one layer, lane l holding the l-th (slot pair, cos, sin),
  // ~0u for none; and the input positions of slots lane + 64 t. Each round
  // then costs one LDS round trip instead of three.
  uint32_t rij[kRounds], rsrc[kSlotRounds];
  float rc[kRounds], rs[kRounds];
  int n_rounds = 0;
  bool in_regs = false;
  if (wave == 0) {
    for (int L = 0; L < n_layers; ++L) n_rounds += (max(tls[L + 1], tls[L]) - tls[L] + 63) / 64;
    in_regs = n_rounds <= kRounds && ns <= 64 * kSlotRounds;
    int L = 0, k = n_layers > 0 ? tls[0] : 0;
#pragma unroll
    for (int t = 0; t < kRounds; ++t) {
      while (L < n_layers && k >= max(tls[L + 1], tls[L])) {
        ++L;
        if (L < n_layers) k = tls[L];
      }
      uint32_t ij = ~0u;
      float c = 0.0f, sn = 0.0f;
      if (in_regs && L < n_layers) {
        const int kk = k + (int)lane;
        if (kk < max(tls[L + 1], tls[L])) {
          ij = tij[kk];
          c = tcs[kk][0];
          sn = tcs[kk][1];
        }
        k += 64;
      }
      rij[t] = ij;
      rc[t] = c;
      rs[t] = sn;
    }
#pragma unroll
    for (int t = 0; t < kSlotRounds; ++t) {
      const int sl = (int)lane + 64 * t;
      rsrc[t] = in_regs && sl < ns ? (uint32_t)src[sl] : 0xFFFFu;
    }
  }
  if (blockIdx.x < rows) load_row(blockIdx.x);
  int buf = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, buf ^= 1) {
    uint16_t* rb = raw + (size_t)buf * cols;
#pragma unroll
    for (int u = 0; u < kCpt; ++u) {
      const int c = tid + u * kThreads;
      if (c < chunks) reinterpret_cast<u32x4_t*>(rb)[c] = nxt[u];
    }
    if (r + gridDim.x < rows) load_row(r + gridDim.x);  // in flight during this row
    __syncthreads();
    if (wave == 0 && in_regs) {
#pragma unroll
      for (int t = 0; t < kSlotRounds; ++t)
        if (rsrc[t] != 0xFFFFu) zs[(int)lane + 64 * t] = __uint_as_float((uint32_t)rb[rsrc[t]] << 16);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < kRounds; ++t) {
        if (t >= n_rounds) break;
        if (rij[t] != ~0u) {
          const int i = (int)(rij[t] & 0xFFFFu), j = (int)(rij[t] >> 16);
          const float zi = zs[i], zj = zs[j];
          zs[i] = rc[t] * zi - rs[t] * zj;
          zs[j] = rs[t] * zi + rc[t] * zj;
        }
        wave_lds_sync();
      }
#pragma unroll
      for (int t = 0; t < kSlotRounds; ++t) {
        const int sl = (int)lane + 64 * t;
        if (sl < ns) zb[sl] = (uint16_t)(pack_bf16x2(zs[sl], 0.0f) & 0xFFFFu);
      }
    } else if (wave == 0) {
      for (int s = (int)lane; s < ns; s += 64) {
        const uint32_t q = src[s];
        if (q != 0xFFFFu) zs[s] = __uint_as_float((uint32_t)rb[q] << 16);
      }
      wave_lds_sync();
      for (int L = 0; L < n_layers; ++L) {
        const int k0 = tls[L], k1 = max(tls[L + 1], k0);
        for (int k = k0 + (int)lane; k < k1; k += 64) {
          const uint32_t ij = tij[k];
          const int i = (int)(ij & 0xFFFFu), j = (int)(ij >> 16);
          const float2_t q = tcs[k];
          const float c = q[0], s = q[1];
          const float zi = zs[i], zj = zs[j];
          zs[i] = c * zi - s * zj;
          zs[j] = s * zi + c * zj;
        }
        wave_lds_sync();
      }
      for (int s = (int)lane; s < ns; s += 64)
        zb[s] = (uint16_t)(pack_bf16x2(zs[s], 0.0f) & 0xFFFFu);
    }
    __syncthreads();
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + r * ld_out);
#pragma unroll
    for (int u = 0; u < kCpt; ++u) {
      const int c = tid + u * kThreads;
      if (c >= chunks) continue;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pair = code[u * 4 + e];
        uint32_t v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t h = (pair >> (16 * q)) & 0xFFFFu;
          v[q] = (h & 0x8000u) ? zb[h & 0x7FFFu] : rb[h];
        }
        w[e] = v[0] | (v[1] << 16);
      }
      __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, dst + c);
    }
  }
}

}  // namespace

void launch_givens_rows(int64_t rows, int64_t cols, const void* x, int64_t ld_x,
                        const int32_t* perm, const int32_t* pairs, const float* cs,
                        const int32_t* layer_start, int n_layers, int n_rot, void* out,
                        int64_t ld_out, hipStream_t st) {
  const DeviceInfo di = device_info();
  auto xp = static_cast<const uint16_t*>(x);
  auto op = static_cast<uint16_t*>(out);
  // with a permutation: the compact kernel when its tables fit (slots below
  // 2^15, LDS for at least one work-group); 142 -> 108 us at 16384 x 8192 with
  // 255 rotations in 13 layers. Without one the row-wide kernel stays: its
  // 16-byte LDS reads of the fp32 row beat the compact kernel's per-element
  // reads (94 against 103 us).
  const size_t clds = compact_lds(cols, n_rot, n_layers);
  if (perm && n_rot < (1 << 14) && clds + 1024 <= (size_t)di.lds) {
    const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(8, (size_t)di.lds / (clds + 1024)));
    const int64_t wgs = (int64_t)di.cus * per_cu;
    const int grid = (int)(rows < wgs ? rows : wgs);
#define FP4_GIVENS_C(K)                                                                     \
  hipLaunchKernelGGL((givens_compact_kernel<K>), dim3(grid), dim3(kThreads), clds, st, xp, ld_x, \
                     perm, pairs, cs, layer_start, n_layers, n_rot, op, ld_out, rows, (int)cols)
    if (cols <= 8 * 4 * kThreads) FP4_GIVENS_C(4);
    else FP4_GIVENS_C(8);
#undef FP4_GIVENS_C
    return;
  }
  const size_t row_lds = (perm ? 6 : 4) * (size_t)cols;
  // tables: 4 + 8 bytes per rotation (the second array 8-byte aligned), then
  // the layer starts
  const size_t tab_lds = 12 * (size_t)n_rot + 4 * (size_t)(n_rot & 1) + 4 * (size_t)(n_layers + 1);
  const bool staged = row_lds + tab_lds + 1024 <= (size_t)di.lds;
  const size_t lds = row_lds + (staged ? tab_lds : 0);
  const int per_cu = (int)std::max<size_t>(1, std::min<size_t>(8, (size_t)di.lds / (lds + 1024)));
  const int64_t wgs = (int64_t)di.cus * per_cu;
  const int grid = (int)(rows < wgs ? rows : wgs);
#define FP4_GIVENS(P, S)                                                                    \
  hipLaunchKernelGGL((givens_rows_kernel<P, S>), dim3(grid), dim3(kThreads), lds, st, xp, ld_x, \
                     perm, pairs, cs, layer_start, n_layers, n_rot, op, ld_out, rows, (int)cols)
  if (perm && staged) FP4_GIVENS(true, true);
  else if (perm) FP4_GIVENS(true, false);
  else if (staged) FP4_GIVENS(false, true);
  else FP4_GIVENS(false, false);
#undef FP4_GIVENS
}

}  // namespace fp4
