// Parameter-free RMS normalisation of the query and key rows (QK-norm) for gfx950.
//
// Operation: the model's RMS normalisations carry no trainable parameters (walkthrough "A fully
// hand-made copy of ChatGPT for $100 and 8,000 lines of code", section "Pretraining", the
// paragraph on the optimisers); applied to q and k per head it gives attention inputs of unit
// RMS:
//   r = 1 / sqrt(mean_d x_d^2 + eps),  x_hat = x * r   (one row = one token of one head).
// The normalised rows are what the attention kernels read, and the backward needs them again, so
// they are written once (bf16, round to nearest even) together with r (fp32, [B, H, T]); the
// norm's own backward runs inside the dQ and dK/dV epilogues (bwd.hip).  The QK-norm forward
// normalises q itself, in its prologue (fwd.hip), and runs this pass on k alone (q null).
//
// Memory-bound: one read and one write of each row.  D / 8 lanes hold one row (16 bytes each), so a
// wave normalises 64 / (D / 8) rows and the sum of squares is a reduction over D / 8 lanes.
#include "common.h"
#include "launch.h"

namespace swattn {

template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
#pragma unroll
  for (int off = 1; off < N; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void qk_rmsnorm_kernel(NormArgs p) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const int64_t rows = (int64_t)p.B * p.T * p.H;  // rows of q, then rows of k
  const int64_t row = (p.q ? 0 : rows) + (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  if (row >= 2 * rows) return;  // every lane of a row group leaves together
  const bool is_k = row >= rows;
  const int64_t r = is_k ? row - rows : row;  // (b, t, h) in [B, T, H] order
  const uint16_t* src = (is_k ? p.k : p.q) + r * D + 8 * c;
  uint16_t* dst = (is_k ? p.kn : p.qn) + r * D + 8 * c;
  const uint4 v = ldg16(src);
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(w[e]);
    x[2 * e + 1] = bf16_hi(w[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = lane_group_sum<LPR>(ss);
  const float rinv = 1.f / sqrtf(ss / (float)D + p.eps);
  uint4 o;
  o.x = pack_bf16x2(x[0] * rinv, x[1] * rinv);
  o.y = pack_bf16x2(x[2] * rinv, x[3] * rinv);
  o.z = pack_bf16x2(x[4] * rinv, x[5] * rinv);
  o.w = pack_bf16x2(x[6] * rinv, x[7] * rinv);
  *reinterpret_cast<uint4*>(dst) = o;
  if (c == 0) {
    const int64_t bt = r / p.H;
    const int h = (int)(r % p.H);
    const int64_t b = bt / p.T, t = bt % p.T;
    (is_k ? p.rk : p.rq)[(b * p.H + h) * p.T + t] = rinv;
  }
}

hipError_t launch_qk_rmsnorm(const NormArgs& a, hipStream_t s) {
  const int64_t rows = (a.q ? 2 : 1) * (int64_t)a.B * a.T * a.H;  // q null: k only
  const int rpb = 256 / (a.D / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (a.D == 64)
    hipLaunchKernelGGL((qk_rmsnorm_kernel<64>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((qk_rmsnorm_kernel<128>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace swattn
