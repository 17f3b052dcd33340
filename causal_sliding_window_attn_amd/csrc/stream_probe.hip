// Streaming-read reference for the decode roofline (measurement only; not part of the attention
// path).  Each workgroup reads its own contiguous slice of the buffer with nontemporal 16-byte
// loads, sixteen in flight per thread, and XOR-folds them into one word per thread so that the
// loads cannot be dropped.  Of the read forms measured on an MI355X at the decode's transfer
// size (a few hundred MB) this one sustains the most: a grid-wide stride (every workgroup one
// 4 KB piece of each 4 MB stretch) reaches about 20% less, and plain loads about 8% less than
// nontemporal ones.  Timing it over the same number of bytes the decode step reads, from buffers
// larger than the last-level cache, gives the read bandwidth this GPU actually sustains at that
// size -- the practical ceiling for an HBM-bound kernel, next to the published peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 16;
constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src,
                                                               size_t n16,
                                                               uint32_t* __restrict__ out) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  for (size_t i = beg + threadIdx.x; i < end; i += (size_t)kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      v[u] = j < end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + j))
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer `src`; `out` is a device
// buffer of blocks * 256 uint32.  Returns 0, -1 for bad arguments, -4 for a launch error.
extern "C" int swattn_stream_read(const void* src, size_t bytes, void* out, int blocks,
                                  void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---------------------------------------------------------------------------------------------
// Access-pattern references for the decode (measurement only): the same cache bytes a decode of
// the [B, Lcap, H, D] bf16 caches reads (rows max(0, L - w) .. L - 1 of every sequence, all heads,
// K and V), read with nontemporal 16-byte loads and no arithmetic, in two orders:
//   pieces: one workgroup of 8 waves per (sequence, head), 64-row chunks dealt to the waves, D / 8
//     lanes per row's 2 D bytes of the head and 64 / (D / 8) rows per load instruction -- the
//     decode's own order;
//   rows:   one workgroup of 512 threads per (sequence, 32-row chunk), consecutive threads on
//     consecutive 16 bytes of the chunk's rows, all heads together.
// The gap between the two is what reading whole rows would gain over the decode's order.
namespace {

__device__ __forceinline__ uint32_t fold_nt(const uint16_t* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return x[0] ^ x[1] ^ x[2] ^ x[3];
}

template <int D>
__global__ __launch_bounds__(512) void pattern_pieces_kernel(const uint16_t* kc, const uint16_t* vc,
                                                             const int* lens, int H, int Lcap,
                                                             int window, uint32_t* out) {
  constexpr int LPK = D / 8, KPI = 64 / LPK, NL = 64 / KPI;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = min(max(lens[b], 0), Lcap);
  const int j0 = L - min(window, L);
  const int kq = lane / LPK, dc = lane % LPK;
  const int64_t rs = (int64_t)H * D;
  const uint16_t* kb = kc + (int64_t)b * Lcap * rs + h * D + 8 * dc;
  const uint16_t* vb = vc + (int64_t)b * Lcap * rs + h * D + 8 * dc;
  uint32_t acc = 0;
  const int nc = (L - j0 + 63) / 64;
  for (int c = wave; c < nc; c += 8) {
    uint32_t x[2 * NL];
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int j = min(j0 + c * 64 + r * KPI + kq, L - 1);
      x[2 * r] = fold_nt(kb + j * rs);
      x[2 * r + 1] = fold_nt(vb + j * rs);
    }
#pragma unroll
    for (int r = 0; r < 2 * NL; ++r) acc ^= x[r];
  }
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(512) void pattern_rows_kernel(const uint16_t* kc, const uint16_t* vc,
                                                           const int* lens, const int* cstart,
                                                           int B, int row_elems, int Lcap,
                                                           int window, uint32_t* out) {
  constexpr int R = 32, U = 8;
  const int gid = blockIdx.x;
  int lo = 0, hi = B - 1;  // the sequence whose chunk range holds gid: cstart[b] <= gid
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cstart[mid] <= gid) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo, c = gid - cstart[b];
  const int L = min(max(lens[b], 0), Lcap);
  const int j0 = L - min(window, L);
  const int r0 = j0 + c * R, r1 = min(r0 + R, L);
  uint32_t acc = 0;
  if (r0 < r1) {
    const uint16_t* kb = kc + ((int64_t)b * Lcap + r0) * row_elems;
    const uint16_t* vb = vc + ((int64_t)b * Lcap + r0) * row_elems;
    const int64_t n16 = (int64_t)(r1 - r0) * row_elems / 8;
    for (int64_t i = threadIdx.x; i < n16; i += 512 * U) {
      uint32_t x[2 * U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = min(i + u * 512, n16 - 1);
        x[2 * u] = fold_nt(kb + 8 * j);
        x[2 * u + 1] = fold_nt(vb + 8 * j);
      }
#pragma unroll
      for (int u = 0; u < 2 * U; ++u) acc ^= x[u];
    }
  }
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = acc;
}

}  // namespace

// kc, vc: [B, Lcap, H, D] bf16 caches; lens: device int32 [B]; window >= 1.  pattern 0 (pieces):
// `out` holds B * H * 512 uint32, cstart is unused.  pattern 1 (rows): cstart is a device int32
// [B + 1] of prefix sums of ceil(min(window, L_b) / 32) (cstart[B] the chunk count, launched as
// the grid), `out` holds cstart[B] * 512 uint32.  D is 64 or 128.  Returns 0, -1 for bad
// arguments, -4 for a launch error.
extern "C" int swattn_decode_pattern_read(int pattern, const void* kc, const void* vc,
                                          const int* lens, const int* cstart, int nchunks, int B,
                                          int H, int Lcap, int D, int window, void* out,
                                          void* stream) {
  if (!kc || !vc || !lens || !out || B < 1 || H < 1 || Lcap < 1 || window < 1 ||
      (D != 64 && D != 128))
    return -1;
  auto s = static_cast<hipStream_t>(stream);
  auto k = static_cast<const uint16_t*>(kc);
  auto v = static_cast<const uint16_t*>(vc);
  auto o = static_cast<uint32_t*>(out);
  if (pattern == 0) {
    if (D == 64)
      hipLaunchKernelGGL(pattern_pieces_kernel<64>, dim3(B * H), dim3(512), 0, s, k, v, lens, H,
                         Lcap, window, o);
    else
      hipLaunchKernelGGL(pattern_pieces_kernel<128>, dim3(B * H), dim3(512), 0, s, k, v, lens, H,
                         Lcap, window, o);
  } else if (pattern == 1) {
    if (!cstart || nchunks < 1) return -1;
    hipLaunchKernelGGL(pattern_rows_kernel, dim3(nchunks), dim3(512), 0, s, k, v, lens, cstart, B,
                       H * D, Lcap, window, o);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
