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
