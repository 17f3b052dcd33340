// Streaming-read reference for the decode roofline (measurement only; not part of the attention
// path).  Every thread XOR-folds 16-byte words at a grid-wide stride, eight loads in flight, and
// writes one word so that the loads cannot be dropped.  Timing it over the same number of bytes the
// decode step reads, from buffers larger than the last-level cache, gives the read bandwidth this
// GPU actually sustains at that transfer size -- the practical ceiling for an HBM-bound kernel,
// next to the published peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (size_t i = tid; i < n16; i += stride * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = i + u * stride;
      v[u] = j < n16 ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from the 16-byte aligned device buffer `src`; `out` is a device
// buffer of blocks * 256 uint32.  Returns 0, -1 for bad arguments, -4 for a launch error.
extern "C" int swattn_stream_read(const void* src, size_t bytes, void* out, int blocks,
                                  void* stream) {
  if (!src || !out || blocks < 1 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16,
                     static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
