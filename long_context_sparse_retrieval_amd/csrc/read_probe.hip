// Streaming-read probe: the practical HBM read rate of this device, the
// ceiling the bandwidth-bound kernels of librtp.so are compared with.  Not part
// of the decode path; built into its own small library (libreadprobe.so).
//
// Every thread reads 16-byte words in a grid-stride loop, U independent loads
// in flight per thread, and folds them into one register; a word that can
// only be written when the fold hits a chosen value keeps the loads alive.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                          unsigned *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Enqueue one pass reading `bytes` (a multiple of 16) at src (16-byte aligned)
// with `blocks` workgroups of 256 threads and `unroll` (4, 8 or 16) loads in
// flight per thread.  sink: one device word (written only by chance).
// Returns 0, or -1 for invalid arguments, -5 for a failed launch.
int readprobe_stream(const void *src, size_t bytes, unsigned *sink, int blocks, int unroll, void *stream) {
  if (!src || !sink || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) || blocks < 1) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint4 *p = static_cast<const uint4 *>(src);
  const size_t n16 = bytes / 16;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
