// Streaming-read probe: the practical HBM read rate of this device, the
// ceiling the bandwidth-bound kernels of librtp.so are compared with.  Not part
// of the decode path; built into its own small library (libreadprobe.so).
//
// Two access patterns, each with plain or non-temporal 16-byte loads:
//  - grid-stride: the whole grid sweeps the buffer, each thread taking every
//    (grid * 256)-th 16-byte word, U independent loads in flight per thread;
//  - chunked: each workgroup streams its own contiguous chunk, consecutive
//    threads on consecutive words, with a rolling window of U loads per
//    thread (the access pattern of the indexer scan).
// Every word read is folded into one register; a word written only when the
// fold hits a chosen value keeps the loads alive.
//
// A third probe, exp_lds_kernel, measures the arithmetic ceiling of the
// chunked prefill's histogram pass (exponential + LDS integer atomic per
// score, no memory traffic).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtp_internal.h"

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ v4u load16(const v4u *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void grid_stride_kernel(const v4u *__restrict__ src, size_t n16,
                                                          unsigned *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = load16<NT>(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// chunk16: 16-byte words per workgroup, a multiple of 256 * U
template <int U, bool NT>
__global__ __launch_bounds__(256) void chunked_kernel(const v4u *__restrict__ src, size_t n16, size_t chunk16,
                                                      unsigned *__restrict__ sink) {
  const size_t c0 = (size_t)blockIdx.x * chunk16;
  const size_t c1 = c0 + chunk16 < n16 ? c0 + chunk16 : n16;
  unsigned acc = 0;
  if (c0 + chunk16 <= n16) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load16<NT>(src + c0 + u * 256 + threadIdx.x);
    for (size_t base = c0; base < c1; base += U * 256) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        const size_t nx = base + (U + u) * 256 + threadIdx.x;
        if (base + U * 256 < c1) v[u] = load16<NT>(src + nx);          // workgroup-uniform
      }
    }
  } else {
    for (size_t i = c0 + threadIdx.x; i < c1; i += 256) {
      const v4u v = load16<NT>(src + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// rows: each thread reads whole 32-byte rows as two 16-byte loads,
// consecutive threads on consecutive rows (each load instruction covers every
// other 16-byte word of its span), with a rolling window of U rows -- the
// access pattern of the indexer-key scan.
template <int U, bool NT>
__global__ __launch_bounds__(256) void rows_kernel(const v4u *__restrict__ src, size_t n16, size_t chunk16,
                                                   unsigned *__restrict__ sink) {
  const size_t c0 = (size_t)blockIdx.x * chunk16;
  unsigned acc = 0;
  if (c0 + chunk16 <= n16) {
    v4u a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = load16<NT>(src + c0 + 2 * (u * 256 + threadIdx.x));
      b[u] = load16<NT>(src + c0 + 2 * (u * 256 + threadIdx.x) + 1);
    }
    for (size_t base = c0; base < c0 + chunk16; base += 2 * U * 256) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w ^ b[u].x ^ b[u].y ^ b[u].z ^ b[u].w;
        const size_t nx = base + 2 * ((U + u) * 256 + threadIdx.x);
        if (base + 2 * U * 256 < c0 + chunk16) {                       // workgroup-uniform
          a[u] = load16<NT>(src + nx);
          b[u] = load16<NT>(src + nx + 1);
        }
      }
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <bool NT>
int launch(const v4u *p, size_t n16, unsigned *sink, int blocks, int unroll, int chunked, hipStream_t s) {
  if (chunked) {
    const size_t per = ((n16 + blocks - 1) / blocks + 256 * 32 - 1) / (256 * 32) * (256 * 32);
    const int nb = (int)((n16 + per - 1) / per);
    if (chunked == 2) {        // 32-byte rows, two loads each (whole chunks only)
      switch (unroll) {
        case 4: hipLaunchKernelGGL((rows_kernel<4, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
        case 8: hipLaunchKernelGGL((rows_kernel<8, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
        case 16: hipLaunchKernelGGL((rows_kernel<16, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
        default: return -1;
      }
      return hipGetLastError() == hipSuccess ? 0 : -5;
    }
    switch (unroll) {
      case 4: hipLaunchKernelGGL((chunked_kernel<4, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
      case 8: hipLaunchKernelGGL((chunked_kernel<8, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
      case 16: hipLaunchKernelGGL((chunked_kernel<16, NT>), dim3(nb), dim3(256), 0, s, p, n16, per, sink); break;
      default: return -1;
    }
  } else {
    switch (unroll) {
      case 4: hipLaunchKernelGGL((grid_stride_kernel<4, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
      case 8: hipLaunchKernelGGL((grid_stride_kernel<8, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
      case 16: hipLaunchKernelGGL((grid_stride_kernel<16, NT>), dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
      default: return -1;
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// The per-score work of the chunked prefill's histogram pass without the
// indexer: each lane bins scores of one of 16 queries (lane mod 16) into that
// query's 256-bin histogram in LDS with one 64-bit integer atomic, the weight
// being the in-cell exp(s - c/8) as a fixed-point integer (the selection
// kernels' own score_cell / cell_weight).  Scores: 16 per lane, uniform in
// [-3, 3) from a per-lane generator, each moved by 2^-12 per round so that no
// round can reuse the previous one's arithmetic.  The rate of this loop is the
// ceiling of that pass on this device.
__global__ __launch_bounds__(256) void exp_lds_kernel(int rounds, unsigned *__restrict__ sink) {
  __shared__ unsigned long long hist[16][rtp::kBins];
  for (int x = threadIdx.x; x < 16 * rtp::kBins; x += 256) (&hist[0][0])[x] = 0ull;
  __syncthreads();
  const int q = threadIdx.x & 15;
  constexpr int cq = 24;                                 // max cell of scores below 3
  uint32_t st = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
  float s[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    st = st * 1664525u + 1013904223u;
    s[k] = (float)(st >> 8) * (6.0f / 16777216.0f) - 3.0f;
  }
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float sc = s[k];
      const int cell = rtp::score_cell(sc);
      int j = cq - cell;
      const int ref = j >= rtp::kBins - 1 ? cq - (rtp::kBins - 1) : cell;
      j = j >= rtp::kBins - 1 ? rtp::kBins - 1 : j;
      const uint32_t w = rtp::cell_weight(sc, ref);
      atomicAdd(&hist[q][j], (unsigned long long)w | (1ull << 41));
      s[k] = sc + 0.000244140625f;
    }
  }
  __syncthreads();
  if (hist[q][threadIdx.x >> 4] == 0x9e3779b97f4a7c15ull) sink[0] = 1u;
}

}  // namespace

extern "C" {

// Enqueue one pass reading `bytes` (a multiple of 16) at src (16-byte aligned)
// with `blocks` workgroups of 256 threads (chunked 1: about that many, each a
// contiguous chunk; chunked 2: the same as 32-byte rows read as two loads,
// U rows in flight per thread) and `unroll` (4, 8 or 16) loads in flight per
// thread;
// nontemporal != 0 uses non-temporal loads.  sink: one device word (written
// only by chance).  Returns 0, or -1 for invalid arguments, -5 for a failed
// launch.
// Enqueue `blocks` workgroups of exp_lds_kernel, each binning 256 * 16 *
// rounds scores (rounds in 1..2048).  sink: one device word (written only by
// chance).  Returns 0, -1 for invalid arguments, -5 for a failed launch.
int readprobe_exp_lds(int blocks, int rounds, unsigned *sink, void *stream) {
  if (!sink || blocks < 1 || rounds < 1 || rounds > 2048) return -1;
  hipLaunchKernelGGL(exp_lds_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), rounds,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int readprobe_stream(const void *src, size_t bytes, unsigned *sink, int blocks, int unroll, int chunked,
                     int nontemporal, void *stream) {
  if (!src || !sink || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) || blocks < 1) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const v4u *p = static_cast<const v4u *>(src);
  return nontemporal ? launch<true>(p, bytes / 16, sink, blocks, unroll, chunked, s)
                     : launch<false>(p, bytes / 16, sink, blocks, unroll, chunked, s);
}

}  // extern "C"
