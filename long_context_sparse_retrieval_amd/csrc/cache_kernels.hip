// Cache writers (post-RoPE keys, indexer keys) and the standalone indexer score.
//
// "Full Attention Strikes Back" (RTPurbo) section 2.2 eq. (1): RoPE rotates
// channel pair i of a row at position n by n * theta_i.  Section 3.2 eq. (4):
// the indexer scores s(m, n) = (W_q q_pre_m) . (W_k k_pre_n) on pre-RoPE
// features with rank-16 projections.
#include "rtp_internal.h"

namespace rtp {

// ------------------------------------------------------------------ RoPE keys
// One wave per row, one lane per channel pair; angles n * theta_i in fp64.
__global__ __launch_bounds__(kWG) void rope_keys_kernel(Geo g, const rtp_bf16 *k_pre, rtp_bf16 *k_out,
                                                        long long n0,
                                                        long long rows_per_bg) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long total = rows_per_bg * g.B * g.Hkv;
  if (row >= total) return;
  const long long bg = row / rows_per_bg;
  const long long n = n0 + (row - bg * rows_per_bg);
  const size_t off = ((size_t)bg * g.Ncap + n) * kD + 2 * lane;
  const uint32_t w = *reinterpret_cast<const uint32_t *>(k_pre + off);
  double sn, cs;
  sincos((double)n * rope_freq(g.theta, lane), &sn, &cs);
  *reinterpret_cast<uint32_t *>(k_out + off) = rope_pair_bf16(w, sn, cs);
}

int launch_rope_keys(const Geo &g, const rtp_bf16 *k_pre, rtp_bf16 *k_out, long long n0, long long n1,
                     hipStream_t s) {
  const long long rows = (n1 - n0) * g.B * g.Hkv;
  if (rows == 0) return RTP_OK;
  const long long blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(rope_keys_kernel, dim3((unsigned)blocks), dim3(kWG), 0, s, g, k_pre, k_out, n0, n1 - n0);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

// ------------------------------------------------------------------ indexer keys
// 16 rows x 16 outputs per workgroup; the exact fp64 dot of 128 bf16 products
// is rounded once to bf16.
__global__ __launch_bounds__(kWG) void index_keys_kernel(Geo g, const rtp_bf16 *__restrict__ k_pre,
                                                         const rtp_bf16 *__restrict__ w_k,
                                                         rtp_bf16 *__restrict__ k_idx, long long n0,
                                                         long long per, int blocks_per) {
  __shared__ double s_w[kD][kR + 1];
  __shared__ double s_x[16][kD + 1];
  const int tid = threadIdx.x;
  const int br = blockIdx.x / blocks_per, blk = blockIdx.x % blocks_per;
  const int b = br / g.Hi, r = br % g.Hi;                // r: indexer-key head
  const int kvg = g.rhead[r * g.ig] / g.G;
  const long long nb = n0 + (long long)blk * 16;
  const int nrows = (int)min<long long>(16, per - (long long)blk * 16);
  for (int i = tid; i < kD * kR; i += kWG) {
    const uint16_t wb = w_k[(size_t)r * kD * kR + i];
    s_w[i / kR][i % kR] = (double)__uint_as_float((uint32_t)wb << 16);
  }
  for (int i = tid; i < 16 * kD; i += kWG) {
    const int rr = i / kD, c = i % kD;
    double x = 0.0;
    if (rr < nrows) {
      const uint16_t xb = k_pre[(((size_t)b * g.Hkv + kvg) * g.Ncap + nb + rr) * kD + c];
      x = (double)__uint_as_float((uint32_t)xb << 16);
    }
    s_x[rr][c] = x;
  }
  __syncthreads();
  const int rr = tid >> 4, j = tid & 15;
  if (rr >= nrows) return;
  double acc = 0.0;
#pragma unroll 8
  for (int c = 0; c < kD; ++c) acc = fma(s_x[rr][c], s_w[c][j], acc);
  k_idx[(((size_t)b * g.Hi + r) * g.Ncap + nb + rr) * kR + j] = f64_to_bf16(acc);
}

int launch_index_keys(const Geo &g, const rtp_bf16 *k_pre, const rtp_bf16 *w_k, rtp_bf16 *k_idx, long long n0,
                      long long n1, hipStream_t s) {
  const long long per = n1 - n0;
  if (per == 0 || g.Hi == 0) return RTP_OK;
  const int blocks_per = (int)((per + 15) / 16);
  hipLaunchKernelGGL(index_keys_kernel, dim3((unsigned)((long long)blocks_per * g.B * g.Hi)), dim3(kWG), 0, s, g,
                     k_pre, w_k, k_idx, n0, per, blocks_per);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

// ------------------------------------------------------------------ standalone scores
// One workgroup per (query unit, 1024-token block); one token per thread per step.
__global__ __launch_bounds__(kWG) void index_score_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                          const rtp_bf16 *__restrict__ w_q,
                                                          const rtp_bf16 *__restrict__ k_idx,
                                                          float *__restrict__ logits, int blocks_per_unit) {
  __shared__ double s_q[kR];
  __shared__ double s_tmp[16][kR];
  const int unit = blockIdx.x / blocks_per_unit;
  const int blk = blockIdx.x % blocks_per_unit;
  const int i = unit % g.nq, br = unit / g.nq;
  const int r = br % g.Hr, b = br / g.Hr;
  const int hq = g.rhead[r];
  project_query(q_pre + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, w_q + (size_t)r * kD * kR, s_q, s_tmp);
  double q[kR];
#pragma unroll
  for (int j = 0; j < kR; ++j) q[j] = s_q[j];
  const long long m = g.N - g.nq + i;
  const uint4 *rows = reinterpret_cast<const uint4 *>(k_idx + ((size_t)b * g.Hi + r / g.ig) * g.Ncap * kR);
  float *out = logits + (size_t)unit * g.N;
  for (int k = 0; k < 4; ++k) {
    const long long n = (long long)blk * 1024 + k * kWG + threadIdx.x;
    if (n >= g.N) break;
    float s = -INFINITY;
    if (n <= m) s = dot16_exact(q, rows[2 * n], rows[2 * n + 1]);
    out[n] = s;
  }
}

int launch_index_score(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                       float *logits, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  const int bpu = (int)((g.N + 1023) / 1024);
  hipLaunchKernelGGL(index_score_kernel, dim3((unsigned)((long long)bpu * g.units)), dim3(kWG), 0, s, g, q_pre, w_q,
                     k_idx, logits, bpu);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

// ------------------------------------------------------------------ workspace fill
__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

int launch_fill_zero(void *ws, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return RTP_OK;
  const size_t nb = (n16 + kWG - 1) / kWG;
  const unsigned blocks = (unsigned)(nb < 4096 ? nb : 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kWG), 0, s, reinterpret_cast<uint4 *>(ws), n16);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace rtp
