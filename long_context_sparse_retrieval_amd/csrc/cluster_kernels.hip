// Cluster index of the retrieval heads' cached tokens and the coarse-to-fine
// decode over it.
//
// RTPurboV2 article, finding three: the cached tokens are grouped into K
// clusters in the rank-16 indexer space (K = 128 in its example); a query is
// first matched against the K centres and full attention then runs only over
// the clusters it hits, with a dynamic top-p.  The article names neither the
// clustering method nor the hit rule; this library takes Lloyd's k-means on
// the bf16 indexer keys (exact fp64 distances, centres rounded to bf16 after
// each round, centre j starting at the key at position floor(j N / K), ties to
// the lowest index) and a top-p over clusters in which cluster j weighs
// n_j exp(s_j) (its member count times the softmax weight of its centre
// score), with the token path's 256-bin histogram and ordered fill.
//
// Build (once per cache): init, then rounds of assign + accumulate (per
// workgroup LDS sums, exact fp64 so any order gives the same bits) and
// update; a final assignment writes per-tile cluster counts, a per-head scan
// turns them into offsets, and a scatter writes the member positions grouped
// by cluster and ascending inside each cluster (wave ballots rank equal
// clusters in position order).
//
// Decode: one workgroup per query scores the centres and picks the hit
// clusters (exact integer masses as in the token path); one workgroup per
// (query, cluster) copies a hit cluster's members into the query's list; the
// split-K sparse attention of the library runs over the lists.
#include "block_util.h"

namespace rtp {

namespace {

constexpr int kClTile = 4096;          // tokens per assignment workgroup
constexpr int kClKeys = 4;             // keys scored together by one thread (centre reads shared)

struct ClAssignShared {
  double c[kMaxClusters][kR];          // centres, widened
  double cc[kMaxClusters];             // their squared norms
  double sum[kMaxClusters][kR];        // per-workgroup member sums (accumulate rounds)
  uint32_t cnt[kMaxClusters];
};

__device__ __forceinline__ double bfd(rtp_bf16 v) { return (double)__uint_as_float((uint32_t)v << 16); }

// centre j = key at position floor(j N / K)
__global__ __launch_bounds__(kWG) void cl_init_kernel(Geo g, ClGeo cg, const rtp_bf16 *__restrict__ k_idx,
                                                      rtp_bf16 *__restrict__ cent) {
  const int u = blockIdx.x;                                      // (b, indexer-key head)
  for (int x = threadIdx.x; x < cg.K * kR; x += kWG) {
    const int j = x / kR, t = x % kR;
    const long long n = (long long)j * g.N / cg.K;
    cent[((size_t)u * cg.K + j) * kR + t] = k_idx[((size_t)u * g.Ncap + n) * kR + t];
  }
  for (int x = threadIdx.x; x < cg.K * kR; x += kWG) cg.sum[(size_t)u * cg.K * kR + x] = 0.0;
  for (int x = threadIdx.x; x < cg.K; x += kWG) cg.cnt[(size_t)u * cg.K + x] = 0u;
}

// Nearest centre of every key of one tile; MODE 0: accumulate member sums and
// counts; MODE 1: write the assignment and the tile's per-cluster counts.
template <int MODE>
__global__ __launch_bounds__(kWG) void cl_assign_kernel(Geo g, ClGeo cg, const rtp_bf16 *__restrict__ k_idx,
                                                        const rtp_bf16 *__restrict__ cent) {
  __shared__ ClAssignShared sm;
  const int tid = threadIdx.x;
  const int u = blockIdx.x / cg.ntiles, tile = blockIdx.x % cg.ntiles;
  const int K = cg.K;
  for (int x = tid; x < K * kR; x += kWG) {
    const int j = x / kR, t = x % kR;
    sm.c[j][t] = bfd(cent[((size_t)u * K + j) * kR + t]);
    sm.sum[j][t] = 0.0;
  }
  for (int j = tid; j < K; j += kWG) sm.cnt[j] = 0u;
  __syncthreads();
  for (int j = tid; j < K; j += kWG) {
    double a = 0.0;
#pragma unroll
    for (int t = 0; t < kR; ++t) a = fma(sm.c[j][t], sm.c[j][t], a);
    sm.cc[j] = a;
  }
  __syncthreads();
  const long long n0 = (long long)tile * kClTile;
  const long long n1 = n0 + kClTile < g.N ? n0 + kClTile : g.N;
  // kClKeys keys per thread (n, n + kWG, ...): every centre value read from
  // LDS serves all of them; each key keeps its own FMA chain in channel order
  for (long long nbase = n0 + tid; nbase < n1; nbase += (long long)kClKeys * kWG) {
    double x[kClKeys][kR], xx[kClKeys];
    long long nk[kClKeys];
#pragma unroll
    for (int k = 0; k < kClKeys; ++k) {
      nk[k] = nbase + (long long)k * kWG;
      const long long n = nk[k] < n1 ? nk[k] : nbase;             // absent keys repeat the first
      const uint4 *row = reinterpret_cast<const uint4 *>(k_idx + ((size_t)u * g.Ncap + n) * kR);
      const uint4 a = row[0], b2 = row[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b2.x, b2.y, b2.z, b2.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[k][2 * t] = (double)bf_lo(w[t]);
        x[k][2 * t + 1] = (double)bf_hi(w[t]);
      }
      xx[k] = 0.0;
#pragma unroll
      for (int t = 0; t < kR; ++t) xx[k] = fma(x[k][t], x[k][t], xx[k]);
    }
    double best[kClKeys];
    int bj[kClKeys];
#pragma unroll
    for (int k = 0; k < kClKeys; ++k) {
      best[k] = INFINITY;
      bj[k] = 0;
    }
    for (int j = 0; j < K; ++j) {
      double xc[kClKeys];
#pragma unroll
      for (int k = 0; k < kClKeys; ++k) xc[k] = 0.0;
#pragma unroll
      for (int t = 0; t < kR; ++t) {
        const double c = sm.c[j][t];
#pragma unroll
        for (int k = 0; k < kClKeys; ++k) xc[k] = fma(x[k][t], c, xc[k]);
      }
#pragma unroll
      for (int k = 0; k < kClKeys; ++k) {
        const double d = __dadd_rn(__dsub_rn(xx[k], __dmul_rn(2.0, xc[k])), sm.cc[j]);
        if (d < best[k]) {                                       // strict: ties keep the lower index
          best[k] = d;
          bj[k] = j;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kClKeys; ++k) {
      if (nk[k] >= n1) break;
      if (MODE == 0) {
#pragma unroll
        for (int t = 0; t < kR; ++t) atomicAdd(&sm.sum[bj[k]][t], x[k][t]);
        atomicAdd(&sm.cnt[bj[k]], 1u);
      } else {
        cg.assign[(size_t)u * g.N + nk[k]] = bj[k];
        atomicAdd(&sm.cnt[bj[k]], 1u);
      }
    }
  }
  __syncthreads();
  if (MODE == 0) {
    for (int x = tid; x < K * kR; x += kWG) {
      const double v = sm.sum[x / kR][x % kR];
      if (v != 0.0) atomicAdd(&cg.sum[(size_t)u * K * kR + x], v);
    }
    for (int j = tid; j < K; j += kWG)
      if (sm.cnt[j]) atomicAdd(&cg.cnt[(size_t)u * K + j], sm.cnt[j]);
  } else {
    for (int j = tid; j < K; j += kWG) cg.hist[((size_t)u * cg.ntiles + tile) * K + j] = sm.cnt[j];
  }
}

// new centre = bf16(member mean) for every non-empty cluster; sums cleared
__global__ __launch_bounds__(kWG) void cl_update_kernel(Geo g, ClGeo cg, rtp_bf16 *__restrict__ cent) {
  const int u = blockIdx.x;
  for (int x = threadIdx.x; x < cg.K * kR; x += kWG) {
    const int j = x / kR;
    const uint32_t c = cg.cnt[(size_t)u * cg.K + j];
    double *s = &cg.sum[(size_t)u * cg.K * kR + x];
    if (c) cent[(size_t)u * cg.K * kR + x] = f64_to_bf16(*s / (double)c);
    *s = 0.0;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < cg.K; j += kWG) cg.cnt[(size_t)u * cg.K + j] = 0u;
}

// counts and offsets of one head, and the per-tile exclusive prefix of every
// cluster's count (in hist, in place)
__global__ __launch_bounds__(kWG) void cl_offsets_kernel(Geo g, ClGeo cg, int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets) {
  __shared__ uint32_t red[4];
  const int u = blockIdx.x, j = threadIdx.x;
  uint32_t tot = 0;
  if (j < cg.K) {
    uint32_t *h = cg.hist + (size_t)u * cg.ntiles * cg.K + j;
    for (int t = 0; t < cg.ntiles; ++t) {
      const uint32_t c = h[(size_t)t * cg.K];
      h[(size_t)t * cg.K] = tot;
      tot += c;
    }
  }
  uint32_t all;
  const uint32_t ex = block_excl_scan<uint32_t>(j < cg.K ? tot : 0u, all, red);
  if (j < cg.K) {
    counts[(size_t)u * cg.K + j] = (int32_t)tot;
    offsets[(size_t)u * (cg.K + 1) + j] = (int32_t)ex;
  }
  if (j == 0) offsets[(size_t)u * (cg.K + 1) + cg.K] = (int32_t)all;
}

// member positions grouped by cluster, ascending inside each cluster
__global__ __launch_bounds__(kWG) void cl_scatter_kernel(Geo g, ClGeo cg, const int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ members) {
  __shared__ int32_t base[kMaxClusters];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int u = blockIdx.x / cg.ntiles, tile = blockIdx.x % cg.ntiles;
  for (int j = tid; j < cg.K; j += kWG)
    base[j] = offsets[(size_t)u * (cg.K + 1) + j] + (int32_t)cg.hist[((size_t)u * cg.ntiles + tile) * cg.K + j];
  const long long n0 = (long long)tile * kClTile;
  const long long n1 = n0 + kClTile < g.N ? n0 + kClTile : g.N;
  for (long long c0 = n0; c0 < n1; c0 += kWG) {
    const long long n = c0 + tid;
    const int j = n < n1 ? cg.assign[(size_t)u * g.N + n] : -1;
    for (int w = 0; w < 4; ++w) {                                // waves in position order
      __syncthreads();
      if (wv == w) {
        bool pending = j >= 0;
        while (__any(pending)) {
          const unsigned long long pend = __ballot(pending);
          const int leader = __ffsll((long long)pend) - 1;
          const int lj = __shfl(j, leader);
          const unsigned long long same = __ballot(pending && j == lj);
          if (pending && j == lj) {
            const int rank = __popcll(same & ((1ull << lane) - 1ull));
            members[(size_t)u * g.N + base[lj] + rank] = (int32_t)n;
          }
          if (lane == leader) base[lj] += __popcll(same);
          pending = pending && j != lj;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ decode
struct ClSelShared {
  double q[kR];
  double qtmp[16][kR];
  unsigned long long hist[kBins];
  double red_d[4];
  uint32_t red_u32[4];
  unsigned long long red_u[4];
  int red_i[4];
  double wcum[kBins];
};

// Coarse stage of one query: centre scores, hit clusters (top-p over
// n_j exp(s_j)), and each hit cluster's start in the query's member list.
__global__ __launch_bounds__(kWG) void cl_select_kernel(Geo g, ClGeo cg, const rtp_bf16 *__restrict__ q_pre,
                                                        const rtp_bf16 *__restrict__ w_q,
                                                        const rtp_bf16 *__restrict__ cent,
                                                        const int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ count_opt) {
  __shared__ ClSelShared sm;
  const int tid = threadIdx.x, j = tid;
  const int unit = blockIdx.x;
  const int br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int u = b * g.Hi + r / g.ig;
  project_query(q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + unit % g.nq) * kD, w_q + (size_t)r * kD * kR,
                sm.q, sm.qtmp);
  const int nj = j < cg.K ? counts[(size_t)u * cg.K + j] : 0;
  float s = -INFINITY;
  if (j < cg.K) {
    const uint4 *row = reinterpret_cast<const uint4 *>(cent + ((size_t)u * cg.K + j) * kR);
    s = dot16_exact(sm.q, row[0], row[1]);
  }
  const bool live = nj > 0;
  const int cell = live ? score_cell(s) : INT32_MIN;
  const int c = block_max<int>(cell, sm.red_i);
  const long long dj = live ? (long long)c - cell : 0;
  const int bin = live ? (dj >= kBins - 1 ? kBins - 1 : (int)dj) : -1;
  // in-cell weights (2^23 = 1), times the member count; the clamp bin is
  // weighted relative to its base cell c - 255
  unsigned long long w = 0;
  if (live) w = (unsigned long long)nj * cell_weight(s, bin == kBins - 1 ? c - (kBins - 1) : cell);
  sm.hist[tid] = 0ull;
  __syncthreads();
  if (live) atomicAdd(&sm.hist[bin], w);
  __syncthreads();
  const double Wb = (double)sm.hist[tid] * 0x1p-23 * exp(-(double)tid * 0.125);
  double Z;
  const double excl = block_excl_scan<double>(Wb, Z, sm.red_d);
  const double need = g.p * Z;
  int bstar = block_min<int>(excl + Wb >= need ? tid : kBins, sm.red_i);
  if (bstar >= kBins) bstar = kBins - 1;
  sm.wcum[tid] = excl;
  __syncthreads();
  const double before = sm.wcum[bstar];
  const bool all = g.p >= 1.0 || bstar >= kBins - 1;
  const double r_u = (need - before) * 0x1p23 * exp((double)bstar * 0.125);
  // ordered fill of bin b*: its clusters in ascending index while the mass before them is below the residual
  unsigned long long wtot;
  const unsigned long long pre = block_excl_scan<unsigned long long>(live && bin == bstar ? w : 0ull, wtot, sm.red_u);
  bool hit = live && (all || bin < bstar || (bin == bstar && (double)pre < r_u));
  uint32_t total;
  const uint32_t start = block_excl_scan<uint32_t>(hit ? (uint32_t)nj : 0u, total, sm.red_u32);
  if (j < cg.K) cg.start[(size_t)unit * cg.K + j] = hit ? (int32_t)start : -1;
  if (tid == 0) {
    cg.total[unit] = (int32_t)total;
    if (count_opt) count_opt[unit] = (int32_t)total;
  }
}

// Members of hit cluster j of one query, copied into its list (and the
// optional caller copy); one workgroup per (query, cluster).
__global__ __launch_bounds__(kWG) void cl_gather_kernel(Geo g, ClGeo cg, const int32_t *__restrict__ offsets,
                                                        const int32_t *__restrict__ members,
                                                        int32_t *__restrict__ idx_opt, long long cap) {
  const int unit = blockIdx.x / cg.K, j = blockIdx.x % cg.K;
  const int32_t st = cg.start[(size_t)unit * cg.K + j];
  if (st < 0) return;
  const int br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int u = b * g.Hi + r / g.ig;
  const int32_t o0 = offsets[(size_t)u * (cg.K + 1) + j], o1 = offsets[(size_t)u * (cg.K + 1) + j + 1];
  int32_t *dst = cg.list + (size_t)unit * g.N;
  for (int32_t x = o0 + threadIdx.x; x < o1; x += kWG) {
    const int32_t pos = members[(size_t)u * g.N + x];
    const long long a = (long long)st + (x - o0);
    dst[a] = pos;
    if (idx_opt && a < cap) idx_opt[(size_t)unit * cap + a] = pos;
  }
}

}  // namespace

int launch_cluster_build(const Geo &g, const ClGeo &cg, const rtp_bf16 *k_idx, int iters, rtp_bf16 *cent,
                         int32_t *counts, int32_t *offsets, int32_t *members, hipStream_t s) {
  const unsigned nu = (unsigned)(g.B * g.Hi);
  if (nu == 0) return RTP_OK;
  const unsigned na = nu * (unsigned)cg.ntiles;
  hipLaunchKernelGGL(cl_init_kernel, dim3(nu), dim3(kWG), 0, s, g, cg, k_idx, cent);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(cl_assign_kernel<0>, dim3(na), dim3(kWG), 0, s, g, cg, k_idx, cent);
    hipLaunchKernelGGL(cl_update_kernel, dim3(nu), dim3(kWG), 0, s, g, cg, cent);
  }
  hipLaunchKernelGGL(cl_assign_kernel<1>, dim3(na), dim3(kWG), 0, s, g, cg, k_idx, cent);
  hipLaunchKernelGGL(cl_offsets_kernel, dim3(nu), dim3(kWG), 0, s, g, cg, counts, offsets);
  hipLaunchKernelGGL(cl_scatter_kernel, dim3(na), dim3(kWG), 0, s, g, cg, offsets, members);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

int launch_cluster_select(const Geo &g, const ClGeo &cg, const rtp_bf16 *q_pre, const rtp_bf16 *w_q,
                          const rtp_bf16 *cent, const int32_t *counts, const int32_t *offsets,
                          const int32_t *members, int32_t *idx_opt, int32_t *count_opt, long long cap, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  hipLaunchKernelGGL(cl_select_kernel, dim3((unsigned)g.units), dim3(kWG), 0, s, g, cg, q_pre, w_q, cent, counts,
                     count_opt);
  hipLaunchKernelGGL(cl_gather_kernel, dim3((unsigned)(g.units * cg.K)), dim3(kWG), 0, s, g, cg, offsets, members,
                     idx_opt, cap);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

int cluster_tile() { return kClTile; }

}  // namespace rtp
