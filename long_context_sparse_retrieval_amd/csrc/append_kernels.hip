// Cache append: the post-RoPE keys, the values and the indexer keys of new
// positions written in one launch.
//
// "Full Attention Strikes Back" (RTPurbo) section 2.2 eq. (1): the key cache
// holds R(n) k_n; section 3.2 eq. (4): each indexer-key head caches the rank-16
// projection of the pre-RoPE key, W_k k_n.  Both come from the same new key
// row, so one pass reads it once for every cache it feeds.
//
// Two mappings.  A decode step appends one token (or a few): one workgroup per
// (sequence, new row), a thread per (KV group, channel pair) and per
// (indexer-key head, output), so the 128-term projections run side by side.
// A bulk append (prefill of the caches) takes 256 new rows of one KV group per
// workgroup: each thread holds one row and projects it for every indexer-key
// head of the group in turn, the head's matrix widened to fp64 in LDS once
// and read as broadcasts.  Both accumulate the 128
// products in fp64 in channel order and round once, so their bits agree with
// rtp_rope_keys / rtp_index_keys.
#include "rtp_internal.h"

namespace rtp {

namespace {

constexpr int kApRows = kWG;       // new rows per bulk workgroup (one per thread in the projections)
constexpr int kApSmall = 8;        // appends of at most this many rows use the per-row mapping
constexpr int kApKvBatch = 8;      // KV groups whose rows are loaded together

__device__ __forceinline__ double bf16_val(rtp_bf16 v) { return (double)__uint_as_float((uint32_t)v << 16); }

// Post-RoPE key and value of KV groups kv0 .. kv0 + kApKvBatch - 1 at new row t
// (position n), channel pair `pair`; loads first, then the stores.  RING: the
// layer has ring groups (without them the rows follow the plain
// [B, Hkv, Ncap, D] stride and no ring lookup is made).
template <bool RING>
__device__ __forceinline__ void append_kv_pairs(const Geo &g, const rtp_bf16 *__restrict__ k_new,
                                                const rtp_bf16 *__restrict__ v_new, rtp_bf16 *__restrict__ kc,
                                                rtp_bf16 *__restrict__ vc, int b, int kv0, long long t,
                                                long long n_new, long long n, long long n_end, int pair,
                                                double sn, double cs) {
  uint32_t kw[kApKvBatch], vw[kApKvBatch];
#pragma unroll
  for (int u = 0; u < kApKvBatch; ++u) {
    const int kv = kv0 + u < g.Hkv ? kv0 + u : g.Hkv - 1;           // clamped, unconditional loads
    const size_t src = (((size_t)b * g.Hkv + kv) * n_new + t) * kD + 2 * pair;
    kw[u] = *reinterpret_cast<const uint32_t *>(k_new + src);
    vw[u] = *reinterpret_cast<const uint32_t *>(v_new + src);
  }
#pragma unroll
  for (int u = 0; u < kApKvBatch; ++u) {
    const bool ring = RING && kv0 + u < g.Hkv && kv_is_ring(g, kv0 + u);
    if (kv0 + u < g.Hkv && (!RING || kv_keep(g, ring, n, n_end))) {
      const size_t row = RING ? kv_group_base(g, b, kv0 + u) + kv_row(g, ring, n)
                              : ((size_t)b * g.Hkv + kv0 + u) * g.Ncap + n;
      const size_t dst = row * kD + 2 * pair;
      *reinterpret_cast<uint32_t *>(kc + dst) = rope_pair_bf16(kw[u], sn, cs);
      *reinterpret_cast<uint32_t *>(vc + dst) = vw[u];
    }
  }
}

// A few new rows: one workgroup per (sequence, new row).  Every load a thread
// needs is issued before its first use, so the projection costs one memory
// round trip and a 128-deep FMA chain.
template <bool RING>
__global__ __launch_bounds__(kWG) void append_small_kernel(Geo g, const rtp_bf16 *__restrict__ k_new,
                                                           const rtp_bf16 *__restrict__ v_new,
                                                           const rtp_bf16 *__restrict__ w_k, rtp_bf16 *__restrict__ kc,
                                                           rtp_bf16 *__restrict__ vc, rtp_bf16 *__restrict__ k_idx,
                                                           long long n0, long long n_new) {
  const int tid = threadIdx.x;
  const int b = (int)(blockIdx.x / n_new);
  const long long t = blockIdx.x % n_new, n = n0 + t;
  // keys and values: thread (batch of KV groups, channel pair)
  const int pair = tid & 63;
  double sn, cs;
  sincos((double)n * rope_freq(g.theta, pair), &sn, &cs);
  for (int kv0 = (tid >> 6) * kApKvBatch; kv0 < g.Hkv; kv0 += 4 * kApKvBatch)
    append_kv_pairs<RING>(g, k_new, v_new, kc, vc, b, kv0, t, n_new, n, n0 + n_new, pair, sn, cs);
  // indexer keys: thread (indexer-key head, output channel)
  for (int x = tid; x < g.Hi * kR; x += kWG) {
    const int i = x / kR, j = x % kR;
    const int kv = g.rhead[i * g.ig] / g.G;
    const uint4 *xr = reinterpret_cast<const uint4 *>(k_new + (((size_t)b * g.Hkv + kv) * n_new + t) * kD);
    const rtp_bf16 *wc = w_k + (size_t)i * kD * kR + j;
    uint4 xv[kD / 8];
    rtp_bf16 wv[kD];
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) xv[c] = xr[c];
#pragma unroll
    for (int c = 0; c < kD; ++c) wv[c] = wc[c * kR];
    const uint32_t *xw = &xv[0].x;
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < kD; ++c) {
      const float xf = (c & 1) ? bf_hi(xw[c >> 1]) : bf_lo(xw[c >> 1]);
      acc = fma((double)xf, bf16_val(wv[c]), acc);
    }
    k_idx[(((size_t)b * g.Hi + i) * g.Ncap + n) * kR + j] = f64_to_bf16(acc);
  }
}

// Bulk append: one workgroup per (sequence, KV group, run of kApRows new rows).
struct AppendShared {
  double w[kD][kR];                        // one indexer-key head's matrix, widened
};

template <bool RING>
__global__ __launch_bounds__(kWG) void append_bulk_kernel(Geo g, const rtp_bf16 *__restrict__ k_new,
                                                          const rtp_bf16 *__restrict__ v_new,
                                                          const rtp_bf16 *__restrict__ w_k, rtp_bf16 *__restrict__ kc,
                                                          rtp_bf16 *__restrict__ vc, rtp_bf16 *__restrict__ k_idx,
                                                          long long n0, long long n_new) {
  __shared__ AppendShared sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the runs of one (sequence, KV group) are consecutive workgroups: a
  // retrieval group's rows stay in L2 while its heads re-read them (measured
  // faster than interleaving the groups)
  const long long bpb = (n_new + kApRows - 1) / kApRows;
  const int bg = (int)(blockIdx.x / bpb), blk = (int)(blockIdx.x % bpb);
  const int b = bg / g.Hkv, kv = bg % g.Hkv;
  const long long t0 = (long long)blk * kApRows;
  const int nr = (int)(n_new - t0 < kApRows ? n_new - t0 : kApRows);
  const size_t src0 = ((size_t)bg * n_new + t0) * kD;                 // first new row of this block
  const bool ring = RING && kv_is_ring(g, kv);
  const size_t gbase = RING ? kv_group_base(g, b, kv) * kD : (size_t)bg * g.Ncap * kD;
  // indexer-key heads fed by this KV group: a contiguous range [i0, i1)
  int i0 = g.Hi, i1 = g.Hi;
  for (int i = 0; i < g.Hi; ++i) {
    const bool mine = g.rhead[i * g.ig] / g.G == kv;
    if (mine && i0 == g.Hi) i0 = i;
    if (!mine && i0 < g.Hi && i1 == g.Hi) i1 = i;
  }
  // keys and values: wave wv takes rows wv * 64 .. wv * 64 + 63, four at a time; lane = channel pair
  const double th = rope_freq(g.theta, lane);
  for (int r0 = wv * 64; r0 < wv * 64 + 64 && r0 < nr; r0 += 4) {
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u < nr ? r0 + u : nr - 1;
      kw[u] = *reinterpret_cast<const uint32_t *>(k_new + src0 + (size_t)r * kD + 2 * lane);
      vw[u] = *reinterpret_cast<const uint32_t *>(v_new + src0 + (size_t)r * kD + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long n = n0 + t0 + r0 + u;
      if (r0 + u < nr && (!RING || kv_keep(g, ring, n, n0 + n_new))) {
        double sn, cs;
        sincos((double)n * th, &sn, &cs);
        const size_t dst = gbase + (size_t)(RING ? kv_row(g, ring, n) : n) * kD + 2 * lane;
        *reinterpret_cast<uint32_t *>(kc + dst) = rope_pair_bf16(kw[u], sn, cs);
        *reinterpret_cast<uint32_t *>(vc + dst) = vw[u];
      }
    }
  }
  // indexer keys: thread = row; the head's matrix is widened into LDS once and
  // read as broadcasts; the row streams in 16-byte steps, four steps ahead
  const uint4 *xr = reinterpret_cast<const uint4 *>(k_new + src0 + (size_t)(tid < nr ? tid : nr - 1) * kD);
  for (int i = i0; i < i1; ++i) {
    uint4 x0 = xr[0], x1 = xr[1], x2 = xr[2], x3 = xr[3];
    __syncthreads();                                      // the previous head's matrix is no longer read
    {
      const uint4 w8 = reinterpret_cast<const uint4 *>(w_k + (size_t)i * kD * kR)[tid];   // 8 of 2048
      const uint32_t ww[4] = {w8.x, w8.y, w8.z, w8.w};
      double *dst = &sm.w[0][0] + 8 * tid;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = (double)bf_lo(ww[e]);
        dst[2 * e + 1] = (double)bf_hi(ww[e]);
      }
    }
    __syncthreads();
    double acc[kR];
#pragma unroll
    for (int j = 0; j < kR; ++j) acc[j] = 0.0;
    // channels 8 c8 .. 8 c8 + 7 of the row (in x4) against the matrix rows in LDS
    auto step = [&](const uint4 &x4, int c8) {
      const uint32_t xw[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const double xf = (double)((cc & 1) ? bf_hi(xw[cc >> 1]) : bf_lo(xw[cc >> 1]));
        const double2 *wr = reinterpret_cast<const double2 *>(sm.w[c8 * 8 + cc]);
#pragma unroll
        for (int j2 = 0; j2 < kR / 2; ++j2) {
          const double2 w2 = wr[j2];
          acc[2 * j2] = fma(xf, w2.x, acc[2 * j2]);
          acc[2 * j2 + 1] = fma(xf, w2.y, acc[2 * j2 + 1]);
        }
      }
    };
#pragma unroll 1
    for (int c8 = 0; c8 < kD / 8; c8 += 4) {
      const int nx = c8 + 4 < kD / 8 ? c8 + 4 : c8;        // the next four steps (clamped at the end)
      const uint4 y0 = xr[nx], y1 = xr[nx + 1], y2 = xr[nx + 2], y3 = xr[nx + 3];
      step(x0, c8);
      step(x1, c8 + 1);
      step(x2, c8 + 2);
      step(x3, c8 + 3);
      x0 = y0;
      x1 = y1;
      x2 = y2;
      x3 = y3;
    }
    if (tid < nr) {
      uint32_t o[kR / 2];
#pragma unroll
      for (int j2 = 0; j2 < kR / 2; ++j2)
        o[j2] = (uint32_t)f64_to_bf16(acc[2 * j2]) | ((uint32_t)f64_to_bf16(acc[2 * j2 + 1]) << 16);
      uint4 *dst = reinterpret_cast<uint4 *>(k_idx + (((size_t)b * g.Hi + i) * g.Ncap + n0 + t0 + tid) * kR);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

}  // namespace

int launch_append_kv(const Geo &g, const rtp_bf16 *k_new, const rtp_bf16 *v_new, const rtp_bf16 *w_k, rtp_bf16 *kc,
                     rtp_bf16 *vc, rtp_bf16 *k_idx, long long n0, long long n_new, hipStream_t s) {
  if (n_new == 0) return RTP_OK;
  const dim3 small_grid((unsigned)(g.B * n_new));
  const dim3 bulk_grid((unsigned)((long long)g.B * g.Hkv * ((n_new + kApRows - 1) / kApRows)));  // runs per (b, group)
  if (n_new <= kApSmall && g.any_ring)
    hipLaunchKernelGGL(append_small_kernel<true>, small_grid, dim3(kWG), 0, s, g, k_new, v_new, w_k, kc, vc, k_idx,
                       n0, n_new);
  else if (n_new <= kApSmall)
    hipLaunchKernelGGL(append_small_kernel<false>, small_grid, dim3(kWG), 0, s, g, k_new, v_new, w_k, kc, vc, k_idx,
                       n0, n_new);
  else if (g.any_ring)
    hipLaunchKernelGGL(append_bulk_kernel<true>, bulk_grid, dim3(kWG), 0, s, g, k_new, v_new, w_k, kc, vc, k_idx,
                       n0, n_new);
  else
    hipLaunchKernelGGL(append_bulk_kernel<false>, bulk_grid, dim3(kWG), 0, s, g, k_new, v_new, w_k, kc, vc, k_idx,
                       n0, n_new);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace rtp
