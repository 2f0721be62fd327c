// Workgroup-wide scans and reductions for 256-thread (4 x wave64) workgroups,
// and the split-K attention building blocks shared by the attention kernels.
//
// Attention: "Full Attention Strikes Back" (RTPurbo) section 3.2 eq. (5),
// softmax(q . k / sqrt(d_h)) weighted sum of v over a row set.
#pragma once

#include <type_traits>

#include "rtp_internal.h"

namespace rtp {

// Exclusive prefix of v over the workgroup in thread order; `total` receives
// the sum.  s_buf needs 4 entries and is reused after the call returns.
template <typename V>
__device__ __forceinline__ V block_excl_scan(V v, V &total, V *s_buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  V x = v;
  if constexpr (sizeof(V) == 4 && std::is_integral<V>::value) {
    x = (V)wave_incl_scan_u32((uint32_t)v);
  } else if constexpr (sizeof(V) == 8) {
    x = wave_incl_scan64(v);
  } else {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const V y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
  }
  if (lane == 63) s_buf[w] = x;
  __syncthreads();
  V base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) base += s_buf[i];
    tot += s_buf[i];
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// Wave-wide reduction of a 32-bit value with DPP: within each row of 16
// (quad swaps, half-row and row mirrors), then row 0 into row 1 and row 2 into
// row 3 (row broadcast 15), then rows 0-1 into rows 2-3 (row broadcast 31);
// lane 63 ends with the result.  Lanes whose source is absent keep their value.
template <int CTRL, int RMASK, typename V>
__device__ __forceinline__ V dpp_keep(V x) {
  const int xi = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(V, __builtin_amdgcn_update_dpp(xi, xi, CTRL, RMASK, 0xF, false));
}

template <typename V, typename Op>
__device__ __forceinline__ V wave_reduce(V v, Op op) {
  v = op(v, dpp_keep<0xB1, 0xF>(v));
  v = op(v, dpp_keep<0x4E, 0xF>(v));
  v = op(v, dpp_keep<0x141, 0xF>(v));
  v = op(v, dpp_keep<0x140, 0xF>(v));
  v = op(v, dpp_keep<0x142, 0xA>(v));
  v = op(v, dpp_keep<0x143, 0xC>(v));
  return __builtin_bit_cast(V, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <typename V>
__device__ __forceinline__ V block_max(V v, V *s_buf) {
  static_assert(sizeof(V) == 4, "32-bit values");
  v = wave_reduce(v, [](V a, V b) { return b > a ? b : a; });
  if ((threadIdx.x & 63) == 0) s_buf[threadIdx.x >> 6] = v;
  __syncthreads();
  V r = s_buf[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) r = s_buf[i] > r ? s_buf[i] : r;
  __syncthreads();
  return r;
}

template <typename V>
__device__ __forceinline__ V block_min(V v, V *s_buf) {
  static_assert(sizeof(V) == 4, "32-bit values");
  v = wave_reduce(v, [](V a, V b) { return b < a ? b : a; });
  if ((threadIdx.x & 63) == 0) s_buf[threadIdx.x >> 6] = v;
  __syncthreads();
  V r = s_buf[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) r = s_buf[i] < r ? s_buf[i] : r;
  __syncthreads();
  return r;
}

// Maximum of a and minimum of b over the workgroup with one pair of barriers.
__device__ __forceinline__ void block_max_min(float &a, int &b, float *s_f, int *s_i) {
  a = wave_reduce(a, [](float x, float y) { return fmaxf(x, y); });
  b = wave_reduce(b, [](int x, int y) { return y < x ? y : x; });
  if ((threadIdx.x & 63) == 0) {
    s_f[threadIdx.x >> 6] = a;
    s_i[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  a = fmaxf(fmaxf(s_f[0], s_f[1]), fmaxf(s_f[2], s_f[3]));
  b = min(min(s_i[0], s_i[1]), min(s_i[2], s_i[3]));
  __syncthreads();
}

// Handoff between the workgroups of one kernel without agent-scope release
// fences: such a fence writes back the whole L2 of the XCD, and those
// writebacks serialise across the GPU (about 0.2 us each).  Instead, every
// result that another workgroup of the same kernel reads is published with a
// coherent store (agent-scope relaxed atomic: written through the L2), each
// thread waits for its stores to complete, and the workgroup then counts in
// with a relaxed atomic.  Only the last workgroup to arrive performs an
// agent-scope acquire (an L2 invalidate) before reading the others' results.
template <typename V>
__device__ __forceinline__ void st_coherent(V *p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in exactly one workgroup of a group of n (the last to arrive),
// which may then read every result the others published with st_coherent.
// The counter is left at zero for the next call.
__device__ __forceinline__ bool arrive_last(uint32_t *ctr, uint32_t n, int *s_flag) {
  __builtin_amdgcn_s_waitcnt(0);          // this thread's coherent stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == n - 1;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Copies a softmax state from LDS to global memory with coherent stores.
__device__ __forceinline__ void publish_partial(Partial *dst, const Partial *src) {
  const int t = threadIdx.x;
  if (t < kD) st_coherent(&dst->o[t], src->o[t]);
  if (t == kD) st_coherent(&dst->m, src->m);
  if (t == kD + 1) st_coherent(&dst->l, src->l);
}

// cos/sin of m * theta_i (FASB eq. (1)) in fp64 for the 64 channel pairs,
// into tab[64] (x = cos, y = sin).  Threads 0..63; ends with a barrier.
// Sine and cosine of the RoPE angle m * theta_pair in fp64: the angle is
// reduced by 2 pi (three-part constant, fused multiply-adds) so that sin/cos
// take their short-argument path at any position.
__device__ __forceinline__ void rope_sincos(long long m, double theta, int pair, double &sn, double &cs) {
  const double x = (double)m * rope_freq(theta, pair);
  const double k = rint(x * 0.15915494309189535);
  double y = fma(-k, 6.283185307179586232, x);
  y = fma(-k, 2.4492935982947064e-16, y);
  y = fma(-k, -5.9895396194366793e-33, y);
  sincos(y, &sn, &cs);
}

__device__ __forceinline__ void rope_table(long long m, double theta, double2 *tab) {
  const int t = threadIdx.x;
  if (t < kD / 2) {
    double sn, cs;
    rope_sincos(m, theta, t, sn, cs);
    tab[t] = make_double2(cs, sn);
  }
  __syncthreads();
}

// q_rot = R(m) q_pre with a table from rope_table, scaled, into dst[128].
// Threads 0..63 rotate one channel pair each; ends with a barrier.
__device__ __forceinline__ void rotate_query(const rtp_bf16 *q_row, const double2 *tab, float scale, float *dst) {
  const int t = threadIdx.x;
  if (t < kD / 2) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(q_row)[t];
    const double a = (double)bf_lo(w), b = (double)bf_hi(w);
    const double cs = tab[t].x, sn = tab[t].y;
    dst[2 * t] = (float)(a * cs - b * sn) * scale;
    dst[2 * t + 1] = (float)(a * sn + b * cs) * scale;
  }
  __syncthreads();
}

struct AttnShared {
  float m[4], l[4];
  float o[4][kD];
};

// Softmax state of one (pre-scaled) query over rows[0..cnt) of K/V rows at
// base + n * D.  Rows outside [0, nmax) are skipped.  16 lanes cover one row
// (8 channels each), a wave holds 4 rows per step.  The workgroup's state is
// written to *dst (m, l and the unnormalised o).  Ends with a barrier.
// STREAM: the rows are read once per call (non-temporal loads); otherwise
// they are cached (many queries of a chunked prefill gather from the same
// K/V group, which then stays in the L2 and the Infinity Cache).
template <bool STREAM = true>
__device__ __forceinline__ void attend_rows(const float *q_s, const int *rows, int cnt, long long nmax,
                                            const rtp_bf16 *__restrict__ kb, const rtp_bf16 *__restrict__ vb,
                                            Partial *dst, AttnShared *sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, grp = lane >> 4, sub = lane & 15;
  // scores in base 2 (the query carries log2(e)); the reference maximum m
  // moves only when a score passes it by more than 8 (any reference gives the
  // same o / l, this one keeps every weight below 2^8), for the whole wave at
  // once, so a row costs one exponential and one FMA per channel
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = q_s[sub * 8 + i] * 1.4426950408889634f;
  float m = -1.0e30f, l = 0.f, o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  // U rows in flight per 16-lane group (80 per workgroup), a rolling window:
  // slot u is refilled with the row U slots ahead as soon as it is consumed
  constexpr int U = 5;
  uint4 kr[U], vr[U];
  bool ok[U];
  auto fetch = [&](int u, int ri) {
    const long long n = ri < cnt ? (long long)rows[ri] : -1;
    ok[u] = n >= 0 && n < nmax;
    kr[u] = make_uint4(0, 0, 0, 0);
    vr[u] = make_uint4(0, 0, 0, 0);
    if (ok[u]) {
      if (STREAM) {
        kr[u] = ld_stream(kb + n * kD + sub * 8);
        vr[u] = ld_stream(vb + n * kD + sub * 8);
      } else {
        kr[u] = *reinterpret_cast<const uint4 *>(kb + n * kD + sub * 8);
        vr[u] = *reinterpret_cast<const uint4 *>(vb + n * kD + sub * 8);
      }
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) fetch(u, u * 16 + wv * 4 + grp);
  for (int base = 0; base < cnt; base += 16 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
      const uint32_t vw[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
      const bool oku = ok[u];
      float d = q[0] * bf_lo(kw[0]);
      d = fmaf(q[1], bf_hi(kw[0]), d);
#pragma unroll
      for (int i = 1; i < 4; ++i) d = fmaf(q[2 * i + 1], bf_hi(kw[i]), fmaf(q[2 * i], bf_lo(kw[i]), d));
      d = row16_sum(d);
      if (oku) {
        const bool bump = d > m + 8.f;
        if (__builtin_amdgcn_ballot_w64(bump)) {
          const float mn = bump ? d : m;
          const float a = __builtin_amdgcn_exp2f(m - mn);
          l *= a;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] *= a;
          m = mn;
        }
        const float pw = __builtin_amdgcn_exp2f(d - m);
        l += pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = fmaf(pw, bf_lo(vw[i]), o[2 * i]);
          o[2 * i + 1] = fmaf(pw, bf_hi(vw[i]), o[2 * i + 1]);
        }
      }
      fetch(u, base + (U + u) * 16 + wv * 4 + grp);
    }
  }
  // back to natural-log units for the merges (an empty state has m = -inf)
  m = l > 0.f ? m * 0.6931471805599453f : -INFINITY;
  // merge the 4 row groups of the wave
  {
    float o2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o2[i] = lane_xor<16>(o[i]);
    merge_state(m, l, o, lane_xor<16>(m), lane_xor<16>(l), o2, 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) o2[i] = lane_xor<32>(o[i]);
    merge_state(m, l, o, lane_xor<32>(m), lane_xor<32>(l), o2, 8);
  }
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sm->o[wv][sub * 8 + i] = o[i];
    if (sub == 0) {
      sm->m[wv] = m;
      sm->l[wv] = l;
    }
  }
  __syncthreads();
  if (threadIdx.x < kD) {
    const int d = threadIdx.x;
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) merge_state(mm, ll, &oo, sm->m[w], sm->l[w], &sm->o[w][d], 1);
    dst->o[d] = oo;
    if (d == 0) {
      dst->m = mm;
      dst->l = ll;
    }
  }
  __syncthreads();
}

struct CombineShared {
  float red[8][kD];
  float m8[8], l8[8];
};

// Normalised combination of np split-K states into out[0..D) by the whole
// workgroup, in one round of loads for up to 64 states: 8 groups of 32
// threads, group x merging states x, x + 8, ... (a float4 of channels per
// thread, eight states in flight), then the 8 group states merged in a fixed
// order.
__device__ __forceinline__ void combine_partials(const Partial *parts, int np, float *out, CombineShared *sm) {
  const int tid = threadIdx.x, d4 = tid & 31, grp = tid >> 5;
  float m = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int x0 = grp; x0 < np; x0 += 64) {
    float pm[8], pl[8];
    float4 po[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {          // clamped, unconditional loads: up to 64 states in one round
      const int x = x0 + 8 * u < np ? x0 + 8 * u : np - 1;
      pm[u] = parts[x].m;
      pl[u] = parts[x].l;
      po[u] = reinterpret_cast<const float4 *>(parts[x].o)[d4];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (x0 + 8 * u >= np) break;
      const float o2[4] = {po[u].x, po[u].y, po[u].z, po[u].w};
      merge_state(m, l, o, pm[u], pl[u], o2, 4);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) sm->red[grp][4 * d4 + c] = o[c];
  if (d4 == 0) {
    sm->m8[grp] = m;
    sm->l8[grp] = l;
  }
  __syncthreads();
  if (tid < kD) {
    float mm = -INFINITY, ll = 0.f, oo = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) merge_state(mm, ll, &oo, sm->m8[x], sm->l8[x], &sm->red[x][tid], 1);
    out[tid] = ll > 0.f ? oo / ll : 0.f;
  }
  __syncthreads();
}

// Normalised combination of np split-K states into out[0..D) by one wave:
// lane l holds channels 2l and 2l + 1; sixteen states are loaded per round and
// merged in index order.
__device__ __forceinline__ void wave_combine(const Partial *parts, int np, float *out) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY, l = 0.f, o[2] = {0.f, 0.f};
  for (int x0 = 0; x0 < np; x0 += 16) {
    float pm[16], pl[16];
    float2 po[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {         // clamped, unconditional loads
      const int x = x0 + u < np ? x0 + u : np - 1;
      pm[u] = parts[x].m;
      pl[u] = parts[x].l;
      po[u] = reinterpret_cast<const float2 *>(parts[x].o)[lane];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float o2[2] = {po[u].x, po[u].y};
      if (x0 + u < np) merge_state(m, l, o, pm[u], pl[u], o2, 2);
    }
  }
  out[2 * lane] = l > 0.f ? o[0] / l : 0.f;
  out[2 * lane + 1] = l > 0.f ? o[1] / l : 0.f;
}

}  // namespace rtp
