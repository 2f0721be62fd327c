// Sliding-window attention with sinks (local heads) and sparse attention over
// given index sets (retrieval heads).
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2: local heads attend to a
// sliding window plus attention sinks; retrieval heads attend over their Top-P
// set, eq. (5): O = sum_{n in S} softmax(q . k_n / sqrt(d_h)) v_n with the
// post-RoPE query and keys.
//
// Both are HBM-bound gathers of bf16 rows.  16 lanes cover one 256-byte row
// (16 bytes each, coalesced); a wave holds 4 rows per step; split-K workgroups
// write softmax states that the last workgroup of each query combines.  An
// SWA workgroup serves up to four local q heads of one KV group, so a window
// row is read once for all of them (GQA); when a group has more local heads
// than that, the head blocks of one chunk are placed on the same XCD so the
// second read of a row hits that XCD's L2.
#include "block_util.h"

namespace rtp {

namespace {

constexpr float kScale = 0.08838834764831845f;   // 1 / sqrt(128)

struct SwaShared {
  float q[kSwaHeads][kD];
  float m[4][kSwaHeads], l[4][kSwaHeads];
  float o[4][kSwaHeads][kD];
  double2 rope[kD / 2];
  int heads[kSwaHeads];
  int flag;
  CombineShared cb;
};

// Position of window row ri for a query at m: sinks first, then the window.
__device__ __forceinline__ long long swa_row(long long ri, long long lo, long long ns) {
  return ri < ns ? ri : lo + (ri - ns);
}

__global__ __launch_bounds__(kWG) void swa_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                  const rtp_bf16 *__restrict__ kc,
                                                  const rtp_bf16 *__restrict__ vc, float *__restrict__ out) {
  __shared__ SwaShared sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, sub = lane & 15;
  // XCD-aware mapping: blocks x and x + 8 hold the head blocks of one chunk
  const int x = blockIdx.x, xcd = x & 7, y = x >> 3;
  const int hb = y % g.swa_hb, z = y / g.swa_hb;
  const long long chunk_id = (long long)z * 8 + xcd;          // over (unit, chunk)
  if (chunk_id >= (long long)g.swa_units * g.swa_nch) return;
  const int unit = (int)(chunk_id / g.swa_nch), ch = (int)(chunk_id % g.swa_nch);
  const int i = unit % g.nq, bl = unit / g.nq, lgi = bl % g.nlg, b = bl / g.nlg;
  const int kvg = g.lgroup[lgi];
  const long long m = g.N - g.nq + i;
  const long long lo = m - g.window + 1 > 0 ? m - g.window + 1 : 0;
  const long long ns = g.n_sink < lo ? g.n_sink : lo;
  const long long L = ns + (m - lo + 1);
  const long long r0 = (long long)ch * g.swa_chunk;
  const long long r1 = r0 + g.swa_chunk < L ? r0 + g.swa_chunk : L;

  // local heads of this block
  if (tid == 0) {
    int cnt = 0, seen = 0;
    for (int h = kvg * g.G; h < (kvg + 1) * g.G; ++h) {
      if (!((g.lmask[h >> 5] >> (h & 31)) & 1u)) continue;
      if (seen >= hb * kSwaHeads && cnt < kSwaHeads) sm.heads[cnt++] = h;
      ++seen;
    }
    for (int c = cnt; c < kSwaHeads; ++c) sm.heads[c] = -1;
  }
  rope_table(m, g.theta, sm.rope);       // ends with a barrier (also publishes sm.heads)
  for (int hh = 0; hh < kSwaHeads; ++hh) {
    const int h = sm.heads[hh];
    if (h >= 0) {
      rotate_query(q_pre + (((size_t)b * g.Hq + h) * g.nq + i) * kD, sm.rope, kScale, sm.q[hh]);
    } else {
      if (tid < kD) sm.q[hh][tid] = 0.f;
      __syncthreads();
    }
  }

  float q[kSwaHeads][8];
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[hh][e] = sm.q[hh][sub * 8 + e];
  float mm[kSwaHeads], ll[kSwaHeads], oo[kSwaHeads][8];
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh) {
    mm[hh] = -INFINITY;
    ll[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[hh][e] = 0.f;
  }
  const size_t cbase = ((size_t)b * g.Hkv + kvg) * g.Ncap * kD;
  const rtp_bf16 *kb = kc + cbase, *vb = vc + cbase;
  constexpr int U = 2;
  for (long long base = r0; base < r1; base += 16 * U) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long ri = base + u * 16 + wv * 4 + grp;
      ok[u] = ri < r1;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        const long long n = swa_row(ri, lo, ns);
        kr[u] = *reinterpret_cast<const uint4 *>(kb + n * kD + sub * 8);
        vr[u] = *reinterpret_cast<const uint4 *>(vb + n * kD + sub * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
      const uint32_t vw[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
      float kf[8], vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf_lo(kw[e]);
        kf[2 * e + 1] = bf_hi(kw[e]);
        vf[2 * e] = bf_lo(vw[e]);
        vf[2 * e + 1] = bf_hi(vw[e]);
      }
#pragma unroll
      for (int hh = 0; hh < kSwaHeads; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += q[hh][e] * kf[e];
        d = row16_sum(d);
        if (ok[u]) {
          const float mn = fmaxf(mm[hh], d);
          const float a = __expf(mm[hh] - mn), pw = __expf(d - mn);
          ll[hh] = ll[hh] * a + pw;
#pragma unroll
          for (int e = 0; e < 8; ++e) oo[hh][e] = oo[hh][e] * a + pw * vf[e];
          mm[hh] = mn;
        }
      }
    }
  }
  // merge row groups of the wave, then waves through LDS
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh) {
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(mm[hh], off), l2 = __shfl_xor(ll[hh], off);
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(oo[hh][e], off);
      merge_state(mm[hh], ll[hh], oo[hh], m2, l2, o2, 8);
    }
    if (grp == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.o[wv][hh][sub * 8 + e] = oo[hh][e];
      if (sub == 0) {
        sm.m[wv][hh] = mm[hh];
        sm.l[wv][hh] = ll[hh];
      }
    }
  }
  __syncthreads();
  // partials laid out [unit][head block][head][chunk]
  Partial *parts = g.swa_part + ((size_t)(unit * g.swa_hb + hb) * kSwaHeads) * g.swa_nch;
  for (int x2 = tid; x2 < kSwaHeads * kD; x2 += kWG) {
    const int hh = x2 / kD, d = x2 % kD;
    float m_ = -INFINITY, l_ = 0.f, o_ = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) merge_state(m_, l_, &o_, sm.m[w][hh], sm.l[w][hh], &sm.o[w][hh][d], 1);
    Partial *p = parts + (size_t)hh * g.swa_nch + ch;
    st_coherent(&p->o[d], o_);
    if (d == 0) {
      st_coherent(&p->m, m_);
      st_coherent(&p->l, l_);
    }
  }
  if (!arrive_last(g.ctr_swa + unit * g.swa_hb + hb, (uint32_t)g.swa_nch, &sm.flag)) return;
  for (int hh = 0; hh < kSwaHeads; ++hh) {
    const int h = sm.heads[hh];
    if (h < 0) continue;
    combine_partials(parts + (size_t)hh * g.swa_nch, g.swa_nch, out + (((size_t)b * g.Hq + h) * g.nq + i) * kD,
                     &sm.cb);
  }
}

struct SpShared {
  float q[kD];
  int list[1024];
  int flag;
  Partial extra;
  AttnShared at;
  double2 rope[kD / 2];
  CombineShared cb;
};

// Sparse attention over a given index list: one workgroup per (query, chunk).
__global__ __launch_bounds__(kWG) void sparse_attn_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                          const rtp_bf16 *__restrict__ kc,
                                                          const rtp_bf16 *__restrict__ vc,
                                                          const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ count, long long cap,
                                                          float *__restrict__ out) {
  __shared__ SpShared sm;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / kSpChunks, ch = blockIdx.x % kSpChunks;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int hq = g.rhead[r], kvg = hq / g.G;
  const long long m = g.N - g.nq + i;
  rope_table(m, g.theta, sm.rope);
  rotate_query(q_pre + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, sm.rope, kScale, sm.q);
  long long cnt = count[unit];
  if (cnt > cap) cnt = cap;
  if (cnt < 0) cnt = 0;
  const long long per = (cnt + kSpChunks - 1) / kSpChunks;
  const long long a0 = (long long)ch * per;
  const long long a1 = a0 + per < cnt ? a0 + per : cnt;
  const size_t cbase = ((size_t)b * g.Hkv + kvg) * g.Ncap * kD;
  // running state of this chunk: thread d < 128 holds channel d
  float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;
  for (long long s0 = a0; s0 < a1; s0 += 1024) {
    const int n = (int)(a1 - s0 < 1024 ? a1 - s0 : 1024);
    __syncthreads();
    for (int x = tid; x < n; x += kWG) sm.list[x] = idx[(size_t)unit * cap + s0 + x];
    __syncthreads();
    attend_rows(sm.q, sm.list, n, g.N, kc + cbase, vc + cbase, &sm.extra, &sm.at);
    if (tid < kD) merge_state(run_m, run_l, &run_o, sm.extra.m, sm.extra.l, &sm.extra.o[tid], 1);
  }
  Partial *dst = g.part + (size_t)unit * kSpChunks + ch;
  if (tid < kD) {
    st_coherent(&dst->o[tid], run_o);
    if (tid == 0) {
      st_coherent(&dst->m, run_m);
      st_coherent(&dst->l, run_l);
    }
  }
  if (!arrive_last(g.ctr_fin + unit, (uint32_t)kSpChunks, &sm.flag)) return;
  combine_partials(g.part + (size_t)unit * kSpChunks, kSpChunks, out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD,
                   &sm.cb);
}

}  // namespace

int launch_swa(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, float *out, hipStream_t s) {
  if (g.swa_units == 0) return RTP_OK;
  const long long chunks = (long long)g.swa_units * g.swa_nch;
  const long long z = (chunks + 7) / 8;
  const long long grid = z * 8 * g.swa_hb;
  hipLaunchKernelGGL(swa_kernel, dim3((unsigned)grid), dim3(kWG), 0, s, g, q_pre, k, v, out);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

int launch_sparse_attn(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v, const int32_t *idx,
                       const int32_t *count, long long cap, float *out, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3((unsigned)((long long)g.units * kSpChunks)), dim3(kWG), 0, s, g, q_pre,
                     k, v, idx, count, cap, out);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace rtp
