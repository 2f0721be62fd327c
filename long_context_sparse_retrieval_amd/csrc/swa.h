// Sliding-window attention with attention sinks for the local heads, as
// workgroups that run inside the scan launch (their latency hides under the
// indexer stream) or on their own.
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2: local heads attend, in
// prefill and decode alike, to a sliding window plus attention sinks; the
// attention itself is eq. (5)'s softmax(q . k / sqrt(d_h)) over those rows.
//
// A workgroup serves up to four local q heads of one KV group over one chunk
// of window rows, so a K/V row is read once for all of them (GQA).  16 lanes
// cover one 256-byte row (16 bytes each, coalesced); every lane group keeps
// four rows in flight, so a 64-row chunk is requested in one round.  Chunk
// states are combined by the last workgroup of each (sequence, group, query),
// one wave per head.
#pragma once

#include "block_util.h"

namespace rtp {

constexpr float kInvSqrtD = 0.08838834764831845f;   // 1 / sqrt(128)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kScoreFloor = -1.0e30f;               // initial reference maximum (base 2)
constexpr float kSlack = 8.0f;                        // base-2 headroom before the reference moves

struct SwaShared {
  float q[kSwaHeads][kD];
  float m[4][kSwaHeads], l[4][kSwaHeads];
  float o[4][kSwaHeads][kD];
  double2 rope[kD / 2];
  int heads[kSwaHeads];
  int flag;
};

// The k-th local q head of KV group kvg (ascending head index), or -1.
__device__ __forceinline__ int local_head(const Geo &g, int kvg, int k) {
  int seen = 0;
  for (int h = kvg * g.G; h < (kvg + 1) * g.G; ++h) {
    if (!((g.lmask[h >> 5] >> (h & 31)) & 1u)) continue;
    if (seen == k) return h;
    ++seen;
  }
  return -1;
}

// Cache row of window row ri: the ns sinks first (row = position), then the
// window, whose j-th position lies in row wbase + j of a full group (wbase =
// its first position), and for a ring group in row wbase + j, less W once
// j >= wwrap (the rows wrap; the window spans at most W positions, so once).
// Positions and ring rows stay below 2^31, so 32-bit arithmetic holds.
template <bool RING>
__device__ __forceinline__ int swa_row(int ri, int ns, int wbase, int wwrap, int W) {
  const int j = ri - ns;
  if (!RING) return ri < ns ? ri : wbase + j;
  return ri < ns ? ri : (j < wwrap ? wbase : wbase - W) + j;
}

// Number of SWA workgroups of a launch (a multiple of 8 for the XCD mapping).
__host__ __device__ __forceinline__ long long swa_blocks(const Geo &g) {
  const long long chunks = (long long)g.swa_units * g.swa_nch;
  return (chunks + 7) / 8 * 8 * g.swa_hb;
}

// One SWA workgroup; x = its index among the SWA workgroups of the launch.
// RING: the block's KV group is stored as a ring (rows wrap); RING_LAYOUT:
// the layer has ring groups (group bases follow the ring layout).
// defer: publish the chunk states only (a later launch merges them).
template <bool RING, bool RING_LAYOUT>
__device__ __forceinline__ void swa_block_rows(const Geo &g, long long x, const rtp_bf16 *__restrict__ q_pre,
                                               const rtp_bf16 *__restrict__ kc, const rtp_bf16 *__restrict__ vc,
                                               float *__restrict__ out, SwaShared &sm, bool defer) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = lane >> 4, sub = lane & 15;
  // XCD-aware mapping: blocks x and x + 8 hold the head blocks of one chunk (same XCD)
  const long long xcd = x & 7, y = x >> 3;
  const int hb = (int)(y % g.swa_hb);
  const long long chunk_id = (y / g.swa_hb) * 8 + xcd;     // over (unit, chunk)
  if (chunk_id >= (long long)g.swa_units * g.swa_nch) return;
  const int unit = (int)(chunk_id / g.swa_nch), ch = (int)(chunk_id % g.swa_nch);
  const int i = unit % g.nq, bl = unit / g.nq, lgi = bl % g.nlg, b = bl / g.nlg;
  const int kvg = g.lgroup[lgi];
  const int m = (int)(g.N - g.nq + i);          // N < 2^31
  const int lo = m - g.window + 1 > 0 ? m - g.window + 1 : 0;
  const int ns = g.n_sink < lo ? g.n_sink : lo;
  const int L = ns + (m - lo + 1);
  const int r0 = ch * g.swa_chunk;
  const int r1 = r0 + g.swa_chunk < L ? r0 + g.swa_chunk : L;
  const size_t cbase = kv_group_elems<RING_LAYOUT>(g, b, kvg);
  const rtp_bf16 *kb = kc + cbase, *vb = vc + cbase;
  // one query per sequence reads its window once (non-temporal loads); with
  // many queries (chunked prefill) consecutive queries share almost every row,
  // which then stays cached
  const bool stream = g.nq == 1;
  auto ld_row = [&](const rtp_bf16 *p) -> uint4 {
    return stream ? ld_stream(p) : *reinterpret_cast<const uint4 *>(p);
  };
  // window rows: positions lo.. in rows lo.. of a full group; in a ring group
  // position n >= n_sink sits in row n_sink + (n - n_sink) mod W (below n_sink
  // and, when lo < n_sink, everywhere in the window that is row n as well)
  int wbase = lo, wwrap = INT_MAX;
  if (RING && lo >= g.n_sink) {
    const int r_lo = (lo - g.n_sink) % g.window;
    wbase = g.n_sink + r_lo;
    wwrap = g.window - r_lo;
  }

  // request the first rows before preparing the queries
  constexpr int U = 3;
  uint4 kr[U], vr[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ri = r0 + u * 16 + wv * 4 + grp;
    ok[u] = ri < r1;
    kr[u] = vr[u] = make_uint4(0, 0, 0, 0);
    if (ok[u]) {
      const size_t n = (size_t)swa_row<RING>(ri, ns, wbase, wwrap, g.window);
      kr[u] = ld_row(kb + n * kD + sub * 8);
      vr[u] = ld_row(vb + n * kD + sub * 8);
    }
  }
  // every head's query in one round: thread (hh, t) loads and rotates channel
  // pair t of the hh-th local head of this head block (threads 0..63 also
  // build the RoPE table of position m)
  const int hh_mine = tid >> 6, pt = tid & 63;
  const int h_mine = local_head(g, kvg, hb * kSwaHeads + hh_mine);
  uint32_t qw = 0;
  if (h_mine >= 0)
    qw = reinterpret_cast<const uint32_t *>(q_pre + (((size_t)b * g.Hq + h_mine) * g.nq + i) * kD)[pt];
  rope_table(m, g.theta, sm.rope);       // ends with a barrier
  {
    const double a = (double)bf_lo(qw), c2 = (double)bf_hi(qw);
    const double cs = sm.rope[pt].x, sn = sm.rope[pt].y;
    sm.q[hh_mine][2 * pt] = h_mine >= 0 ? (float)(a * cs - c2 * sn) * kInvSqrtD : 0.f;
    sm.q[hh_mine][2 * pt + 1] = h_mine >= 0 ? (float)(a * sn + c2 * cs) * kInvSqrtD : 0.f;
    if (pt == 0) sm.heads[hh_mine] = h_mine;
  }
  __syncthreads();
  // scores in base 2: the query carries log2(e), so a weight is one v_exp
  float q[kSwaHeads][8];
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[hh][e] = sm.q[hh][sub * 8 + e] * kLog2e;
  // running state per head: reference maximum (base 2; starts at a finite
  // floor so an empty lane group needs no special case), sum, output
  float mm[kSwaHeads], ll[kSwaHeads], oo[kSwaHeads][8];
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh) {
    mm[hh] = kScoreFloor;
    ll[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[hh][e] = 0.f;
  }
  // rolling window: slot u is refilled with the row 16 U ahead as soon as it
  // is used, so about U rows per lane group stay in flight throughout
  for (int base = r0; base < r1; base += 16 * U) {
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
      // every head's score, then the four lane-group sums interleaved
      float d[kSwaHeads];
#pragma unroll
      for (int hh = 0; hh < kSwaHeads; ++hh) {
        float x = q[hh][0] * kf[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) x = fmaf(q[hh][e], kf[e], x);
        d[hh] = x;
      }
      row16_sum_n(d);
      // online softmax with a lazy reference: a head's maximum moves only
      // when a score passes it by more than kSlack (any reference gives the
      // same o / l; this one keeps every weight below 2^kSlack).  One test
      // for the wave and its four heads; a head that does not move is scaled
      // by exp2(0) = 1, exactly.  A row past the chunk adds nothing.
      const bool oku = ok[u];
      float rise = d[0] - mm[0];
#pragma unroll
      for (int hh = 1; hh < kSwaHeads; ++hh) rise = fmaxf(rise, d[hh] - mm[hh]);
      if (__builtin_amdgcn_ballot_w64(oku && rise > kSlack)) {
#pragma unroll
        for (int hh = 0; hh < kSwaHeads; ++hh) {
          const float mn = oku && d[hh] - mm[hh] > kSlack ? d[hh] : mm[hh];
          const float a = __builtin_amdgcn_exp2f(mm[hh] - mn);
          ll[hh] *= a;
#pragma unroll
          for (int e = 0; e < 8; ++e) oo[hh][e] *= a;
          mm[hh] = mn;
        }
      }
#pragma unroll
      for (int hh = 0; hh < kSwaHeads; ++hh) {
        const float pw = oku ? __builtin_amdgcn_exp2f(d[hh] - mm[hh]) : 0.f;
        ll[hh] += pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) oo[hh][e] = fmaf(pw, vf[e], oo[hh][e]);
      }
      const int ri = base + (U + u) * 16 + wv * 4 + grp;
      ok[u] = ri < r1;
      if (ok[u]) {
        const size_t n = (size_t)swa_row<RING>(ri, ns, wbase, wwrap, g.window);
        kr[u] = ld_row(kb + n * kD + sub * 8);
        vr[u] = ld_row(vb + n * kD + sub * 8);
      }
    }
  }
  // back to natural-log units for the merges (an empty state has m = -inf)
#pragma unroll
  for (int hh = 0; hh < kSwaHeads; ++hh) mm[hh] = ll[hh] > 0.f ? mm[hh] * kLn2 : -INFINITY;
  // merge the row groups of each wave, then the waves through LDS
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
  if (defer) return;
  if (!arrive_last(g.ctr_swa + (size_t)(unit * g.swa_hb + hb) * g.cstride, (uint32_t)g.swa_nch, &sm.flag)) return;
  // wave hh combines head hh's chunk states (all heads in one round of loads)
  const int h = sm.heads[wv];
  if (h >= 0)
    wave_combine(parts + (size_t)wv * g.swa_nch, g.swa_nch, out + (((size_t)b * g.Hq + h) * g.nq + i) * kD);
}

// One SWA workgroup; x = its index among the SWA workgroups of the launch.
// In a layer with ring groups the layout of the block's KV group is uniform
// over the workgroup, so the full and the ring rows each get their own code.
template <bool RING_LAYOUT>
__device__ __forceinline__ void swa_block(const Geo &g, long long x, const rtp_bf16 *__restrict__ q_pre,
                                          const rtp_bf16 *__restrict__ kc, const rtp_bf16 *__restrict__ vc,
                                          float *__restrict__ out, SwaShared &sm, bool defer) {
  if (!RING_LAYOUT) {
    swa_block_rows<false, false>(g, x, q_pre, kc, vc, out, sm, defer);
    return;
  }
  const long long chunk_id = ((x >> 3) / g.swa_hb) * 8 + (x & 7);
  if (chunk_id >= (long long)g.swa_units * g.swa_nch) return;
  const int unit = (int)(chunk_id / g.swa_nch);
  if (kv_is_ring(g, g.lgroup[(unit / g.nq) % g.nlg]))
    swa_block_rows<true, true>(g, x, q_pre, kc, vc, out, sm, defer);
  else
    swa_block_rows<false, true>(g, x, q_pre, kc, vc, out, sm, defer);
}

// Number of workgroups that merge deferred chunk states: one per (unit, head block).
__host__ __device__ __forceinline__ long long swa_combine_blocks(const Geo &g) {
  return (long long)g.swa_units * g.swa_hb;
}

// Merge of the deferred chunk states of one (unit, head block), in the launch
// after the window workgroups: wave w takes the block's w-th local head (the
// same split the window workgroups use).
__device__ __forceinline__ void swa_combine_block(const Geo &g, long long y, float *__restrict__ out) {
  const int hb = (int)(y % g.swa_hb), unit = (int)(y / g.swa_hb);
  const int i = unit % g.nq, bl = unit / g.nq, lgi = bl % g.nlg, b = bl / g.nlg;
  const int wv = threadIdx.x >> 6;
  const int h = local_head(g, g.lgroup[lgi], hb * kSwaHeads + wv);
  if (h < 0) return;
  const Partial *parts = g.swa_part + ((size_t)(unit * g.swa_hb + hb) * kSwaHeads + wv) * g.swa_nch;
  wave_combine(parts, g.swa_nch, out + (((size_t)b * g.Hq + h) * g.nq + i) * kD);
}

}  // namespace rtp
