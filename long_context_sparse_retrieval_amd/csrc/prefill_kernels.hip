// Chunked prefill (nq > 1 causal queries per head): the indexer as a GEMM on
// the matrix cores, exact per-query 256-bin Top-P, and attention over the
// selected rows.
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2: eq. (4) scores every
// earlier position of each query with the rank-16 indexer, eq. (5) keeps the
// Top-P set and attends over it.  Query i of a chunk of nq sits at position
// m_i = N - nq + i and sees positions 0..m_i.
//
// Design for gfx950.  One selection workgroup owns 16 queries of one head and
// their whole prefixes, so each query's histogram lives in LDS and never has
// to be merged across workgroups.  The K = 16 contraction is one
// v_mfma_f32_16x16x16_bf16 per 16 keys (16 keys x 16 queries per wave; each
// lane gets four keys of one query, so a row of 16 lanes updates 16 different
// query histograms and LDS atomics rarely collide); the
// products of two bf16 values are exact in fp32, only the order of the 16-term
// sum is the matrix core's.  The logits are never stored: four passes
// recompute them from the indexer keys (4 MiB per head at 128K, resident in
// the Infinity Cache) -- per-query maximum, exact integer histogram, per-chunk
// counts and bin-b* mass, then the ordered selection.  Keys are split into
// chunks, each processed in position order by one wave, so the selected
// positions come out in ascending order with offsets from a per-chunk prefix.
#include "block_util.h"

namespace rtp {

namespace {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQB = 16;         // queries per selection workgroup (the matrix-core M dimension)
constexpr int kMaxCh = 128;     // key chunks per query
constexpr int kUnroll = 8;      // 16-key blocks whose loads are issued together

// Per query of a selection workgroup.
struct PfSel {
  double r_u;     // residual of p*Z in in-cell units of bin b*
  int c;          // max cell
  int bstar;      // boundary bin; 256 when every position is taken
  int all;
  int cstar;      // crossing chunk (-1: none)
  int n_sure;     // positions above b*
  int valid;
};

// PACK: each bin's count rides in the top bits of its mass (one LDS atomic
// per position, no count array: 34 KB instead of 50 KB of LDS, so four
// workgroups share a CU instead of three).  A bin's mass is below
// (prefix length) * 1.14 * 2^23, so with the count from bit 41 up the packing
// holds for prefixes of up to 2^17 positions; longer ones keep the counts apart.
constexpr int kPfCountShift = 41;
constexpr unsigned long long kPfMassMask = (1ull << kPfCountShift) - 1;
constexpr long long kPfPackMaxN = 1ll << 17;

template <bool PACK>
struct PfShared {
  union {
    struct {
      unsigned long long mass[kQB][kBins];
      uint32_t cnt[PACK ? 1 : kQB][kBins];
    } h;
    struct {
      unsigned long long bm[kQB][kMaxCh];   // bin-b* mass per chunk, then its exclusive prefix
      int ns[kQB][kMaxCh];                  // positions above b* per chunk, then exclusive prefix
      int nb[kQB][kMaxCh];                  // bin-b* positions per chunk, then exclusive prefix
    } c;
  };
  PfSel sel[kQB];
  float wmax[4][kQB];
};

// Selection: one workgroup per (b, r, block of 16 queries of the chunk [i0, i0 + nqc)).
// Writes the selected positions of each query to idx_ws[unit_local][capw] (and,
// optionally, to idx[unit][cap], truncated) and its count to cnt_ws / count.
template <bool PACK>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4, 8))) void pf_select_kernel(Geo g, const rtp_bf16 *__restrict__ k_idx, int i0, int nqc,
                                                        int kc, int32_t *__restrict__ idx_ws, long long capw,
                                                        int32_t *__restrict__ cnt_ws, int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ count, long long cap) {
  __shared__ PfShared<PACK> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, row = lane >> 4, col = lane & 15;
  const int nblk = (nqc + kQB - 1) / kQB;
  const int br = blockIdx.x / nblk, qb = blockIdx.x % nblk;
  const int r = br % g.Hr, b = br / g.Hr;
  const int qi0 = i0 + qb * kQB;                         // first query index (0..nq) of the block
  const int nvalid = min(kQB, i0 + nqc - qi0);
  const long long mpos0 = g.N - g.nq;                    // position of query index 0
  const long long m_last = mpos0 + qi0 + nvalid - 1;
  const uint2 *keys = reinterpret_cast<const uint2 *>(k_idx + ((size_t)b * g.Hi + r / g.ig) * g.Ncap * kR);

  // Matrix-core operands: A = 16 keys x 16 dims (lane: key col, dims 4 row ..
  // 4 row + 3), B = 16 dims x 16 queries (lane: query col, the same dims), so
  // lane (row, col) receives the scores of query col against keys 4 row .. 4 row
  // + 3 of the block: the 16 lanes of a row serve 16 different queries.
  bf16x4_t bq;
  const int qc = col;                                    // this lane's query
  const bool qv = qc < nvalid;
  {
    const QPrep *qp = g.qprep + ((size_t)br * g.nq + qi0 + (qv ? qc : 0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float f = qv ? (float)qp->qi[4 * row + j] : 0.f;
      bq[j] = (short)(__float_as_uint(f) >> 16);        // the values are bf16, so exact
    }
  }
  const long long mq = mpos0 + qi0 + qc;                 // position of this lane's query
  const int nch = (int)((m_last + 1 + kc - 1) / kc);

  // Runs body(n0, d) for every 16-key block of the chunks this wave owns, in
  // position order within a chunk; d[i] = score of key n0 + 4 row + i.
  auto sweep = [&](auto &&body, auto &&chunk_begin, auto &&chunk_end) {
    for (int ch = wv; ch < nch; ch += 4) {
      chunk_begin(ch);
      const long long k0 = (long long)ch * kc;
      const long long k1 = k0 + kc < m_last + 1 ? k0 + kc : m_last + 1;
      for (long long n0 = k0; n0 < k1; n0 += 16 * kUnroll) {
        uint2 kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {              // clamped, unconditional loads
          long long nr = n0 + 16 * u + col;
          nr = nr < g.N ? nr : g.N - 1;
          kv[u] = keys[nr * 4 + row];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (n0 + 16 * u >= k1) break;                   // wave-uniform
          bf16x4_t ak;
          ak[0] = (short)(kv[u].x & 0xffffu);
          ak[1] = (short)(kv[u].x >> 16);
          ak[2] = (short)(kv[u].y & 0xffffu);
          ak[3] = (short)(kv[u].y >> 16);
          const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ak, bq, zero, 0, 0, 0);
          body(n0 + 16 * u + 4 * row, d);
        }
      }
      chunk_end(ch);
    }
  };
  auto nop = [](int) {};
  // sum over the four lanes of a column (the same query)
  auto col_sum_i = [](int v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
  };
  // exclusive prefix over the rows of a column, and the column total
  auto col_scan = [&](unsigned long long v, unsigned long long &total) {
    unsigned long long x = v;
    const unsigned long long t1 = __shfl_up(x, 16);
    if (row >= 1) x += t1;
    const unsigned long long t2 = __shfl_up(x, 32);
    if (row >= 2) x += t2;
    total = __shfl(x, 48 + col);
    return x - v;
  };

  // ---- pass 1: per-query maximum
  float mx = -INFINITY;
  sweep([&](long long nb0, const f32x4_t &d) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (qv && nb0 + i <= mq) mx = fmaxf(mx, d[i]);
        },
        nop, nop);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (row == 0) sm.wmax[wv][qc] = mx;
  for (int x = tid; x < kQB * kBins; x += kWG) {
    (&sm.h.mass[0][0])[x] = 0ull;
    if (!PACK) (&sm.h.cnt[0][0])[x] = 0u;
  }
  __syncthreads();
  if (tid < kQB) {
    const float v = fmaxf(fmaxf(sm.wmax[0][tid], sm.wmax[1][tid]), fmaxf(sm.wmax[2][tid], sm.wmax[3][tid]));
    sm.sel[tid].c = tid < nvalid ? score_cell(v) : 0;
    sm.sel[tid].valid = tid < nvalid ? 1 : 0;
  }
  __syncthreads();
  const int cq = sm.sel[qc].c;

  // ---- pass 2: exact 256-bin histogram per query (bins relative to the query's max cell)
  sweep([&](long long nb0, const f32x4_t &d) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (!(qv && nb0 + i <= mq)) continue;
            const float s = d[i];
            const int cell = score_cell(s);
            int j = cq - cell;
            uint32_t w;
            if (j >= kBins - 1) {
              j = kBins - 1;
              w = token_weight(g, s, cq - (kBins - 1));
            } else {
              w = token_weight(g, s, cell);
            }
            if (PACK) {
              atomicAdd(&sm.h.mass[qc][j], (unsigned long long)w | (1ull << kPfCountShift));
            } else {
              atomicAdd(&sm.h.mass[qc][j], (unsigned long long)w);
              atomicAdd(&sm.h.cnt[qc][j], 1u);
            }
          }
        },
        nop, nop);
  __syncthreads();

  // ---- threshold per query: wave w takes queries w, w + 4, ...; lane holds bins 4 lane .. 4 lane + 3
  for (int q = wv; q < kQB; q += 4) {
    if (q >= nvalid) continue;                            // wave-uniform
    double W[4];
    double loc = 0.0;
    int cnt_lt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * lane + k;
      W[k] = (double)(PACK ? sm.h.mass[q][j] & kPfMassMask : sm.h.mass[q][j]) * 0x1p-23 *
             bin_scale(g, -(double)j * 0.125);
      loc += W[k];
    }
    double incl = loc;                                    // wave inclusive scan (fixed order)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const double Z = __shfl(incl, 63);
    double e = incl - loc;
    const double need = g.topk ? (double)g.topk : g.p * Z;     // top-k: Z counts positions
    int cand = kBins;
    double before_c = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (cand == kBins && e + W[k] >= need) {
        cand = 4 * lane + k;
        before_c = e;
      }
      e += W[k];
    }
    int bstar = cand;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bstar = min(bstar, __shfl_xor(bstar, off));
    if (bstar >= kBins) bstar = kBins - 1;
    const double before = __shfl(before_c, bstar / 4);
    // the query's bins are relative to its own maximum, so for top-k the
    // clamp bin is an ordinary boundary
    const int all = (g.topk ? need >= Z : (g.p >= 1.0 || bstar >= kBins - 1)) ? 1 : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * lane + k;
      const int cj = PACK ? (int)(sm.h.mass[q][j] >> kPfCountShift) : (int)sm.h.cnt[PACK ? 0 : q][j];
      cnt_lt += j < bstar ? cj : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt_lt += __shfl_xor(cnt_lt, off);
    if (lane == 0) {
      PfSel &ps = sm.sel[q];
      ps.all = all;
      ps.bstar = all ? kBins : bstar;
      ps.r_u = (need - before) * 0x1p23 * bin_scale(g, (double)bstar * 0.125);
      ps.n_sure = all ? (int)(mpos0 + qi0 + q + 1) : cnt_lt;
    }
  }
  __syncthreads();                                        // the histogram is dead from here on
  for (int x = tid; x < kQB * kMaxCh; x += kWG) {
    (&sm.c.bm[0][0])[x] = 0ull;
    (&sm.c.ns[0][0])[x] = 0;
    (&sm.c.nb[0][0])[x] = 0;
  }
  const int bs = sm.sel[qc].bstar, allq = sm.sel[qc].all;
  __syncthreads();

  // ---- pass 3: per chunk, positions above b*, positions in b* and their mass
  {
    int ns = 0, nbb = 0;
    unsigned long long bm = 0;
    sweep([&](long long nb0, const f32x4_t &d) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (!(qv && nb0 + i <= mq)) continue;
              const float s = d[i];
              const int cell = score_cell(s);
              const int j = min(cq - cell, kBins - 1);
              if (j < bs) {
                ++ns;
              } else if (!allq && j == bs) {
                ++nbb;
                bm += token_weight(g, s, cell);
              }
            }
          },
          [&](int) {
            ns = nbb = 0;
            bm = 0ull;
          },
          [&](int ch) {
            const int a1 = col_sum_i(ns), a2 = col_sum_i(nbb);
            unsigned long long a3 = bm + __shfl_xor(bm, 16);
            a3 += __shfl_xor(a3, 32);
            if (row == 0) {
              sm.c.ns[qc][ch] = a1;
              sm.c.nb[qc][ch] = a2;
              sm.c.bm[qc][ch] = a3;
            }
          });
  }
  __syncthreads();

  // ---- per query: exclusive prefixes over chunks (position order) and the crossing chunk
  for (int q = wv; q < kQB; q += 4) {
    if (q >= nvalid) continue;
    const PfSel ps = sm.sel[q];
    // lane holds chunks 2 lane, 2 lane + 1
    unsigned long long m0 = 0, m1 = 0;
    int s0 = 0, s1 = 0, b0 = 0, b1 = 0;
    if (2 * lane < nch) { m0 = sm.c.bm[q][2 * lane]; s0 = sm.c.ns[q][2 * lane]; b0 = sm.c.nb[q][2 * lane]; }
    if (2 * lane + 1 < nch) { m1 = sm.c.bm[q][2 * lane + 1]; s1 = sm.c.ns[q][2 * lane + 1]; b1 = sm.c.nb[q][2 * lane + 1]; }
    unsigned long long mi = m0 + m1;
    int si = s0 + s1, bi = b0 + b1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long ym = __shfl_up(mi, off);
      const int ys = __shfl_up(si, off), yb = __shfl_up(bi, off);
      if (lane >= off) {
        mi += ym;
        si += ys;
        bi += yb;
      }
    }
    const unsigned long long Pm0 = mi - m0 - m1, Pm1 = Pm0 + m0;
    const int Ps0 = si - s0 - s1, Ps1 = Ps0 + s0, Pb0 = bi - b0 - b1, Pb1 = Pb0 + b0;
    int cross = -1;
    if (!ps.all) {
      if (2 * lane < nch && b0 > 0 && (double)Pm0 < ps.r_u) cross = 2 * lane;
      if (2 * lane + 1 < nch && b1 > 0 && (double)Pm1 < ps.r_u) cross = 2 * lane + 1;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cross = max(cross, __shfl_xor(cross, off));
    if (2 * lane < nch) { sm.c.bm[q][2 * lane] = Pm0; sm.c.ns[q][2 * lane] = Ps0; sm.c.nb[q][2 * lane] = Pb0; }
    if (2 * lane + 1 < nch) { sm.c.bm[q][2 * lane + 1] = Pm1; sm.c.ns[q][2 * lane + 1] = Ps1; sm.c.nb[q][2 * lane + 1] = Pb1; }
    if (lane == 0) sm.sel[q].cstar = cross;
  }
  __syncthreads();

  // ---- pass 4: ordered selection; positions above b* at [0, n_sure), taken bin-b* positions after them
  {
    const int cs = sm.sel[qc].cstar, nsure = sm.sel[qc].n_sure;
    const double ru = sm.sel[qc].r_u;
    const size_t ul = (size_t)br * nqc + (qi0 - i0) + qc;    // chunk-local unit of this lane's query
    const size_t ug = (size_t)br * g.nq + qi0 + qc;           // global unit
    int rs = 0, rb = 0, cur = 0;
    unsigned long long rm = 0;
    sweep([&](long long nb0, const f32x4_t &d) {
            bool sure[4], bnd[4];
            uint32_t w[4];
            int ls = 0, lt = 0;
            uint32_t lw = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool ok = qv && nb0 + i <= mq;
              const float s = d[i];
              const int cell = score_cell(s);
              const int j = min(cq - cell, kBins - 1);
              sure[i] = ok && j < bs;
              bnd[i] = ok && !allq && j == bs;
              w[i] = (bnd[i] && cur == cs) ? token_weight(g, s, cell) : 0u;
              ls += sure[i] ? 1 : 0;
              lw += w[i];
            }
            // ordered fill inside the crossing chunk: mass of the earlier bin-b* keys of the block
            unsigned long long wtot;
            const unsigned long long wpre = col_scan(lw, wtot);
            unsigned long long acc = (unsigned long long)sm.c.bm[qc][cur] + rm + wpre;
            bool take[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              take[i] = bnd[i] && (cur < cs || (cur == cs && (double)acc < ru));
              acc += w[i];
              lt += take[i] ? 1 : 0;
            }
            rm += wtot;
            unsigned long long stot, ttot;
            const unsigned long long spre = col_scan((unsigned long long)ls, stot);
            const unsigned long long tpre = col_scan((unsigned long long)lt, ttot);
            long long as = (long long)sm.c.ns[qc][cur] + rs + (long long)spre;
            long long at = (long long)nsure + sm.c.nb[qc][cur] + rb + (long long)tpre;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int n = (int)(nb0 + i);
              if (sure[i]) {
                idx_ws[ul * capw + as] = n;
                if (idx && as < cap) idx[ug * cap + as] = n;
                ++as;
              }
              if (take[i]) {
                if (at < capw) idx_ws[ul * capw + at] = n;
                if (idx && at < cap) idx[ug * cap + at] = n;
                ++at;
              }
            }
            rs += (int)stot;
            rb += (int)ttot;
          },
          [&](int ch) {
            cur = ch;
            rs = rb = 0;
            rm = 0ull;
          },
          [&](int ch) {
            if (qv && ch == cs && row == 0) {
              const int c_ = nsure + sm.c.nb[qc][ch] + rb;
              cnt_ws[ul] = c_;
              if (count) count[ug] = c_;
            }
          });
  }
  // queries without a crossing chunk: every position (p >= 1 or b* the clamp
  // bin) -- the residual is positive otherwise, so the first chunk holding a
  // bin-b* position always crosses
  if (tid < nvalid && sm.sel[tid].cstar < 0) {
    const int c_ = sm.sel[tid].n_sure;
    cnt_ws[(size_t)br * nqc + (qi0 - i0) + tid] = c_;
    if (count) count[(size_t)br * g.nq + qi0 + tid] = c_;
  }
}

// Query preparation for every (b, r, i) of the chunk: exact indexer query and
// the rotated, 1/sqrt(D)-scaled attention query (fp64 angles).
struct PrepShared {
  double q[kR];
  double qtmp[16][kR];
  double2 rope[kD / 2];
};

__global__ __launch_bounds__(kWG) void pf_qprep_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                       const rtp_bf16 *__restrict__ w_q) {
  __shared__ PrepShared sm;
  const int unit = blockIdx.x;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const long long m = g.N - g.nq + i;
  const rtp_bf16 *q_row = q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD;
  QPrep *qp = g.qprep + unit;
  project_query(q_row, w_q + (size_t)r * kD * kR, sm.q, sm.qtmp);
  if (threadIdx.x < kR) qp->qi[threadIdx.x] = sm.q[threadIdx.x];
  rope_table(m, g.theta, sm.rope);
  rotate_query(q_row, sm.rope, 0.08838834764831845f, qp->qrot);
}

// Split-K workgroups per query in the prefill attention.  One: at 1.5 K rows
// per query the per-workgroup set-up and the split-K hand-off cost more than
// the extra parallelism gains (the whole 128K chunked call: 6.9 ms with one
// workgroup per query, 7.5 ms with 2, 8.4 with 4, 10.0 with 8 or 16).
constexpr int kPfSplit = 1;

struct PfAttnShared {
  float q[kD];
  int list[1024];
  int flag;
  Partial extra;
  AttnShared at;
  CombineShared cb;
};

// Attention of the chunk's retrieval queries over their selected rows:
// kPfSplit workgroups per query; with more than one, the last combines their
// split-K states.
__global__ __launch_bounds__(kWG) void pf_attn_kernel(Geo g, int i0, int nqc, const rtp_bf16 *__restrict__ kc,
                                                      const rtp_bf16 *__restrict__ vc,
                                                      const int32_t *__restrict__ idx_ws, long long capw,
                                                      const int32_t *__restrict__ cnt_ws, float *__restrict__ out) {
  __shared__ PfAttnShared sm;
  const int tid = threadIdx.x;
  const int ul = blockIdx.x / kPfSplit, sp = blockIdx.x % kPfSplit;
  const int ii = ul % nqc, br = ul / nqc, r = br % g.Hr, b = br / g.Hr;
  const int i = i0 + ii;
  const int hq = g.rhead[r], kvg = hq / g.G;
  const size_t ug = (size_t)br * g.nq + i;
  if (tid < kD) sm.q[tid] = g.qprep[ug].qrot[tid];
  long long cnt = cnt_ws[ul];
  cnt = cnt < 0 ? 0 : (cnt > capw ? capw : cnt);
  const long long per = (cnt + kPfSplit - 1) / kPfSplit;
  const long long a0 = (long long)sp * per;
  const long long a1 = a0 + per < cnt ? a0 + per : cnt;
  const size_t cbase = kv_group_base(g, b, kvg) * kD;
  const int32_t *list = idx_ws + (size_t)ul * capw;
  float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;
  for (long long s0 = a0; s0 < a1; s0 += 1024) {
    const int n = (int)(a1 - s0 < 1024 ? a1 - s0 : 1024);
    __syncthreads();
    for (int x = tid; x < n; x += kWG) sm.list[x] = list[s0 + x];
    __syncthreads();
    attend_rows<false>(sm.q, sm.list, n, g.N - g.nq + i + 1, kc + cbase, vc + cbase, &sm.extra, &sm.at);
    if (tid < kD) merge_state(run_m, run_l, &run_o, sm.extra.m, sm.extra.l, &sm.extra.o[tid], 1);
  }
  if constexpr (kPfSplit == 1) {      // the query's whole list: normalise in place
    if (tid < kD) out[(((size_t)b * g.Hq + hq) * g.nq + i) * kD + tid] = run_l > 0.f ? run_o / run_l : 0.f;
    return;
  }
  Partial *dst = g.part + (size_t)ul * kPfSplit + sp;
  if (tid < kD) {
    st_coherent(&dst->o[tid], run_o);
    if (tid == 0) {
      st_coherent(&dst->m, run_m);
      st_coherent(&dst->l, run_l);
    }
  }
  if (!arrive_last(g.ctr_fin + (size_t)ul * g.cstride, (uint32_t)kPfSplit, &sm.flag)) return;
  combine_partials(g.part + (size_t)ul * kPfSplit, kPfSplit, out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, &sm.cb);
}

}  // namespace

int pf_split() { return kPfSplit; }

int launch_pf_qprep(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  hipLaunchKernelGGL(pf_qprep_kernel, dim3((unsigned)g.units), dim3(kWG), 0, s, g, q_pre, w_q);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

int launch_pf_select(const Geo &g, const rtp_bf16 *k_idx, int i0, int nqc, int32_t *idx_ws, long long capw,
                     int32_t *cnt_ws, int32_t *idx, int32_t *count, long long cap, hipStream_t s) {
  if (g.units == 0 || nqc <= 0) return RTP_OK;
  const long long span = g.N;                            // longest prefix
  long long kc = (span + kMaxCh - 1) / kMaxCh;
  kc = (kc + 16 * kUnroll - 1) / (16 * kUnroll) * (16 * kUnroll);
  if (kc < 1024) kc = 1024;
  const int nblk = (nqc + kQB - 1) / kQB;
  const long long grid = (long long)g.B * g.Hr * nblk;
  if (g.N <= kPfPackMaxN)
    hipLaunchKernelGGL(pf_select_kernel<true>, dim3((unsigned)grid), dim3(kWG), 0, s, g, k_idx, i0, nqc, (int)kc,
                       idx_ws, capw, cnt_ws, idx, count, cap);
  else
    hipLaunchKernelGGL(pf_select_kernel<false>, dim3((unsigned)grid), dim3(kWG), 0, s, g, k_idx, i0, nqc, (int)kc,
                       idx_ws, capw, cnt_ws, idx, count, cap);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

int launch_pf_attn(const Geo &g, int i0, int nqc, const rtp_bf16 *k, const rtp_bf16 *v, const int32_t *idx_ws,
                   long long capw, const int32_t *cnt_ws, float *out, hipStream_t s) {
  if (g.units == 0 || nqc <= 0) return RTP_OK;
  const long long grid = (long long)g.B * g.Hr * nqc * kPfSplit;
  hipLaunchKernelGGL(pf_attn_kernel, dim3((unsigned)grid), dim3(kWG), 0, s, g, i0, nqc, k, v, idx_ws, capw, cnt_ws,
                     out);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace rtp
