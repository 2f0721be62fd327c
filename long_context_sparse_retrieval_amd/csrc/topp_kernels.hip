// Indexer scan with fused per-tile histogram, histogram merge, and selection
// (+ optional gather attention) -- the sort-free dynamic Top-P of RTPurbo.
//
// "Full Attention Strikes Back" (RTPurbo) section 3.2: eq. (4) scores every
// cached token of a retrieval head with the rank-16 indexer; eq. (5) keeps the
// Top-P set of those scores and attends over it.  DeepRead summary of RTPurbo,
// hardware-optimised kernels: Top-P through a 256-bin histogram per head,
// fused with scoring, instead of a sort.
//
// Design for gfx950.  The scan is bandwidth-bound (32 bytes of indexer key per
// token): each workgroup streams one tile of T tokens with coalesced 16-byte
// loads, keeps the tile's scores in LDS, and builds per-wave 256-bin histograms
// in LDS with integer atomics.  Bins are 1/8 logit wide on a fixed grid, so
// tile histograms merge exactly by an integer shift; masses are summed as
// exact 64-bit integers of in-cell weights (deterministic in any order).  The
// last workgroup of a query merges all tiles (boundary bin b*, per-tile prefix
// of bin-b* mass and output offsets).  A second kernel re-reads one code byte
// per token, takes every token above b* and the ordered prefix of bin b*
// (recomputing only those tokens' scores), gathers their K/V rows and writes a
// split-K softmax state; the last workgroup of a query combines them.
#include "block_util.h"

namespace rtp {

namespace {

constexpr int kBnd = 254;   // highest regular bin; bin 255 is the clamp bin

template <int T>
struct ScanShared {
  static constexpr int TPT = T / kWG;
  float lg[T + kWG];                       // scores by tile position, one pad slot per TPT
  unsigned long long mass[4][kBins];       // per-wave histograms
  unsigned int cnt[4][kBins];
  double q[kR];
  double qtmp[16][kR];
  double red_d[4];
  unsigned long long red_u[4];
  int red_i[4];
  int flag;
  // merge
  double wcum[kBins];
  double2 rope[kD / 2];
};

template <int T>
__device__ __forceinline__ int lg_slot(int nl) { return nl + nl / ScanShared<T>::TPT; }

// Encodings of the per-query max cell and min base cell for unsigned atomicMax
// on a zero-initialised word (0 means "no tile yet").
__device__ __forceinline__ uint32_t enc_max(int c) { return (uint32_t)c + 0x80000000u; }
__device__ __forceinline__ int dec_max(uint32_t e) { return (int)(e - 0x80000000u); }
__device__ __forceinline__ uint32_t enc_min(int c) { return 0x7fffffffu - (uint32_t)c; }
__device__ __forceinline__ int dec_min(uint32_t e) { return (int)(0x7fffffffu - e); }

// Merge the histograms of one query into its selection parameters (run by the
// last workgroup of the query).  Every tile has added its bins into the
// query's ring of absolute cells (exact 64-bit integer sums), so the global
// histogram is 256 ring reads.  Cells spread over more than kRing would alias
// in the ring; that case falls back to shifting every tile histogram.
template <int T>
__device__ void merge_query(const Geo &g, int unit, long long m, const rtp_bf16 *q_pre, int32_t *count_out,
                            ScanShared<T> &sm) {
  const int tid = threadIdx.x;
  const TileSum *ts = g.tsum + (size_t)unit * g.nt;
  uint64_t *ring = g.ring + (size_t)unit * kRing;
  const int c = dec_max(__hip_atomic_load(g.cmax + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const int base_min = dec_min(__hip_atomic_load(g.cmin + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const long long span = (long long)c - base_min;
  const int j = tid;
  unsigned long long H = 0;
  double w255 = 0.0;
  if (span < kRing) {
    if (j <= kBnd) H = ring[(c - j) & (kRing - 1)];
    for (long long cell = (long long)c - (kBins - 1) - j; cell >= base_min; cell -= kWG) {
      const unsigned long long mj = ring[cell & (kRing - 1)];
      if (mj) w255 += (double)mj * exp((double)(cell - c) * 0.125);
    }
    __syncthreads();
    for (long long cell = (long long)base_min + j; cell <= c; cell += kWG) ring[cell & (kRing - 1)] = 0ull;
  } else {
    // slow path: shift every tile histogram
    for (int t = 0; t < g.nt; ++t) {
      const int ct = ts[t].c_t;
      if (ct == INT32_MIN) continue;
      const long long d = (long long)c - ct;
      if (j <= kBnd && j - d >= 0) H += ts[t].mass[j - d];
      if (j + d >= kBins - 1) {
        const unsigned long long mj = ts[t].mass[j];
        if (mj) w255 += (double)mj * exp(-(double)(j + d) * 0.125);
      }
    }
    __syncthreads();
    for (int x = j; x < kRing; x += kWG) ring[x] = 0ull;
  }
  if (tid == 0) {
    g.cmax[unit] = 0u;
    g.cmin[unit] = 0u;
  }
  // clamp-bin mass: fixed-order sum over threads
  sm.wcum[j] = w255;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int x = 0; x < kBins; ++x) s += sm.wcum[x];
    sm.red_d[0] = s;
  }
  __syncthreads();
  const double W255 = sm.red_d[0] * 0x1p-23;
  __syncthreads();
  const double Wj = j <= kBnd ? (double)H * 0x1p-23 * exp(-(double)j * 0.125) : W255;
  // cumulative bin masses from the top bin down (fixed order)
  double tot;
  const double excl = block_excl_scan<double>(Wj, tot, sm.red_d);
  const double incl = excl + Wj;
  const double Z = tot;
  const double need = (double)g.p * Z;
  const int cand = (incl >= need) ? j : kBins;
  int bstar = block_min<int>(cand, sm.red_i);
  if (bstar >= kBins) bstar = kBins - 1;
  sm.wcum[j] = excl;                      // mass above bin j
  __syncthreads();
  const double before = sm.wcum[bstar];
  __syncthreads();
  const int all = (g.p >= 1.0f || bstar >= kBins - 1) ? 1 : 0;
  const double r_u = (need - before) * 0x1p23 * exp((double)bstar * 0.125);

  // per tile: bin-b* prefix mass, sure / boundary counts and offsets
  unsigned long long carryP = 0;
  int carryS = 0, carryB = 0, tstar = -1, bo_star = -1;
  for (int t0 = 0; t0 < g.nt; t0 += kWG) {
    const int t = t0 + tid;
    unsigned long long bm = 0;
    int sure = 0, bc = 0;
    const int ct = t < g.nt ? ts[t].c_t : INT32_MIN;
    if (ct != INT32_MIN) {
      const long long bl = (long long)bstar - ((long long)c - ct);
      if (bl >= 1) sure = (int)ts[t].cum[(bl < kBins - 1 ? (int)bl : kBins - 1) - 1];
      if (bl >= 0 && bl <= kBnd) {
        const uint32_t hi = ts[t].cum[bl];
        bc = (int)(hi - (bl ? ts[t].cum[bl - 1] : 0u));
        bm = ts[t].mass[bl];
      }
    }
    unsigned long long totP;
    int totS, totB;
    const unsigned long long P = carryP + block_excl_scan<unsigned long long>(bm, totP, sm.red_u);
    const int so = carryS + block_excl_scan<int>(sure, totS, sm.red_i);
    const int bo = carryB + block_excl_scan<int>(bc, totB, sm.red_i);
    if (t < g.nt) {
      TileSel *tl = g.tsel + (size_t)unit * g.nt + t;
      tl->P = P;
      tl->sure_off = so;
      tl->bnd_off = bo;
    }
    // the crossing tile is the last one whose bin-b* tokens start below the residual;
    // every bin-b* token of the tiles before it is taken
    const bool crossing = t < g.nt && bc > 0 && (double)P < r_u;
    tstar = max(tstar, block_max<int>(crossing ? t : -1, sm.red_i));
    bo_star = max(bo_star, block_max<int>(crossing ? bo : -1, sm.red_i));
    carryP += totP;
    carryS += totS;
    carryB += totB;
  }
  const int total_sure = carryS;
  const int count_base = total_sure + (tstar >= 0 ? bo_star : 0);
  if (tid == 0) {
    HeadSel *hs = g.hsel + unit;
    hs->c = c;
    hs->bstar = bstar;
    hs->r_u = r_u;
    hs->tstar = tstar;
    hs->all = all;
    hs->count_base = count_base;
    hs->total_sure = total_sure;
    hs->nvalid = (int)(m + 1);
    if (all && count_out) count_out[unit] = (int)(m + 1);
  }
  // query preparation for the selection kernel
  QPrep *qp = g.qprep + unit;
  if (tid < kR) qp->qi[tid] = sm.q[tid];
  if (q_pre) {
    const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
    const rtp_bf16 *q_row = q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD;
    rope_table(m, g.theta, sm.rope);
    rotate_query(q_row, sm.rope, 0.08838834764831845f, qp->qrot);
  }
}

// Scan kernel: one workgroup per (query unit, tile of T positions).
template <int T, bool FROM_LOGITS>
__global__ __launch_bounds__(kWG) void scan_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                   const rtp_bf16 *__restrict__ w_q,
                                                   const rtp_bf16 *__restrict__ k_idx,
                                                   const float *__restrict__ logits, int32_t *count_out) {
  constexpr int TPT = T / kWG;
  __shared__ ScanShared<T> sm;
  const int tid = threadIdx.x, wv = tid >> 6;
  const int unit = blockIdx.x / g.nt, t = blockIdx.x % g.nt;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const long long m = g.N - g.nq + i;
  const long long n0 = (long long)t * T;

  for (int x = tid; x < 4 * kBins; x += kWG) {
    (&sm.mass[0][0])[x] = 0ull;
    (&sm.cnt[0][0])[x] = 0u;
  }
  if (!FROM_LOGITS) {
    project_query(q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD, w_q + (size_t)r * kD * kR, sm.q,
                  sm.qtmp);
  } else {
    __syncthreads();
  }

  // pass 1: scores (coalesced: consecutive threads take consecutive positions)
  float mx = -INFINITY;
  if (FROM_LOGITS) {
    const float *row = logits + (size_t)unit * g.N;
#pragma unroll 4
    for (int k = 0; k < TPT; ++k) {
      const int nl = k * kWG + tid;
      const long long n = n0 + nl;
      const float s = (n <= m) ? row[n] : -INFINITY;
      sm.lg[lg_slot<T>(nl)] = s;
      mx = fmaxf(mx, s);
    }
  } else {
    double q[kR];
#pragma unroll
    for (int x = 0; x < kR; ++x) q[x] = sm.q[x];
    const uint4 *rows = reinterpret_cast<const uint4 *>(k_idx + ((size_t)b * g.Hr + r) * g.Ncap * kR);
#pragma unroll 8
    for (int k = 0; k < TPT; ++k) {
      const int nl = k * kWG + tid;
      const long long n = n0 + nl;
      float s = -INFINITY;
      if (n <= m) s = dot16_exact(q, rows[2 * n], rows[2 * n + 1]);
      sm.lg[lg_slot<T>(nl)] = s;
      mx = fmaxf(mx, s);
    }
  }
  mx = block_max<float>(mx, reinterpret_cast<float *>(sm.red_d));
  const int c_t = (mx == -INFINITY) ? INT32_MIN : score_cell(mx);

  // pass 2: histogram and codes (each thread owns TPT consecutive positions)
  uint8_t code[TPT];
  int nv = 0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int nl = tid * TPT + k;
    const float s = sm.lg[lg_slot<T>(nl)];
    code[k] = 255;
    if (s != -INFINITY) {
      const int cell = score_cell(s);
      int jb = c_t - cell;
      uint32_t u;
      if (jb >= kBins - 1) {
        jb = kBins - 1;
        u = cell_weight(s, c_t - (kBins - 1));
      } else {
        u = cell_weight(s, cell);
      }
      atomicAdd(&sm.mass[wv][jb], (unsigned long long)u);
      atomicAdd(&sm.cnt[wv][jb], 1u);
      code[k] = (uint8_t)jb;
      ++nv;
    }
  }
  {
    uint8_t *dst = g.codes + (size_t)unit * g.nt * T + (size_t)t * T + (size_t)tid * TPT;
    if constexpr (TPT % 16 == 0) {
#pragma unroll
      for (int k = 0; k < TPT; k += 16) {
        uint4 v;
        uint32_t w[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          w[x] = (uint32_t)code[k + 4 * x] | ((uint32_t)code[k + 4 * x + 1] << 8) |
                 ((uint32_t)code[k + 4 * x + 2] << 16) | ((uint32_t)code[k + 4 * x + 3] << 24);
        v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
        *reinterpret_cast<uint4 *>(dst + k) = v;
      }
    } else {
#pragma unroll
      for (int k = 0; k < TPT; k += 4) {
        const uint32_t w0 = (uint32_t)code[k] | ((uint32_t)code[k + 1] << 8) | ((uint32_t)code[k + 2] << 16) |
                            ((uint32_t)code[k + 3] << 24);
        *reinterpret_cast<uint32_t *>(dst + k) = w0;
      }
    }
  }
  __syncthreads();

  // tile summary
  TileSum *tsum = g.tsum + (size_t)unit * g.nt + t;
  {
    const int j = tid;
    const unsigned long long ms = sm.mass[0][j] + sm.mass[1][j] + sm.mass[2][j] + sm.mass[3][j];
    const unsigned int cn = sm.cnt[0][j] + sm.cnt[1][j] + sm.cnt[2][j] + sm.cnt[3][j];
    unsigned int tot;
    const unsigned int ex = block_excl_scan<unsigned int>(cn, tot, reinterpret_cast<unsigned int *>(sm.red_i));
    st_coherent(&tsum->mass[j], (uint64_t)ms);
    st_coherent(&tsum->cum[j], (uint32_t)(ex + cn));
    int nvt;
    (void)block_excl_scan<int>(nv, nvt, sm.red_i);
    if (tid == 0) {
      st_coherent(&tsum->c_t, (int32_t)c_t);
      st_coherent(&tsum->nvalid, (int32_t)nvt);
    }
  }
  if (c_t != INT32_MIN) {
    if (tid == 0) {
      atomicMax(g.cmax + unit, enc_max(c_t));
      atomicMax(g.cmin + unit, enc_min(c_t - (kBins - 1)));
    }
    const unsigned long long ms = sm.mass[0][tid] + sm.mass[1][tid] + sm.mass[2][tid] + sm.mass[3][tid];
    if (ms) atomicAdd((unsigned long long *)(g.ring + (size_t)unit * kRing + ((c_t - tid) & (kRing - 1))), ms);
  }
  if (!arrive_last(g.ctr_scan + unit, (uint32_t)g.nt, &sm.flag)) return;
  merge_query<T>(g, unit, m, FROM_LOGITS ? nullptr : q_pre, count_out, sm);
}

struct SelShared {
  int list[8192];
  float q[kD];
  double qi[kR];
  unsigned long long red_u[4];
  int red_i[4];
  int flag;
  AttnShared at;
  CombineShared cb;
  Partial res;
};

// Selection kernel: one workgroup per (query unit, tile); optionally attends.
template <int T, bool FROM_LOGITS, bool ATTEND>
__global__ __launch_bounds__(kWG) void select_kernel(Geo g, const rtp_bf16 *__restrict__ k_idx,
                                                     const float *__restrict__ logits,
                                                     const rtp_bf16 *__restrict__ kc,
                                                     const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                                     int32_t *__restrict__ idx, int32_t *__restrict__ count,
                                                     long long cap) {
  constexpr int TPT = T / kWG;
  static_assert(T <= 8192, "selection list sized for T <= 8192");
  __shared__ SelShared sm;
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / g.nt, t = blockIdx.x % g.nt;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const long long m = g.N - g.nq + i;
  const long long n0 = (long long)t * T;
  const HeadSel hs = g.hsel[unit];
  const TileSum *ts = g.tsum + (size_t)unit * g.nt + t;
  const TileSel tl = g.tsel[(size_t)unit * g.nt + t];
  const int ct = ts->c_t;
  if (tid < kR) sm.qi[tid] = g.qprep[unit].qi[tid];
  if (ATTEND && tid < kD) sm.q[tid] = g.qprep[unit].qrot[tid];
  __syncthreads();

  // classify this thread's TPT consecutive positions
  uint8_t code[TPT];
  {
    const uint8_t *src = g.codes + (size_t)unit * g.nt * T + (size_t)t * T + (size_t)tid * TPT;
    if constexpr (TPT % 16 == 0) {
#pragma unroll
      for (int k = 0; k < TPT; k += 16) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src + k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int x = 0; x < 16; ++x) code[k + x] = (uint8_t)(w[x >> 2] >> (8 * (x & 3)));
      }
    } else {
#pragma unroll
      for (int k = 0; k < TPT; k += 4) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(src + k);
#pragma unroll
        for (int x = 0; x < 4; ++x) code[k + x] = (uint8_t)(w >> (8 * x));
      }
    }
  }
  const long long nbase = n0 + (long long)tid * TPT;
  int bl = -1;                  // local index of bin b*
  bool any = ct != INT32_MIN;
  if (any && !hs.all) {
    const long long d = (long long)hs.c - ct;
    const long long blv = (long long)hs.bstar - d;
    bl = blv < -1 ? -1 : (int)blv;
  }
  const bool bnd_on = any && !hs.all && bl >= 0 && bl <= kBnd && t <= hs.tstar;
  unsigned sure_m = 0, bnd_m = 0;     // bit k: position k of this thread
  unsigned long long bmass = 0;
  uint32_t bu[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const long long n = nbase + k;
    bu[k] = 0;
    if (!any || n > m) continue;
    if (hs.all || (int)code[k] < bl) {
      sure_m |= 1u << k;
    } else if (bnd_on && (int)code[k] == bl) {
      float s;
      if (FROM_LOGITS) {
        s = logits[(size_t)unit * g.N + n];
      } else {
        const uint4 *rows = reinterpret_cast<const uint4 *>(k_idx + ((size_t)b * g.Hr + r) * g.Ncap * kR);
        s = dot16_exact(sm.qi, rows[2 * n], rows[2 * n + 1]);
      }
      bu[k] = cell_weight(s, score_cell(s));
      bmass += bu[k];
      bnd_m |= 1u << k;
    }
  }
  // ordered fill of bin b*: a token is taken while the mass before it is below the residual
  unsigned long long tot_u;
  unsigned long long pre = tl.P + block_excl_scan<unsigned long long>(bmass, tot_u, sm.red_u);
  unsigned take_m = 0;
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (bnd_m & (1u << k)) {
      if ((double)pre < hs.r_u) take_m |= 1u << k;
      pre += bu[k];
    }
  }
  const int ns = __popc(sure_m), nb = __popc(take_m);
  int tot_s, tot_b;
  const int rs = block_excl_scan<int>(ns, tot_s, sm.red_i);
  const int rb = block_excl_scan<int>(nb, tot_b, sm.red_i);
  // outputs: positions above b* first, then the taken bin-b* positions
  const long long so = hs.all ? n0 : (long long)tl.sure_off;
  const long long bo = (long long)hs.total_sure + tl.bnd_off;
  {
    int a = rs, c2 = rb;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int n = (int)(nbase + k);
      if (sure_m & (1u << k)) {
        if (idx && so + a < cap) idx[(size_t)unit * cap + so + a] = n;
        if (ATTEND) sm.list[a] = n;
        ++a;
      }
      if (take_m & (1u << k)) {
        if (idx && bo + c2 < cap) idx[(size_t)unit * cap + bo + c2] = n;
        if (ATTEND) sm.list[tot_s + c2] = n;
        ++c2;
      }
    }
  }
  if (count && !hs.all && t == hs.tstar && tid == 0) count[unit] = hs.count_base + tot_b;
  if (!ATTEND) return;
  __syncthreads();
  const int hq = g.rhead[r];
  const int kvg = hq / g.G;
  const size_t cbase = ((size_t)b * g.Hkv + kvg) * g.Ncap * kD;
  attend_rows(sm.q, sm.list, tot_s + tot_b, g.N, kc + cbase, vc + cbase, &sm.res, &sm.at);
  publish_partial(g.part + (size_t)unit * g.nt + t, &sm.res);
  if (!arrive_last(g.ctr_fin + unit, (uint32_t)g.nt, &sm.flag)) return;
  combine_partials(g.part + (size_t)unit * g.nt, g.nt, out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, &sm.cb);
}

template <int T>
int launch_scan_t(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                  const float *logits, int32_t *count, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)g.units * g.nt);
  if (logits)
    hipLaunchKernelGGL((scan_kernel<T, true>), dim3(grid), dim3(kWG), 0, s, g, q_pre, w_q, k_idx, logits, count);
  else
    hipLaunchKernelGGL((scan_kernel<T, false>), dim3(grid), dim3(kWG), 0, s, g, q_pre, w_q, k_idx, logits, count);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

template <int T>
int launch_select_t(const Geo &g, const rtp_bf16 *k_idx, const float *logits, const rtp_bf16 *k, const rtp_bf16 *v,
                    float *out, int32_t *idx, int32_t *count, long long cap, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)g.units * g.nt);
  if (out) {
    if (logits)
      hipLaunchKernelGGL((select_kernel<T, true, true>), dim3(grid), dim3(kWG), 0, s, g, k_idx, logits, k, v, out,
                         idx, count, cap);
    else
      hipLaunchKernelGGL((select_kernel<T, false, true>), dim3(grid), dim3(kWG), 0, s, g, k_idx, logits, k, v, out,
                         idx, count, cap);
  } else {
    if (logits)
      hipLaunchKernelGGL((select_kernel<T, true, false>), dim3(grid), dim3(kWG), 0, s, g, k_idx, logits, k, v, out,
                         idx, count, cap);
    else
      hipLaunchKernelGGL((select_kernel<T, false, false>), dim3(grid), dim3(kWG), 0, s, g, k_idx, logits, k, v, out,
                         idx, count, cap);
  }
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace

int launch_scan(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx, const float *logits,
                int32_t *count, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  switch (g.T) {
    case 1024: return launch_scan_t<1024>(g, q_pre, w_q, k_idx, logits, count, s);
    case 2048: return launch_scan_t<2048>(g, q_pre, w_q, k_idx, logits, count, s);
    case 4096: return launch_scan_t<4096>(g, q_pre, w_q, k_idx, logits, count, s);
    case 8192: return launch_scan_t<8192>(g, q_pre, w_q, k_idx, logits, count, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

int launch_select(const Geo &g, const rtp_bf16 *k_idx, const float *logits, const rtp_bf16 *k, const rtp_bf16 *v,
                  float *out, int32_t *idx, int32_t *count, long long cap, hipStream_t s) {
  if (g.units == 0) return RTP_OK;
  switch (g.T) {
    case 1024: return launch_select_t<1024>(g, k_idx, logits, k, v, out, idx, count, cap, s);
    case 2048: return launch_select_t<2048>(g, k_idx, logits, k, v, out, idx, count, cap, s);
    case 4096: return launch_select_t<4096>(g, k_idx, logits, k, v, out, idx, count, cap, s);
    case 8192: return launch_select_t<8192>(g, k_idx, logits, k, v, out, idx, count, cap, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

}  // namespace rtp
