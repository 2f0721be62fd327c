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
// second kernel re-reads one code byte per token; each of its workgroups first
// rebuilds the query's global histogram from an exact absolute-cell ring the
// scan tiles filled with integer atomics (boundary bin b*, residual mass,
// per-tile prefix of bin-b* mass), then takes every token of its tile above
// b* and the ordered prefix of bin b* (recomputing only those tokens' scores),
// gathers their K/V rows and writes a split-K softmax state; the last
// workgroup of a query combines them.  The sliding-window workgroups of the
// local heads run inside the scan launch, so their latency hides under the
// indexer stream.
#include "block_util.h"
#include "swa.h"

namespace rtp {

namespace {

constexpr int kBnd = 254;   // highest regular bin; bin 255 is the clamp bin

constexpr int kCells = 512;      // absolute score cells tracked per tile while streaming (64 logit units)

// A histogram entry packs the token count (bits 40..63) above the summed
// in-cell masses (bits 0..39; at most 8192 tokens of < 1.14 * 2^23 each).
constexpr int kCountShift = 40;
constexpr unsigned long long kMassMask = (1ull << kCountShift) - 1;

template <int T>
struct ScanShared {
  static constexpr int TPT = T / kWG;
  uint8_t codes[T];                        // local bin of every position of the tile
  unsigned long long hist[4][kCells];      // per-wave histograms by absolute cell mod kCells:
                                           // count << 40 | exact in-cell mass
  double q[kR];
  double qtmp[16][kR];
  double2 rope[kD / 2];
  float red_f[4];
  int red_i[4];
  unsigned int red_u32[4];
  unsigned long long red_u[4];
  double red_d[4];
};

// Encodings of the per-query max cell and min base cell for unsigned atomicMax
// on a zero-initialised word (0 means "no tile yet").
__device__ __forceinline__ uint32_t enc_max(int c) { return (uint32_t)c + 0x80000000u; }
__device__ __forceinline__ int dec_max(uint32_t e) { return (int)(e - 0x80000000u); }
__device__ __forceinline__ uint32_t enc_min(int c) { return 0x7fffffffu - (uint32_t)c; }
__device__ __forceinline__ int dec_min(uint32_t e) { return (int)(0x7fffffffu - e); }


// Scan workgroups of a launch: units * nt, or with shared indexer keys one
// per (retrieval head, tile) in the order below, padded.
__host__ __device__ __forceinline__ long long scan_blocks(const Geo &g) {
  if (g.ig == 1) return (long long)g.units * g.nt;
  const long long slots = (long long)g.B * g.Hi * g.nq * g.nt;
  return (slots + 7) / 8 * 8 * g.ig;
}

// Query unit and tile of scan workgroup blk; false for padding.  With shared
// indexer keys the ig heads that read the same key rows get workgroups 8
// apart (the same XCD, dispatched together), so the rows come from its L2
// for all but the first.
__device__ __forceinline__ bool scan_unit_tile(const Geo &g, long long blk, int &unit, int &t) {
  if (g.ig == 1) {
    unit = (int)(blk / g.nt);
    t = (int)(blk % g.nt);
    return true;
  }
  const long long xcd = blk & 7, y = blk >> 3;
  const int h = (int)(y % g.ig);
  long long s = (y / g.ig) * 8 + xcd;                    // over (b, indexer head, query, tile)
  t = (int)(s % g.nt);
  s /= g.nt;
  const int i = (int)(s % g.nq);
  s /= g.nq;
  const int ih = (int)(s % g.Hi), b = (int)(s / g.Hi);
  if (b >= g.B) return false;
  unit = ((b * g.Hr) + ih * g.ig + h) * g.nq + i;
  return true;
}

// One scan workgroup: tile t of query unit (scan_unit_tile).
template <int T, bool FROM_LOGITS>
__device__ __forceinline__ void scan_block(const Geo &g, long long blk, const rtp_bf16 *__restrict__ q_pre,
                                           const rtp_bf16 *__restrict__ w_q, const rtp_bf16 *__restrict__ k_idx,
                                           const float *__restrict__ logits, ScanShared<T> &sm) {
  constexpr int TPT = T / kWG;
  constexpr int BATCH = TPT < 5 ? TPT : 5;
  const int tid = threadIdx.x, wv = tid >> 6;
  int unit, t;
  if (!scan_unit_tile(g, blk, unit, t)) return;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const long long m = g.N - g.nq + i;
  const long long n0 = (long long)t * T;

  // pass 1: scores in registers; consecutive threads take consecutive positions.
  // Each score is binned at once by its absolute cell (no tile max needed), so
  // the histogram work overlaps the stream.  The first batch of key rows is
  // requested before the query projection.
  float lg[TPT];
  float mx = -INFINITY;
  int cmin = INT32_MAX;
  for (int x = tid; x < 4 * kCells; x += kWG) (&sm.hist[0][0])[x] = 0ull;
  // branchless, so a whole batch of rows stays one basic block and its loads
  // can be issued together; absent positions (-inf) add nothing
  auto bin_abs = [&](float sc) {
    const bool ok = sc != -INFINITY;
    const float s = ok ? sc : 0.f;
    const int cell = score_cell(s);
    const unsigned long long add = ok ? ((unsigned long long)token_weight(g, s, cell) | (1ull << kCountShift)) : 0ull;
    atomicAdd(&sm.hist[wv][cell & (kCells - 1)], add);
    mx = fmaxf(mx, sc);
    cmin = min(cmin, ok ? cell : INT32_MAX);
  };
  if (FROM_LOGITS) {
    __syncthreads();
    const float *row = logits + (size_t)unit * g.N;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const long long n = n0 + k * kWG + tid;
      const float sc = row[n <= m ? n : m];            // clamped, unconditional load
      lg[k] = n <= m ? sc : -INFINITY;
      bin_abs(lg[k]);
    }
  } else {
    // rolling window of BATCH rows per thread: slot u is refilled with the row
    // BATCH positions ahead as soon as it is consumed, so about BATCH rows per
    // thread stay in flight; loads are clamped to a valid row and unconditional
    const uint4 *rows = reinterpret_cast<const uint4 *>(k_idx + ((size_t)b * g.Hi + r / g.ig) * g.Ncap * kR);
    uint4 ra[BATCH], rb[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const long long n = n0 + u * kWG + tid;
      const long long nc = n <= m ? n : m;
      ra[u] = rows[2 * nc];
      rb[u] = rows[2 * nc + 1];
    }
    project_query(q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD, w_q + (size_t)r * kD * kR, sm.q,
                  sm.qtmp);
    double q[kR];
#pragma unroll
    for (int x = 0; x < kR; ++x) {
      const unsigned long long v = (unsigned long long)__double_as_longlong(sm.q[x]);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
      q[x] = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
    }
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int u = k % BATCH;
      const long long n = n0 + k * kWG + tid;
      const float sc = dot16_exact(q, ra[u], rb[u]);
      lg[k] = n <= m ? sc : -INFINITY;
      bin_abs(lg[k]);
      if (k + BATCH < TPT) {
        const long long nn = n + BATCH * kWG;
        const long long nc = nn <= m ? nn : m;
        ra[u] = rows[2 * nc];
        rb[u] = rows[2 * nc + 1];
      }
    }
  }
  block_max_min(mx, cmin, sm.red_f, sm.red_i);
  const int c_t = (mx == -INFINITY) ? INT32_MIN : score_cell(mx);

  // local bins j = c_t - cell; cells 255 or more below c_t form the clamp bin 255,
  // weighted relative to its base cell c_t - 255
  unsigned long long packed = 0;
  // (a span of at most kCells - 2 keeps every cell unique mod kCells and the clamp
  // cells c_t - 255 .. cmin within the 256 threads below)
  if (c_t != INT32_MIN && (long long)c_t - cmin <= kCells - 2) {
    const int j = tid;
    if (j < kBins - 1) {
      const int cell = c_t - j;
#pragma unroll
      for (int w = 0; w < 4; ++w) packed += sm.hist[w][cell & (kCells - 1)];
    }
    // clamp bin: cells c_t - 255 - x for x = 0..(c_t - 255 - cmin), if any
    if ((long long)cmin <= (long long)c_t - (kBins - 1)) {            // block-uniform
      const long long cell = (long long)c_t - (kBins - 1) - tid;
      double cm = 0.0;
      unsigned long long cc = 0;
      if (cell >= cmin) {
        unsigned long long e = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) e += sm.hist[w][cell & (kCells - 1)];
        cm = (double)(e & kMassMask) * bin_scale(g, -(double)tid * 0.125);
        cc = e >> kCountShift;
      }
      double tm;
      (void)block_excl_scan<double>(cm, tm, sm.red_d);
      unsigned long long tc;
      (void)block_excl_scan<unsigned long long>(cc, tc, sm.red_u);
      if (j == kBins - 1) packed = (unsigned long long)tm | (tc << kCountShift);
    }
  } else {
    // cells of this tile span kCells or more: rebin relative to c_t from the scores in registers
    __syncthreads();
    for (int x = tid; x < 4 * kBins; x += kWG) sm.hist[x / kBins][x % kBins] = 0ull;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const float sc = lg[k];
      if (sc == -INFINITY) continue;
      const int cell = score_cell(sc);
      const int jb = c_t - cell >= kBins - 1 ? kBins - 1 : c_t - cell;
      const uint32_t u = jb == kBins - 1 ? token_weight(g, sc, c_t - (kBins - 1)) : token_weight(g, sc, cell);
      atomicAdd(&sm.hist[wv][jb], (unsigned long long)u | (1ull << kCountShift));
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) packed += sm.hist[w][tid];
  }

  // codes (local bins) from the scores in registers
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const float sc = lg[k];
    uint8_t code = 255;
    if (sc != -INFINITY) {
      const int jb = c_t - score_cell(sc);
      code = (uint8_t)(jb >= kBins - 1 ? kBins - 1 : jb);
    }
    sm.codes[k * kWG + tid] = code;
  }
  __syncthreads();
  {
    uint8_t *dst = g.codes + (size_t)unit * g.nt * T + (size_t)t * T + (size_t)tid * TPT;
    const uint8_t *src = sm.codes + tid * TPT;
    if constexpr (TPT % 16 == 0) {
#pragma unroll
      for (int k = 0; k < TPT; k += 16)
        *reinterpret_cast<uint4 *>(dst + k) = *reinterpret_cast<const uint4 *>(src + k);
    } else {
#pragma unroll
      for (int k = 0; k < TPT; k += 4)
        *reinterpret_cast<uint32_t *>(dst + k) = *reinterpret_cast<const uint32_t *>(src + k);
    }
  }

  // tile summary, read by the merge kernel
  TileSum *tsum = g.tsum + (size_t)unit * g.nt + t;
  const unsigned long long ms = packed & kMassMask;
  const unsigned int cn = (unsigned int)(packed >> kCountShift);
  unsigned int tot;
  const unsigned int ex = block_excl_scan<unsigned int>(cn, tot, sm.red_u32);
  tsum->mass[tid] = ms;
  tsum->cum[tid] = ex + cn;
  if (tid == 0) {
    tsum->c_t = c_t;
    tsum->nvalid = (int32_t)tot;
  }
  // absolute-cell histogram of the query: exact integer sums in any order
  if (c_t != INT32_MIN) {
    if (tid == 0) {
      atomicMax(g.cmax + unit, enc_max(c_t));
      atomicMax(g.cmin + unit, enc_min(c_t - (kBins - 1)));
    }
    if (ms) atomicAdd((unsigned long long *)(g.ring + (size_t)unit * kRing + ((c_t - tid) & (kRing - 1))), ms);
  }
  // the query's prepared forms for the finishing workgroups: the indexer query
  // and the rotated, scaled attention query
  if (!FROM_LOGITS && t == 0) {
    QPrep *qp = g.qprep + unit;
    if (tid < kR) qp->qi[tid] = sm.q[tid];
    rope_table(m, g.theta, sm.rope);
    rotate_query(q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD, sm.rope, kInvSqrtD, qp->qrot);
  }
}

template <int T>
union PhaseAShared {
  ScanShared<T> scan;
  SwaShared swa;
};

// Phase A: the local heads' sliding-window workgroups (first) and the
// retrieval heads' scan tiles in one launch.  RING: the layer has ring groups.
template <int T, bool FROM_LOGITS, bool RING>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4, 8))) void phase_a_kernel(Geo g, const rtp_bf16 *__restrict__ q_pre,
                                                      const rtp_bf16 *__restrict__ w_q,
                                                      const rtp_bf16 *__restrict__ k_idx,
                                                      const float *__restrict__ logits,
                                                      const rtp_bf16 *__restrict__ kc,
                                                      const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                                      long long n_swa, int defer_swa) {
  __shared__ PhaseAShared<T> sm;
  const long long x = blockIdx.x;
  if (x < n_swa)
    swa_block<RING>(g, x, q_pre, kc, vc, out, sm.swa, defer_swa != 0);
  else
    scan_block<T, FROM_LOGITS>(g, x - n_swa, q_pre, w_q, k_idx, logits, sm.scan);
}

// Per-workgroup scratch of the global threshold.
struct ThrScratch {
  double wcum[kBins];
  double red_d[4];
  unsigned long long red_u[4];
  uint32_t red_u32[4];
  int red_i[4];
};

// The query's global histogram from the ring (or, when its cells span more
// than the ring holds, from every tile histogram): boundary bin b*, residual
// mass in in-cell units of bin b*, and whether every position is taken.
// H_ring is this thread's ring entry for bin j = tid (cell c - j), loaded by
// the caller.  Every workgroup of a query computes identical values: the
// integer bins are exact and every floating-point sum has a fixed order.
__device__ __forceinline__ void global_threshold(const Geo &g, int unit, int c, int base_min,
                                                 unsigned long long H_ring, unsigned long long R1,
                                                 ThrScratch &sm, int &bstar_out, double &r_u_out, int &all_out) {
  const int tid = threadIdx.x, j = tid;
  const TileSum *ts = g.tsum + (size_t)unit * g.nt;
  const uint64_t *ring = g.ring + (size_t)unit * kRing;
  const long long span = (long long)c - base_min;
  unsigned long long H = 0;
  double w255 = 0.0;
  if (span < kRing) {
    // clamp cells c - 255 - j - 256 x, x = 0, 1, ...: the first one (R1) was loaded by the caller
    H = j <= kBnd ? H_ring : 0ull;
    const long long cell1 = (long long)c - (kBins - 1) - j;
    if (R1) w255 += (double)R1 * bin_scale(g, (double)(cell1 - c) * 0.125);
    for (long long cell = cell1 - kWG; cell >= base_min; cell -= kWG) {
      const unsigned long long mj = ring[cell & (kRing - 1)];
      if (mj) w255 += (double)mj * bin_scale(g, (double)(cell - c) * 0.125);
    }
  } else {
    for (int t = 0; t < g.nt; ++t) {
      const int ct = ts[t].c_t;
      if (ct == INT32_MIN) continue;
      const long long d = (long long)c - ct;
      if (j <= kBnd && j - d >= 0) H += ts[t].mass[j - d];
      if (j + d >= kBins - 1) {
        const unsigned long long mj = ts[t].mass[j];
        if (mj) w255 += (double)mj * bin_scale(g, -(double)(j + d) * 0.125);
      }
    }
  }
  // clamp-bin mass: fixed pairwise tree over the threads
  sm.wcum[j] = w255;
  __syncthreads();
#pragma unroll
  for (int s = kWG / 2; s > 0; s >>= 1) {
    if (j < s) sm.wcum[j] += sm.wcum[j + s];
    __syncthreads();
  }
  const double W255 = sm.wcum[0] * 0x1p-23;
  __syncthreads();
  const double Wj = j <= kBnd ? (double)H * 0x1p-23 * bin_scale(g, -(double)j * 0.125) : W255;
  double Z;
  const double excl = block_excl_scan<double>(Wj, Z, sm.red_d);
  // Top-P needs the mass p Z; top-k needs k tokens (every weight is exactly 1,
  // so Z is the number of positions and every sum here is an exact integer)
  const double need = g.topk ? (double)g.topk : (double)g.p * Z;
  int bstar = block_min<int>(excl + Wj >= need ? j : kBins, sm.red_i);
  if (bstar >= kBins) bstar = kBins - 1;
  sm.wcum[j] = excl;                      // mass above bin j
  __syncthreads();
  const double before = sm.wcum[bstar];
  __syncthreads();
  // Top-P: p >= 1, or the boundary in the clamp bin (whose in-cell masses
  // have no common scale; its mass is below e^-31.75 of the top cell, so
  // everything is taken).  Top-k: k covers every position.
  all_out = (g.topk ? need >= Z : (g.p >= 1.0f || bstar >= kBins - 1)) ? 1 : 0;
  r_u_out = (need - before) * 0x1p23 * bin_scale(g, (double)bstar * 0.125);
  bstar_out = bstar;
}

// Local codes [lo, hi] of a tile (max cell ct) that hold the query's boundary
// bin b*; codes below lo lie above b*.  A regular b* is one local bin (or none:
// lo = hi = -1).  The clamp bin, a boundary only for top-k, gathers every
// local bin at or below the query's cell c - 255.
__device__ __forceinline__ void bnd_range(int bstar, int c, int ct, int &lo, int &hi) {
  const long long d = (long long)c - ct;
  if (bstar <= kBnd) {
    const long long bl = (long long)bstar - d;
    lo = hi = bl < 0 ? -1 : (int)bl;
  } else {
    const long long l = (long long)(kBins - 1) - d;
    lo = l < 0 ? 0 : (int)l;
    hi = kBins - 1;
  }
}

struct FinShared {
  static constexpr int kList = 2048;
  static constexpr int kCodes = 32768;
  uint8_t codes[kCodes];                   // codes of this workgroup's tiles
  int list[kList];                         // positions pending attention
  int blist[kWG];                          // bin-b* positions of the crossing tile, one round
  TileSel tsel[32];                        // selection parameters of this workgroup's tiles
  int ct[32];
  float q[kD];
  double qi[kR];
  int flag;
  union {
    ThrScratch thr;
    AttnShared at;
    CombineShared cb;
  };
  Partial res;
};

// Finish kernel: one workgroup per (query unit, run of fin_tpw tiles).
// Each workgroup first derives the query's threshold from the ring and the
// per-tile prefix of bin-b* mass over all tiles (identical in every workgroup
// of the query).  Tiles before the crossing tile take their whole bin b*,
// tiles after it none; the crossing tile takes the ordered prefix of its
// bin-b* tokens whose preceding mass is below the residual (their scores are
// recomputed in parallel).  Selected positions are written (optional) and
// attended (optional); the last workgroup of the query combines the states
// and resets the ring.
template <int T, bool FROM_LOGITS, bool ATTEND, bool RING>
__global__ __launch_bounds__(kWG) void finish_kernel(Geo g, const rtp_bf16 *__restrict__ k_idx,
                                                     const float *__restrict__ logits,
                                                     const rtp_bf16 *__restrict__ kc,
                                                     const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                                     int32_t *__restrict__ idx, int32_t *__restrict__ count,
                                                     long long cap) {
  constexpr int TPT = T / kWG;             // positions per thread per tile (consecutive)
  static_assert(T <= FinShared::kCodes, "tile larger than the code staging area");
  __shared__ FinShared sm;
  if (ATTEND && blockIdx.x >= (unsigned)(g.units * g.fin_nwg)) {   // deferred window chunk states
    swa_combine_block(g, (long long)blockIdx.x - (long long)g.units * g.fin_nwg, out);
    return;
  }
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / g.fin_nwg, w = blockIdx.x % g.fin_nwg;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int hq = g.rhead[r];
  const long long m = g.N - g.nq + i;
  const int t_begin = w * g.fin_tpw;
  const int t_end = t_begin + g.fin_tpw < g.nt ? t_begin + g.fin_tpw : g.nt;
  const int kvg = hq / g.G;
  const size_t cbase = kv_group_elems<RING>(g, b, kvg);
  const TileSum *ts = g.tsum + (size_t)unit * g.nt;

  // Loads are counted in issue order (vmcnt), so everything the threshold
  // needs is requested before the bulk of codes: the cell range, the first
  // tile maxima and the prepared query, then the ring cells, then the codes.
  const int c = dec_max(g.cmax[unit]);
  const int base_min = dec_min(g.cmin[unit]);
  const int ct0 = tid < g.nt ? ts[tid].c_t : INT32_MIN;
  double qi_v = 0.0;
  float qrot_v = 0.f;
  if (!FROM_LOGITS && tid < kR) qi_v = g.qprep[unit].qi[tid];
  if (ATTEND && tid < kD) qrot_v = g.qprep[unit].qrot[tid];
  const uint64_t *ring = g.ring + (size_t)unit * kRing;
  const unsigned long long H_ring = ring[(c - tid) & (kRing - 1)];
  const long long cell1 = (long long)c - (kBins - 1) - tid;
  const unsigned long long R1 = ((long long)c - base_min < kRing && cell1 >= base_min) ? ring[cell1 & (kRing - 1)] : 0ull;
  {
    // every code of this run goes straight from memory to LDS (gfx950 LDS-DMA
    // loads: lane l of a wave lands at the wave's base + 16 l), so nothing is
    // held in registers while the threshold is worked out
    constexpr int kPer = FinShared::kCodes / 16 / kWG;
    const uint4 *src = reinterpret_cast<const uint4 *>(g.codes + (size_t)unit * g.nt * T + (size_t)t_begin * T);
    const int n16 = (t_end - t_begin) * T / 16;            // a multiple of 64
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int x0 = u * kWG + (tid & ~63);                 // the wave's first 16-byte slot
      if (x0 < n16)
        __builtin_amdgcn_global_load_lds(src + x0 + (tid & 63),
                                         (__attribute__((address_space(3))) void *)(sm.codes + (size_t)x0 * 16),
                                         16, 0, 0);
    }
  }
  if (!FROM_LOGITS && tid < kR) sm.qi[tid] = qi_v;
  if (ATTEND && tid < kD) sm.q[tid] = qrot_v;

  int bstar, all;
  double r_u;
  global_threshold(g, unit, c, base_min, H_ring, R1, sm.thr, bstar, r_u, all);

  // per tile of the query: bin-b* prefix mass, counts above b* and in b*,
  // output offsets; the crossing tile is the last one whose bin-b* tokens
  // start below the residual, and every bin-b* token before it is taken
  unsigned long long carryP = 0;
  int carryS = 0, carryB = 0, tstar = -1, bo_star = -1;
  for (int t0 = 0; t0 < g.nt; t0 += kWG) {
    const int tt = t0 + tid;
    unsigned long long bm = 0;
    int sure = 0, bc = 0;
    const int ctt = t0 == 0 ? ct0 : (tt < g.nt ? ts[tt].c_t : INT32_MIN);
    if (ctt != INT32_MIN && !all) {
      int lo, hi;
      bnd_range(bstar, c, ctt, lo, hi);
      if (lo >= 1) sure = (int)ts[tt].cum[lo - 1];
      if (hi >= 0) {
        bc = (int)(ts[tt].cum[hi] - (lo ? ts[tt].cum[lo - 1] : 0u));
        bm = g.topk ? (unsigned long long)bc << 23 : ts[tt].mass[lo];
      }
    }
    unsigned long long totP, totSB;
    const unsigned long long P = carryP + block_excl_scan<unsigned long long>(bm, totP, sm.thr.red_u);
    const unsigned long long sb =
        block_excl_scan<unsigned long long>(((unsigned long long)sure << 32) | (unsigned)bc, totSB, sm.thr.red_u);
    const int so = carryS + (int)(sb >> 32), bo = carryB + (int)(sb & 0xffffffffu);
    if (tt >= t_begin && tt < t_end) {
      TileSel &tl = sm.tsel[tt - t_begin];
      tl.P = P;
      tl.sure_off = so;
      tl.bnd_off = bo;
      tl.n_sure = sure;
      tl.n_bnd = bc;
      sm.ct[tt - t_begin] = ctt;
    }
    const bool crossing = tt < g.nt && bc > 0 && (double)P < r_u;
    tstar = max(tstar, block_max<int>(crossing ? tt : -1, sm.thr.red_i));
    bo_star = max(bo_star, block_max<int>(crossing ? bo : -1, sm.thr.red_i));
    carryP += totP;
    carryS += (int)(totSB >> 32);
    carryB += (int)(totSB & 0xffffffffu);
  }
  const int total_sure = carryS;
  const int count_base = carryS + (tstar >= 0 ? bo_star : 0);
  if (count && tid == 0 && w == 0) {
    if (all) count[unit] = (int)(m + 1);
    else if (tstar < 0) count[unit] = count_base;
  }
  __builtin_amdgcn_s_waitcnt(0);                        // this wave's code loads have landed in LDS
  __syncthreads();

  float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;    // thread d < 128 holds channel d
  int nlist = 0;                                        // block-uniform
  for (int t = t_begin; t < t_end; ++t) {
    const TileSel tl = sm.tsel[t - t_begin];
    const int ct = sm.ct[t - t_begin];
    if (ct == INT32_MIN) continue;                      // no position in the tile
    int lo = -1, hi = -1;
    if (!all) bnd_range(bstar, c, ct, lo, hi);
    const bool bnd_ok = !all && hi >= 0;
    const bool crossing = bnd_ok && t == tstar;
    const bool take_all_bnd = bnd_ok && t < tstar;
    // block-uniform skip of a tile that contributes nothing
    if (!all && tl.n_sure == 0 && !((take_all_bnd || crossing) && tl.n_bnd > 0)) continue;
    const long long n0 = (long long)t * T;
    const long long nbase = n0 + (long long)tid * TPT;
    // this thread's TPT consecutive codes, read as words
    uint32_t cw[TPT / 4];
    {
      const uint8_t *cd = sm.codes + (t - t_begin) * T + tid * TPT;
      if constexpr (TPT >= 16) {
#pragma unroll
        for (int v = 0; v < TPT / 16; ++v) {
          const uint4 x4 = reinterpret_cast<const uint4 *>(cd)[v];
          cw[4 * v] = x4.x;
          cw[4 * v + 1] = x4.y;
          cw[4 * v + 2] = x4.z;
          cw[4 * v + 3] = x4.w;
        }
      } else {
#pragma unroll
        for (int v = 0; v < TPT / 4; ++v) cw[v] = reinterpret_cast<const uint32_t *>(cd)[v];
      }
    }
    const long long lim = m - nbase;                    // positions beyond the query are never taken
    const unsigned valid_m = lim >= TPT - 1 ? (TPT == 32 ? 0xffffffffu : ((1u << TPT) - 1u))
                                            : (lim < 0 ? 0u : ((1u << (lim + 1)) - 1u));
    unsigned sure_m = 0, bnd_m = 0;
    if (all) {
      sure_m = valid_m;
    } else {
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int code = (int)((cw[k >> 2] >> (8 * (k & 3))) & 0xffu);
        sure_m |= (code < lo ? 1u : 0u) << k;
        bnd_m |= (code >= lo && code <= hi ? 1u : 0u) << k;
      }
      sure_m &= valid_m;
      bnd_m = (take_all_bnd || crossing) ? (bnd_m & valid_m) : 0u;
    }
    unsigned take_m = take_all_bnd ? bnd_m : 0u;
    int emitted_b = 0;
    if (crossing) {
      // ordered fill of bin b*: the tile's bin-b* tokens in position order, a
      // round of 256 at a time, each weighed by one thread; a token is taken
      // while the mass before it is below the residual, so the taken tokens
      // are a prefix of that order
      int nbt;
      const int boff = block_excl_scan<int>(__popc(bnd_m), nbt, sm.thr.red_i);
      nbt = nbt < T ? nbt : T;
      unsigned long long pre = tl.P;
      int ntake = 0;
      for (int r0 = 0; r0 < nbt; r0 += kWG) {
        int jx = boff;
        for (unsigned mm = bnd_m; mm; mm &= mm - 1, ++jx)
          if (jx >= r0 && jx < r0 + kWG) sm.blist[jx - r0] = (int)(nbase + __builtin_ctz(mm));
        __syncthreads();
        const int cnt = nbt - r0 < kWG ? nbt - r0 : kWG;
        uint32_t wt = 0;                                  // < 1.14 * 2^23 each, < 2^32 per round
        if (tid < cnt && g.topk) {
          wt = kUnitWeight;                               // top-k: every token counts once
        } else if (tid < cnt) {
          long long n = sm.blist[tid];
          n = n < 0 ? 0 : (n > m ? m : n);
          float sc;
          if (FROM_LOGITS) {
            sc = logits[(size_t)unit * g.N + n];
          } else {
            const uint4 *rows = reinterpret_cast<const uint4 *>(k_idx + ((size_t)b * g.Hi + r / g.ig) * g.Ncap * kR);
            sc = dot16_exact(sm.qi, rows[2 * n], rows[2 * n + 1]);
          }
          wt = cell_weight(sc, score_cell(sc));
        }
        uint32_t tot_w;
        const uint32_t ex = block_excl_scan<uint32_t>(wt, tot_w, sm.thr.red_u32);
        int ntk;
        (void)block_excl_scan<int>(tid < cnt && (double)(pre + ex) < r_u ? 1 : 0, ntk, sm.thr.red_i);
        ntake += ntk;
        pre += tot_w;
        if (ntk < cnt) break;                           // block-uniform
      }
      int jx = boff;
      for (unsigned mm = bnd_m; mm; mm &= mm - 1, ++jx)
        if (jx < ntake) take_m |= 1u << __builtin_ctz(mm);
      emitted_b = ntake;
    }
    // one scan for both ranks: positions above b* in the low half, bin-b* in the high half
    int tot;
    const int ex = block_excl_scan<int>(__popc(sure_m) | (__popc(take_m) << 16), tot, sm.thr.red_i);
    const int rs = ex & 0xffff, rb = ex >> 16;
    const int ts_ = min(tot & 0xffff, T), tb_ = min(tot >> 16, T);
    if (crossing && count && tid == 0) count[unit] = count_base + emitted_b;
    if (idx) {   // positions above b* first, then the taken bin-b* positions, each ascending
      int32_t *dst = idx + (size_t)unit * cap;
      long long a = (all ? n0 : (long long)tl.sure_off) + rs;
      for (unsigned mm = sure_m; mm; mm &= mm - 1, ++a)
        if ((unsigned long long)a < (unsigned long long)cap) dst[a] = (int)(nbase + __builtin_ctz(mm));
      long long c2 = (long long)total_sure + tl.bnd_off + rb;
      for (unsigned mm = take_m; mm; mm &= mm - 1, ++c2)
        if ((unsigned long long)c2 < (unsigned long long)cap) dst[c2] = (int)(nbase + __builtin_ctz(mm));
    }
    if (ATTEND) {
      const int add = ts_ + tb_;
      if (nlist + add > FinShared::kList && nlist > 0) {   // flush the pending list
        attend_rows(sm.q, sm.list, nlist, g.N, kc + cbase, vc + cbase, &sm.res, &sm.at);
        if (tid < kD) merge_state(run_m, run_l, &run_o, sm.res.m, sm.res.l, &sm.res.o[tid], 1);
        nlist = 0;
      }
      if (add <= FinShared::kList) {
        int a = nlist + rs;
        for (unsigned mm = sure_m; mm; mm &= mm - 1) sm.list[a++] = (int)(nbase + __builtin_ctz(mm));
        a = nlist + ts_ + rb;
        for (unsigned mm = take_m; mm; mm &= mm - 1) sm.list[a++] = (int)(nbase + __builtin_ctz(mm));
        nlist += add;
        __syncthreads();
      } else {
        // a tile with more selected positions than the list: attend it in pieces
        for (int l0 = 0; l0 < add; l0 += FinShared::kList) {
          __syncthreads();
          int a = rs;
          for (unsigned mm = sure_m; mm; mm &= mm - 1, ++a)
            if (a >= l0 && a < l0 + FinShared::kList) sm.list[a - l0] = (int)(nbase + __builtin_ctz(mm));
          a = ts_ + rb;
          for (unsigned mm = take_m; mm; mm &= mm - 1, ++a)
            if (a >= l0 && a < l0 + FinShared::kList) sm.list[a - l0] = (int)(nbase + __builtin_ctz(mm));
          __syncthreads();
          const int cnt = add - l0 < FinShared::kList ? add - l0 : FinShared::kList;
          attend_rows(sm.q, sm.list, cnt, g.N, kc + cbase, vc + cbase, &sm.res, &sm.at);
          if (tid < kD) merge_state(run_m, run_l, &run_o, sm.res.m, sm.res.l, &sm.res.o[tid], 1);
        }
      }
    }
  }
  if (ATTEND) {
    if (nlist > 0) {
      attend_rows(sm.q, sm.list, nlist, g.N, kc + cbase, vc + cbase, &sm.res, &sm.at);
      if (tid < kD) merge_state(run_m, run_l, &run_o, sm.res.m, sm.res.l, &sm.res.o[tid], 1);
    }
    Partial *dst = g.part + (size_t)unit * g.fin_nwg + w;
    if (tid < kD) {
      st_coherent(&dst->o[tid], run_o);
      if (tid == 0) {
        st_coherent(&dst->m, run_m);
        st_coherent(&dst->l, run_l);
      }
    }
  }
  if (!arrive_last(g.ctr_fin + unit, (uint32_t)g.fin_nwg, &sm.flag)) return;
  // last workgroup of the query (every workgroup has read the ring): reset the
  // ring and the cell range for the next call, combine the states
  {
    uint64_t *ring = g.ring + (size_t)unit * kRing;
    if ((long long)c - base_min < kRing) {
      for (long long cell = (long long)base_min + tid; cell <= c; cell += kWG) ring[cell & (kRing - 1)] = 0ull;
    } else {
      for (int x = tid; x < kRing; x += kWG) ring[x] = 0ull;
    }
    if (tid == 0) {
      g.cmax[unit] = 0u;
      g.cmin[unit] = 0u;
    }
  }
  if (ATTEND)
    combine_partials(g.part + (size_t)unit * g.fin_nwg, g.fin_nwg,
                     out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, &sm.cb);
}

template <int T>
int launch_phase_a_t(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                     const float *logits, const rtp_bf16 *k, const rtp_bf16 *v, float *out, bool with_swa,
                     bool defer, hipStream_t s) {
  const long long n_swa = with_swa ? swa_blocks(g) : 0;
  const long long grid = n_swa + (g.units ? scan_blocks(g) : 0);
  if (grid == 0) return RTP_OK;
  // scores given as logits come without local heads (no K/V read)
  if (logits)
    hipLaunchKernelGGL((phase_a_kernel<T, true, false>), dim3((unsigned)grid), dim3(kWG), 0, s, g, q_pre, w_q, k_idx,
                       logits, k, v, out, n_swa, 0);
  else if (g.any_ring && n_swa)
    hipLaunchKernelGGL((phase_a_kernel<T, false, true>), dim3((unsigned)grid), dim3(kWG), 0, s, g, q_pre, w_q, k_idx,
                       logits, k, v, out, n_swa, defer ? 1 : 0);
  else
    hipLaunchKernelGGL((phase_a_kernel<T, false, false>), dim3((unsigned)grid), dim3(kWG), 0, s, g, q_pre, w_q,
                       k_idx, logits, k, v, out, n_swa, defer ? 1 : 0);
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

template <int T>
int launch_finish_t(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                    const float *logits, const rtp_bf16 *k, const rtp_bf16 *v, float *out, int32_t *idx,
                    int32_t *count, long long cap, bool swa_combine, hipStream_t s) {
  const unsigned grid = (unsigned)((long long)g.units * g.fin_nwg + (swa_combine ? swa_combine_blocks(g) : 0));
  if (grid == 0) return RTP_OK;
#define RTP_FIN(FL, AT, RG)                                                                                     \
  hipLaunchKernelGGL((finish_kernel<T, FL, AT, RG>), dim3(grid), dim3(kWG), 0, s, g, k_idx, logits, k, v, out, \
                     idx, count, cap)
  // only the attending build reads K/V, so only it has a ring-layout twin
  if (logits) {
    if (out) RTP_FIN(true, true, false); else RTP_FIN(true, false, false);
  } else if (out) {
    if (g.any_ring) RTP_FIN(false, true, true); else RTP_FIN(false, true, false);
  } else {
    RTP_FIN(false, false, false);
  }
#undef RTP_FIN
  return hipGetLastError() == hipSuccess ? RTP_OK : RTP_ERR_HIP;
}

}  // namespace

int launch_phase_a(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                   const float *logits, const rtp_bf16 *k, const rtp_bf16 *v, float *out, bool with_scan,
                   bool with_swa, hipStream_t s, bool defer_swa_combine) {
  Geo gg = g;
  if (!with_scan) gg.units = 0;
  if (!with_swa && gg.units == 0) return RTP_OK;
  const bool df = with_swa && defer_swa_combine;
  switch (gg.T) {
    case 1024: return launch_phase_a_t<1024>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 2048: return launch_phase_a_t<2048>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 4096: return launch_phase_a_t<4096>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 8192: return launch_phase_a_t<8192>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

int launch_finish(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                  const float *logits, const rtp_bf16 *k, const rtp_bf16 *v, float *out, int32_t *idx,
                  int32_t *count, long long cap, hipStream_t s, bool swa_combine) {
  if (g.units == 0) return RTP_OK;
  const bool sc = swa_combine && out && !logits;       // only the attending build merges window states
  switch (g.T) {
    case 1024: return launch_finish_t<1024>(g, q_pre, w_q, k_idx, logits, k, v, out, idx, count, cap, sc, s);
    case 2048: return launch_finish_t<2048>(g, q_pre, w_q, k_idx, logits, k, v, out, idx, count, cap, sc, s);
    case 4096: return launch_finish_t<4096>(g, q_pre, w_q, k_idx, logits, k, v, out, idx, count, cap, sc, s);
    case 8192: return launch_finish_t<8192>(g, q_pre, w_q, k_idx, logits, k, v, out, idx, count, cap, sc, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

}  // namespace rtp
