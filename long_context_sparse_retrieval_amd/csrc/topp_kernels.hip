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
// loads, keeps the tile's scores in registers, and builds per-wave
// histograms in LDS with integer atomics.  Bins are 1/8 logit wide on a fixed
// grid, so tile histograms merge exactly by an integer shift; masses are
// summed as exact 64-bit integers of in-cell weights (deterministic in any
// order).  Each tile adds its masses into an exact absolute-cell ring of its
// query; the query's last tile to finish reads the ring once and derives the
// whole selection: the boundary bin b*, the residual mass, and per tile the
// bin-b* prefix mass, output offsets and the crossing tile.  The selection
// launch then starts from one round of loads: each of its workgroups re-reads
// one code byte per token of its tiles, takes every token above b* and the
// ordered prefix of bin b* in the crossing tile (recomputing only those
// tokens' scores), gathers their K/V rows and writes a split-K softmax state;
// the last workgroup of a query combines them.  The sliding-window workgroups
// of the local heads run inside the scan launch, so their latency hides under
// the indexer stream.
#include "block_util.h"
#include "swa.h"

namespace rtp {

namespace {

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

constexpr int kBnd = 254;   // highest regular bin; bin 255 is the clamp bin

constexpr int kCells = 2048;     // absolute score cells tracked per tile while streaming (256 logit units)
static_assert(4 * kBins <= kCells, "the rebinning reuses the streaming histogram's storage");

// A histogram entry packs the token count (bits 40..63) above the summed
// in-cell masses (bits 0..39; at most 8192 tokens of < 1.14 * 2^23 each).
constexpr int kCountShift = 40;
constexpr unsigned long long kMassMask = (1ull << kCountShift) - 1;

// Per-workgroup scratch of the global threshold.
struct ThrScratch {
  uint64_t ring[kRing];                    // the query's absolute-cell masses (cell mod kRing)
  unsigned long long tot[4][2];            // per-wave totals of the tile prefix
  int cross_t[4], cross_bo[4];             // per-wave last crossing tile and its offset
  int hit_j[4];
  double hit_before[4], hit_up[4];
  double last_before, last_up;
  double red_d[4];
  unsigned long long red_u[4];
  uint32_t red_u32[4];
  int red_i[4];
};

template <int T>
struct ScanShared {
  static constexpr int TPT = T / kWG;
  uint8_t codes[T];                        // local bin of every position of the tile
  unsigned long long hist[kCells];         // the tile's histogram by absolute cell mod kCells:
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


// Thread j's bin scales, exp(-j/8), exp(-(255 + j)/8) and exp(j/8) (1 for
// top-k): they depend on nothing loaded, so the selection computes them while
// its first loads are in flight.
struct ThrScales {
  double down, clamp0, up;
};
__device__ __forceinline__ ThrScales thr_scales(const Geo &g) {
  const int j = threadIdx.x;
  return ThrScales{bin_scale(g, -(double)j * 0.125), bin_scale(g, (double)(-(kBins - 1) - j) * 0.125),
                   bin_scale(g, (double)j * 0.125)};
}

// The query's global histogram from its ring (in LDS; or, when its cells span
// more than the ring holds, from every tile histogram): boundary bin b*,
// residual mass in in-cell units of bin b*, and whether every position is
// taken.  Every workgroup of a query computes identical values: the integer
// bins are exact and every floating-point sum has a fixed order.
__device__ __forceinline__ void global_threshold(const Geo &g, int unit, int c, int base_min, const ThrScales &scl,
                                                 ThrScratch &sm,
                                                 int &bstar_out, double &r_u_out, int &all_out) {
  const int tid = threadIdx.x, j = tid;
  const TileSum *ts = g.tsum + (size_t)unit * g.nt;
  const long long span = (long long)c - base_min;
  unsigned long long H = 0;
  double w255 = 0.0;
  if (span < kRing) {
    // bin j <= 254 is cell c - j; the clamp bin gathers cells c - 255 - j - 256 x, x = 0, 1, ...
    H = j <= kBnd ? sm.ring[(c - j) & (kRing - 1)] : 0ull;
    for (long long cell = (long long)c - (kBins - 1) - j; cell >= base_min; cell -= kWG) {
      const unsigned long long mj = sm.ring[cell & (kRing - 1)];
      const bool first = cell == (long long)c - (kBins - 1) - j;
      if (mj) w255 += (double)mj * (first ? scl.clamp0 : bin_scale(g, (double)(cell - c) * 0.125));
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
  // clamp-bin mass, summed in a fixed order (wave_sum_f64_last inside each
  // wave, the four wave sums in wave order), so every workgroup gets the same
  // bits
  const int lane = j & 63, wv = j >> 6;
  {
    const double v = wave_sum_f64_last(w255);
    if (lane == 63) sm.red_d[wv] = v;
  }
  __syncthreads();
  const double W255 = (((sm.red_d[0] + sm.red_d[1]) + sm.red_d[2]) + sm.red_d[3]) * 0x1p-23;
  __syncthreads();
  const double Wj = j <= kBnd ? (double)H * 0x1p-23 * scl.down : W255;
  double Z;
  const double excl = block_excl_scan<double>(Wj, Z, sm.red_d);
  // Top-P needs the mass p Z; top-k needs k tokens (every weight is exactly 1,
  // so Z is the number of positions and every sum here is an exact integer)
  const double need = g.topk ? (double)g.topk : g.p * Z;
  // b*: the first bin whose cumulative mass reaches the need, and the mass
  // above it (the last bin when none does, which only p >= 1 allows)
  const bool hit = excl + Wj >= need;
  const unsigned long long bal = __builtin_amdgcn_ballot_w64(hit);
  if (bal ? lane == __builtin_ctzll(bal) : lane == 0) {
    sm.hit_j[wv] = bal ? j : kBins;
    sm.hit_before[wv] = excl;
    sm.hit_up[wv] = scl.up;
  }
  if (j == kBins - 1) {
    sm.last_before = excl;
    sm.last_up = scl.up;
  }
  __syncthreads();
  int bstar = kBins;
  double before = sm.last_before, up = sm.last_up;    // exp(b* / 8)
#pragma unroll
  for (int w = 3; w >= 0; --w)
    if (sm.hit_j[w] < kBins) {
      bstar = sm.hit_j[w];
      before = sm.hit_before[w];
      up = sm.hit_up[w];
    }
  if (bstar >= kBins) bstar = kBins - 1;
  __syncthreads();
  // Top-P: p >= 1, or the boundary in the clamp bin (whose in-cell masses
  // have no common scale; its mass is below e^-31.75 of the top cell, so
  // everything is taken).  Top-k: k covers every position.
  all_out = (g.topk ? need >= Z : (g.p >= 1.0 || bstar >= kBins - 1)) ? 1 : 0;
  r_u_out = (need - before) * 0x1p23 * up;
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

// Position of score k of thread tid in a tile starting at n0: consecutive
// threads on consecutive positions for given logits; for indexer keys the
// pairing of the key stream (lane 2j: row R + j, lane 2j + 1: row R + 32 + j,
// R = n0 + 256 k + 64 wave).
template <bool FROM_LOGITS>
__device__ __forceinline__ long long scan_pos(long long n0, int k, int tid) {
  if (FROM_LOGITS) return n0 + k * kWG + tid;
  return n0 + k * kWG + (tid & ~63) + ((tid & 1) << 5) + ((tid & 63) >> 1);
}

// One scan workgroup: tile t of query unit (scan_unit_tile).
template <int T, bool FROM_LOGITS>
__device__ __forceinline__ void scan_block(const Geo &g, long long blk, const rtp_bf16 *__restrict__ q_pre,
                                           const rtp_bf16 *__restrict__ w_q, const rtp_bf16 *__restrict__ k_idx,
                                           const float *__restrict__ logits, ScanShared<T> &sm) {
  constexpr int TPT = T / kWG;
  constexpr int BATCH = TPT < 4 ? TPT : 4;
  const int tid = threadIdx.x, wv = tid >> 6;
  int unit, t;
  if (!scan_unit_tile(g, blk, unit, t)) return;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const long long m = g.N - g.nq + i;
  const long long n0 = (long long)t * T;

  // pass 1: every score is binned at once by its absolute cell (no tile max
  // needed), so the histogram work overlaps the stream, and each lane keeps
  // its scores' cells as 16-bit integers, two per register (kNoCell: no
  // position).  A tile whose cells leave 16 bits, or span more than the
  // streaming histogram holds, recomputes its scores afterwards (rare).  The
  // first batch of key rows is requested before the query projection.
  constexpr int kNoCell = -32768;
  uint32_t cl[(TPT + 1) / 2];
  // (the byte permute packs the low halves of two cells; the compiler does not
  // see through it, so it cannot keep the 32-bit cells alive instead)
  auto put_cell = [&](int k, int c) {
    cl[k >> 1] = (k & 1) ? __builtin_amdgcn_perm((uint32_t)c, cl[k >> 1], 0x05040100u) : (uint32_t)c;
  };
  auto get_cell = [&](int k) -> int {
    return (k & 1) ? ((int)cl[k >> 1] >> 16) : (int)(int16_t)(cl[k >> 1] & 0xffffu);
  };
  float mx = -INFINITY;
  int cmin = INT32_MAX;
  const bool topk = g.topk != 0;
  for (int x = tid; x < kCells; x += kWG) sm.hist[x] = 0ull;
  // bin one score by its absolute cell and return the cell clamped to 16 bits
  // (kNoCell for an absent score, -inf, which adds nothing when CHECK);
  // branchless, so a whole batch of rows stays one basic block and its loads
  // can be issued together
  auto bin_abs = [&](float sc, auto check_tag) -> int {
    constexpr bool CHECK = decltype(check_tag)::value;
    const bool ok = !CHECK || sc != -INFINITY;
    const float s = ok ? sc : 0.f;
    const int cell = score_cell(s);
    const uint32_t w = topk ? kUnitWeight : cell_weight(s, cell);
    const unsigned long long add = ok ? ((unsigned long long)w | (1ull << kCountShift)) : 0ull;
    atomicAdd(&sm.hist[cell & (kCells - 1)], add);
    mx = fmaxf(mx, sc);
    cmin = min(cmin, ok ? cell : INT32_MAX);
    const int c16 = min(max(cell, -32767), 32767);
    return ok ? c16 : kNoCell;
  };
  // key path: the tile's rows at or before m form one buffer range (loads
  // past it return zeros).  Each load instruction covers 1 KB of consecutive
  // key rows: lane 2j + h of a wave reads half h (8 dims) of row R + j and of
  // row R + 32 + j, so the two lanes of a pair hold complementary halves of
  // two rows.  Each lane forms the two exact half-dots, the pair swaps one of
  // them, and lane 2j keeps the score of row R + j, lane 2j + 1 that of row
  // R + 32 + j (scan_pos); halves of an exact dot add exactly.  (Lanes that
  // read different halves of one 128-byte line in two instructions would
  // fetch the line twice: non-temporal loads do not keep it.)
  const long long valid = m + 1 - n0 < T ? (m + 1 - n0 > 0 ? m + 1 - n0 : 0) : T;
  const int lpos = (int)scan_pos<FROM_LOGITS>(0, 0, tid);
  constexpr int kStep = kWG * 32;                                    // bytes of key rows per step
  double qh[kR / 2];                                                 // this lane's half of q_idx
  const int h = tid & 1, jr = (tid & ~63) + ((tid & 63) >> 1);
  const int voff_a = (jr * 2 + h) * 16, voff_b = ((jr + 32) * 2 + h) * 16;    // rows R + j, R + 32 + j
  // lane 2j sends its half of row R + 32 + j and keeps row R + j; lane 2j + 1
  // the other way round
  auto pair_score = [&](uint4 a, uint4 c) -> float {
    const double pa = dot8_exact(qh, a), pb = dot8_exact(qh, c);
    const double recv = swap_pair(h ? pa : pb);
    return (float)((h ? pb : pa) + recv);
  };
  const __amdgpu_buffer_rsrc_t rows =
      stream_rsrc(FROM_LOGITS ? (const void *)logits
                              : (const void *)(k_idx + (((size_t)b * g.Hi + r / g.ig) * g.Ncap + n0) * kR),
                  FROM_LOGITS ? 0u : (uint32_t)valid * 32u);
  const float *lrow = logits + (size_t)unit * g.N;
  // score k of this lane recomputed from memory (the stream's arithmetic)
  auto rescore = [&](int k) -> float {
    const bool in = k * kWG + lpos < valid;
    if constexpr (FROM_LOGITS) {
      const long long n = n0 + k * kWG + lpos;
      const float sc = lrow[in ? n : m];
      return in ? sc : -INFINITY;
    } else {
      const float sc = pair_score(ld_stream(rows, voff_a, k * kStep), ld_stream(rows, voff_b, k * kStep));
      return in ? sc : -INFINITY;
    }
  };
  if constexpr (FROM_LOGITS) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPT; ++k) put_cell(k, bin_abs(rescore(k), std::true_type{}));
  } else {
    // rolling window of BATCH row pairs per lane: slot u is refilled BATCH
    // steps ahead as soon as it is consumed
    uint4 ra[BATCH], rb[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      ra[u] = ld_stream(rows, voff_a, u * kStep);
      rb[u] = ld_stream(rows, voff_b, u * kStep);
    }
    project_query(q_pre + (((size_t)b * g.Hq + g.rhead[r]) * g.nq + i) * kD, w_q + (size_t)r * kD * kR, sm.q,
                  sm.qtmp);
#pragma unroll
    for (int x = 0; x < kR / 2; ++x) qh[x] = sm.q[8 * h + x];
    // full tiles (every row at or before m) skip the validity test
    auto stream = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int u = k % BATCH;
        float sc = pair_score(ra[u], rb[u]);
        if (!FULL) sc = k * kWG + lpos < valid ? sc : -INFINITY;
        put_cell(k, bin_abs(sc, std::integral_constant<bool, !FULL>{}));
        if (k + BATCH < TPT) {
          ra[u] = ld_stream(rows, voff_a, (k + BATCH) * kStep);
          rb[u] = ld_stream(rows, voff_b, (k + BATCH) * kStep);
        }
      }
    };
    if (valid == T) stream(std::true_type{});
    else stream(std::false_type{});
  }
  block_max_min(mx, cmin, sm.red_f, sm.red_i);
  const int c_t = (mx == -INFINITY) ? INT32_MIN : score_cell(mx);

  // local bins j = c_t - cell; cells 255 or more below c_t form the clamp bin 255,
  // weighted relative to its base cell c_t - 255
  unsigned long long packed = 0;
  // (a span of at most kCells - 2 keeps every cell unique mod kCells; 16-bit
  // cells are exact)
  if (c_t != INT32_MIN && (long long)c_t - cmin <= kCells - 2 && c_t <= 32767 && cmin >= -32767) {
    const int j = tid;
    if (j < kBins - 1) packed = sm.hist[(c_t - j) & (kCells - 1)];
    // clamp bin: cells c_t - 255 - x for x = 0..(c_t - 255 - cmin), if any,
    // thread tid taking x = tid, tid + 256, ...
    if ((long long)cmin <= (long long)c_t - (kBins - 1)) {            // block-uniform
      double cm = 0.0;
      unsigned long long cc = 0;
      for (int x = tid; (long long)c_t - (kBins - 1) - x >= cmin; x += kWG) {
        const unsigned long long e = sm.hist[(c_t - (kBins - 1) - x) & (kCells - 1)];
        cm += (double)(e & kMassMask) * bin_scale(g, -(double)x * 0.125);
        cc += e >> kCountShift;
      }
      double tm;
      (void)block_excl_scan<double>(cm, tm, sm.red_d);
      unsigned long long tc;
      (void)block_excl_scan<unsigned long long>(cc, tc, sm.red_u);
      if (j == kBins - 1) packed = (unsigned long long)tm | (tc << kCountShift);
    }
    // codes (local bins) from the cells in registers
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int cell = get_cell(k);
      const int jb = c_t - cell;
      sm.codes[scan_pos<FROM_LOGITS>(0, k, tid)] =
          (uint8_t)(cell == kNoCell || jb >= kBins - 1 ? kBins - 1 : jb);
    }
  } else {
    // rebin relative to c_t, recomputing the scores (per-wave histograms of
    // the 256 local bins in the same array)
    __syncthreads();
    for (int x = tid; x < 4 * kBins; x += kWG) sm.hist[x] = 0ull;
    __syncthreads();
    for (int k = 0; k < TPT; ++k) {
      const float sc = rescore(k);
      uint8_t code = kBins - 1;
      if (sc != -INFINITY) {
        const int cell = score_cell(sc);
        const int jb = c_t - cell >= kBins - 1 ? kBins - 1 : c_t - cell;
        const uint32_t u = jb == kBins - 1 ? token_weight(g, sc, c_t - (kBins - 1)) : token_weight(g, sc, cell);
        atomicAdd(&sm.hist[wv * kBins + jb], (unsigned long long)u | (1ull << kCountShift));
        code = (uint8_t)jb;
      }
      sm.codes[scan_pos<FROM_LOGITS>(0, k, tid)] = code;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) packed += sm.hist[w * kBins + tid];
  }
  __syncthreads();
  {
    uint8_t *dst = g.codes + (size_t)unit * g.nt * T + (size_t)t * T + (size_t)tid * TPT;
    const uint8_t *src = sm.codes + tid * TPT;
    if constexpr (TPT % 16 == 0) {
#pragma unroll
      for (int k = 0; k < TPT; k += 16)
        __builtin_nontemporal_store(*reinterpret_cast<const v4u_t *>(src + k), reinterpret_cast<v4u_t *>(dst + k));
    } else {
#pragma unroll
      for (int k = 0; k < TPT; k += 4)
        __builtin_nontemporal_store(*reinterpret_cast<const uint32_t *>(src + k), reinterpret_cast<uint32_t *>(dst + k));
    }
  }

  // tile summary, read by the selection launch
  TileSum *tsum = g.tsum + (size_t)unit * g.nt + t;
  const unsigned long long ms = packed & kMassMask;
  const unsigned int cn = (unsigned int)(packed >> kCountShift);
  unsigned int tot;
  const unsigned int ex = block_excl_scan<unsigned int>(cn, tot, sm.red_u32);
  __builtin_nontemporal_store(ms, &tsum->mass[tid]);
  __builtin_nontemporal_store(ex + cn, &tsum->cum[tid]);
  if (tid == 0) {
    tsum->c_t = c_t;
    tsum->nvalid = (int32_t)tot;
  }
  // absolute-cell histogram of the query: exact integer sums in any order
  if (c_t != INT32_MIN) {
    if (tid == 0) {
      atomicMax(g.cmax + (size_t)unit * g.cstride, enc_max(c_t));
      atomicMax(g.cmin + (size_t)unit * g.cstride, enc_min(c_t - (kBins - 1)));
    }
    if (ms) atomicAdd((unsigned long long *)(g.ring + (size_t)unit * kRing + ((c_t - tid) & (kRing - 1))), ms);
  }
  // the query's prepared forms for the selection workgroups: the indexer
  // query and the rotated, scaled attention query
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

struct FinShared {
  static constexpr int kList = 2048;
  static constexpr int kCodes = 16384;
  static constexpr int kTiles = kCodes / 1024;
  uint8_t codes[kCodes];                   // codes of this workgroup's tiles
  int list[kList];                         // positions pending attention
  int blist[kWG];                          // bin-b* positions of the crossing tile, one round
  TileSel tsel[kTiles];                    // selection parameters of this workgroup's tiles
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

// Selection workgroup of query `unit` over its tiles t_begin..t_end-1 (one
// of fin_nwg per query), after the scan launch.  With two rounds of loads,
// every selection workgroup
// of the query derives the same threshold and per-tile parameters: round one
// brings the query's ring (exact masses per absolute cell), its cell range,
// every tile's max cell, the prepared query and this workgroup's codes
// (LDS-DMA); round two the tile summaries' entries at the boundary bin.
// Tiles before the crossing tile take their whole bin b*, tiles after it
// none; the crossing tile takes the ordered prefix of its bin-b* tokens whose
// preceding mass is below the residual (their scores are recomputed in
// parallel).  Selected positions are written (optional) and attended
// (optional); the last workgroup of the query combines the split-K states
// and leaves the query's ring and cell range zero.
template <int T, bool FROM_LOGITS, bool ATTEND, bool RING>
__device__ __forceinline__ void finish_block(const Geo &g, int y, const rtp_bf16 *__restrict__ k_idx,
                                             const float *__restrict__ logits, const rtp_bf16 *__restrict__ kc,
                                             const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                             int32_t *__restrict__ idx, int32_t *__restrict__ count, long long cap,
                                             FinShared &sm) {
  constexpr int TPT = T / kWG;             // positions per thread per tile (consecutive)
  static_assert(T <= FinShared::kCodes, "tile larger than the code staging area");
  const int tid = threadIdx.x;
  const int unit = y / g.fin_nwg, w = y % g.fin_nwg;
  const int i = unit % g.nq, br = unit / g.nq, r = br % g.Hr, b = br / g.Hr;
  const int hq = g.rhead[r];
  const long long m = g.N - g.nq + i;
  const int t_begin = w * g.fin_tpw;
  const int t_end = t_begin + g.fin_tpw < g.nt ? t_begin + g.fin_tpw : g.nt;
  const int kvg = hq / g.G;
  const size_t cbase = kv_group_elems<RING>(g, b, kvg);
  const TileSum *ts = g.tsum + (size_t)unit * g.nt;

  // round one
  const uint64_t *ring = g.ring + (size_t)unit * kRing;
  const uint32_t ecmax = g.cmax[(size_t)unit * g.cstride], ecmin = g.cmin[(size_t)unit * g.cstride];
  const int ct0 = tid < g.nt ? ts[tid].c_t : INT32_MIN;
  double qi_v = 0.0;
  float qrot_v = 0.f;
  if (!FROM_LOGITS && tid < kR) qi_v = g.qprep[unit].qi[tid];
  if (ATTEND && tid < kD) qrot_v = g.qprep[unit].qrot[tid];
  {
    // LDS-DMA (gfx950): lane l of a wave lands at the wave's base + 16 l
    const uint4 *src = reinterpret_cast<const uint4 *>(ring);
    constexpr int kPerRing = kRing * 8 / 16 / kWG;
#pragma unroll
    for (int u = 0; u < kPerRing; ++u) {
      const int x0 = u * kWG + (tid & ~63);
      __builtin_amdgcn_global_load_lds(src + x0 + (tid & 63),
                                       (__attribute__((address_space(3))) void *)(sm.thr.ring + (size_t)x0 * 2), 16,
                                       0, 0);
    }
    constexpr int kPer = FinShared::kCodes / 16 / kWG;
    const uint4 *csrc = reinterpret_cast<const uint4 *>(g.codes + (size_t)unit * g.nt * T + (size_t)t_begin * T);
    const int n16 = (t_end - t_begin) * T / 16;            // a multiple of 64
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int x0 = u * kWG + (tid & ~63);                 // the wave's first 16-byte slot
      if (x0 < n16)
        __builtin_amdgcn_global_load_lds(csrc + x0 + (tid & 63),
                                         (__attribute__((address_space(3))) void *)(sm.codes + (size_t)x0 * 16),
                                         16, 0, 0);
    }
  }
  const ThrScales scl = thr_scales(g);
  if (!FROM_LOGITS && tid < kR) sm.qi[tid] = qi_v;
  if (ATTEND && tid < kD) sm.q[tid] = qrot_v;
  __builtin_amdgcn_s_waitcnt(0);                        // this wave's ring and code loads have landed in LDS
  __syncthreads();

  const int c = dec_max(ecmax), base_min = dec_min(ecmin);
  int bstar, all;
  double r_u;
  global_threshold(g, unit, c, base_min, scl, sm.thr, bstar, r_u, all);

  // round two: per tile of the query, the bin-b* prefix mass, the counts above
  // b* and in b*, the output offsets; the crossing tile is the last one whose
  // bin-b* tokens start below the residual, and every bin-b* token before it
  // is taken
  unsigned long long carryP = 0, carrySB = 0;
  int tstar = -1, bo_star = -1;
  const int lane = tid & 63, wv = tid >> 6;
  for (int t0 = 0; t0 < g.nt; t0 += kWG) {
    const int tt = t0 + tid;
    unsigned long long bm = 0;
    int sure = 0, bc = 0;
    const int ctt = t0 == 0 ? ct0 : (tt < g.nt ? ts[tt].c_t : INT32_MIN);
    if (ctt != INT32_MIN && !all) {
      int lo, hi;
      bnd_range(bstar, c, ctt, lo, hi);
      const unsigned cum_lo = lo >= 1 ? ts[tt].cum[lo - 1] : 0u;
      if (lo >= 1) sure = (int)cum_lo;
      if (hi >= 0) {
        bc = (int)(ts[tt].cum[hi] - cum_lo);
        bm = g.topk ? (unsigned long long)bc << 23 : ts[tt].mass[lo];
      }
    }
    // inclusive prefixes inside the wave of the bin-b* mass and of the packed
    // (above b*, in b*) counts, then the wave totals through LDS
    const unsigned long long sbv = ((unsigned long long)sure << 32) | (unsigned)bc;
    const unsigned long long xp = wave_incl_scan64(bm), xs = wave_incl_scan64(sbv);
    if (lane == 63) {
      sm.thr.tot[wv][0] = xp;
      sm.thr.tot[wv][1] = xs;
    }
    __syncthreads();
    unsigned long long bp = carryP, bs = carrySB, tp = 0, tsb = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wv) {
        bp += sm.thr.tot[w][0];
        bs += sm.thr.tot[w][1];
      }
      tp += sm.thr.tot[w][0];
      tsb += sm.thr.tot[w][1];
    }
    const unsigned long long P = bp + xp - bm, sb = bs + xs - sbv;
    const int so = (int)(sb >> 32), bo = (int)(sb & 0xffffffffu);
    if (tt >= t_begin && tt < t_end) {
      TileSel &tl = sm.tsel[tt - t_begin];
      tl.P = P;
      tl.sure_off = so;
      tl.bnd_off = bo;
      tl.n_sure = sure;
      tl.n_bnd = bc;
      tl.ct = ctt;
    }
    // the crossing tile: the last with bin-b* tokens whose prefix mass is
    // below the residual (offsets grow with the tile, so its offset is the
    // largest among them)
    const bool crossing = tt < g.nt && bc > 0 && (double)P < r_u;
    const unsigned long long cb = __builtin_amdgcn_ballot_w64(crossing);
    if (lane == 0) sm.thr.cross_t[wv] = -1;
    if (cb && lane == 63 - __builtin_clzll(cb)) {
      sm.thr.cross_t[wv] = tt;
      sm.thr.cross_bo[wv] = bo;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (sm.thr.cross_t[w] >= 0) {
        tstar = sm.thr.cross_t[w];
        bo_star = sm.thr.cross_bo[w];
      }
    carryP += tp;
    carrySB += tsb;
    __syncthreads();
  }
  const int carryS = (int)(carrySB >> 32);
  const int total_sure = carryS;
  const int count_base = carryS + (tstar >= 0 ? bo_star : 0);
  if (count && tid == 0 && w == 0) {
    if (all) count[unit] = (int)(m + 1);
    else if (tstar < 0) count[unit] = count_base;
  }
  __syncthreads();

  float run_m = -INFINITY, run_l = 0.f, run_o = 0.f;    // thread d < 128 holds channel d
  int nlist = 0;                                        // block-uniform
  // Positions this run can take at most (workgroup-uniform): when they fit
  // the list, every tile is handled in one pass (masks, then one pair of
  // packed scans for all tiles); otherwise, and when every position is
  // taken, tile by tile.  Both build the same list in the same order.
  int bound = 0;
  for (int t = t_begin; t < t_end; ++t) {
    const TileSel &tl = sm.tsel[t - t_begin];
    bound += tl.n_sure + (t <= tstar ? tl.n_bnd : 0);
  }
  if (!all && bound <= FinShared::kList) {
    constexpr int kMaxT = FinShared::kCodes / T;        // tiles per run at most
    constexpr int kGroups = (kMaxT + 3) / 4;            // tiles per packed scan: 4 fields of 16 bits
    unsigned sure_m[kMaxT], take_m[kMaxT];
    unsigned cross_bnd = 0;
    int cross_tl = -1;
#pragma unroll
    for (int tl = 0; tl < kMaxT; ++tl) {
      sure_m[tl] = take_m[tl] = 0u;
      const int t = t_begin + tl;
      if (t >= t_end) continue;                         // workgroup-uniform
      const TileSel &ts_ = sm.tsel[tl];
      if (ts_.ct == INT32_MIN) continue;
      int lo, hi;
      bnd_range(bstar, c, ts_.ct, lo, hi);
      const bool bnd_ok = hi >= 0;
      const bool crossing = bnd_ok && t == tstar, take_all_bnd = bnd_ok && t < tstar;
      if (ts_.n_sure == 0 && !((take_all_bnd || crossing) && ts_.n_bnd > 0)) continue;
      const long long nbase = (long long)t * T + (long long)tid * TPT;
      uint32_t cw[TPT / 4];
      {
        const uint8_t *cd = sm.codes + tl * T + tid * TPT;
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
      const long long lim = m - nbase;
      const unsigned valid_m = lim >= TPT - 1 ? (TPT == 32 ? 0xffffffffu : ((1u << TPT) - 1u))
                                              : (lim < 0 ? 0u : ((1u << (lim + 1)) - 1u));
      unsigned sm_ = 0, bm_ = 0;
#pragma unroll
      for (int k = 0; k < TPT; ++k) {
        const int code = (int)((cw[k >> 2] >> (8 * (k & 3))) & 0xffu);
        sm_ |= (code < lo ? 1u : 0u) << k;
        bm_ |= (code >= lo && code <= hi ? 1u : 0u) << k;
      }
      sure_m[tl] = sm_ & valid_m;
      bm_ &= valid_m;
      if (take_all_bnd) take_m[tl] = bm_;
      if (crossing) {
        cross_bnd = bm_;
        cross_tl = tl;
      }
    }
    int emitted_b = 0;
    if (cross_tl >= 0) {                                // workgroup-uniform: this run holds the crossing tile
      // ordered fill of bin b* in the crossing tile (see the tile-by-tile path)
      const TileSel &ts_ = sm.tsel[cross_tl];
      const long long nbase = (long long)(t_begin + cross_tl) * T + (long long)tid * TPT;
      int nbt;
      const int boff = block_excl_scan<int>(__popc(cross_bnd), nbt, sm.thr.red_i);
      nbt = nbt < T ? nbt : T;
      unsigned long long pre = ts_.P;
      int ntake = 0;
      for (int r0 = 0; r0 < nbt; r0 += kWG) {
        int jx = boff;
        for (unsigned mm = cross_bnd; mm; mm &= mm - 1, ++jx)
          if (jx >= r0 && jx < r0 + kWG) sm.blist[jx - r0] = (int)(nbase + __builtin_ctz(mm));
        __syncthreads();
        const int cnt = nbt - r0 < kWG ? nbt - r0 : kWG;
        uint32_t wt = 0;
        if (tid < cnt && g.topk) {
          wt = kUnitWeight;
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
        if (ntk < cnt) break;
      }
      int jx = boff;
      unsigned tk = 0;
      for (unsigned mm = cross_bnd; mm; mm &= mm - 1, ++jx)
        if (jx < ntake) tk |= 1u << __builtin_ctz(mm);
#pragma unroll
      for (int tl = 0; tl < kMaxT; ++tl)
        if (tl == cross_tl) take_m[tl] = tk;
      emitted_b = ntake;
      if (count && tid == 0) count[unit] = count_base + emitted_b;
    }
    // ranks of this thread's positions in every tile: 16-bit fields, four
    // tiles per 64-bit scan (a tile holds at most 8192 positions)
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq) {
      unsigned long long ps = 0, pb = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tl = 4 * gq + q;
        if (tl < kMaxT) {
          ps |= (unsigned long long)__popc(sure_m[tl]) << (16 * q);
          pb |= (unsigned long long)__popc(take_m[tl]) << (16 * q);
        }
      }
      unsigned long long tS, tB;
      const unsigned long long eS = block_excl_scan<unsigned long long>(ps, tS, sm.thr.red_u);
      const unsigned long long eB = block_excl_scan<unsigned long long>(pb, tB, sm.thr.red_u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tl = 4 * gq + q;
        if (tl >= kMaxT || t_begin + tl >= t_end) continue;
        const int rs = (int)((eS >> (16 * q)) & 0xffffu), rb = (int)((eB >> (16 * q)) & 0xffffu);
        const int ts_n = (int)((tS >> (16 * q)) & 0xffffu), tb_n = (int)((tB >> (16 * q)) & 0xffffu);
        const long long nbase = (long long)(t_begin + tl) * T + (long long)tid * TPT;
        if (idx) {   // positions above b* first, then the taken bin-b* positions, each ascending
          const TileSel &ts_ = sm.tsel[tl];
          int32_t *dst = idx + (size_t)unit * cap;
          long long a = (long long)ts_.sure_off + rs;
          for (unsigned mm = sure_m[tl]; mm; mm &= mm - 1, ++a)
            if ((unsigned long long)a < (unsigned long long)cap) dst[a] = (int)(nbase + __builtin_ctz(mm));
          long long c2 = (long long)total_sure + ts_.bnd_off + rb;
          for (unsigned mm = take_m[tl]; mm; mm &= mm - 1, ++c2)
            if ((unsigned long long)c2 < (unsigned long long)cap) dst[c2] = (int)(nbase + __builtin_ctz(mm));
        }
        if (ATTEND) {
          int a = nlist + rs;
          for (unsigned mm = sure_m[tl]; mm; mm &= mm - 1) sm.list[a++] = (int)(nbase + __builtin_ctz(mm));
          a = nlist + ts_n + rb;
          for (unsigned mm = take_m[tl]; mm; mm &= mm - 1) sm.list[a++] = (int)(nbase + __builtin_ctz(mm));
        }
        nlist += ts_n + tb_n;
      }
    }
    __syncthreads();
  } else {
    for (int t = t_begin; t < t_end; ++t) {
      const TileSel tl = sm.tsel[t - t_begin];
      const int ct = tl.ct;
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
  if (!arrive_last(g.ctr_fin + (size_t)unit * g.cstride, (uint32_t)g.fin_nwg, &sm.flag)) return;
  // last workgroup of the query (every workgroup has read the ring): leave the
  // query's state zero for the next call, combine the states
  {
    uint64_t *ringw = g.ring + (size_t)unit * kRing;
    if ((long long)c - base_min < kRing) {
      for (long long cell = (long long)base_min + tid; cell <= c; cell += kWG) ringw[cell & (kRing - 1)] = 0ull;
    } else {
      for (int x = tid; x < kRing; x += kWG) ringw[x] = 0ull;
    }
    if (tid == 0) {
      g.cmax[(size_t)unit * g.cstride] = 0u;
      g.cmin[(size_t)unit * g.cstride] = 0u;
    }
  }
  if (ATTEND)
    combine_partials(g.part + (size_t)unit * g.fin_nwg, g.fin_nwg,
                     out + (((size_t)b * g.Hq + hq) * g.nq + i) * kD, &sm.cb);
}

// Selection launch after a scan launch: one workgroup per (query, run of tiles).
template <int T, bool FROM_LOGITS, bool ATTEND, bool RING>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4, 8))) void finish_kernel(Geo g, const rtp_bf16 *__restrict__ k_idx,
                                                     const float *__restrict__ logits,
                                                     const rtp_bf16 *__restrict__ kc,
                                                     const rtp_bf16 *__restrict__ vc, float *__restrict__ out,
                                                     int32_t *__restrict__ idx, int32_t *__restrict__ count,
                                                     long long cap) {
  __shared__ FinShared sm;
  if (ATTEND && blockIdx.x >= (unsigned)(g.units * g.fin_nwg)) {   // deferred window chunk states
    swa_combine_block(g, (long long)blockIdx.x - (long long)g.units * g.fin_nwg, out);
    return;
  }
  finish_block<T, FROM_LOGITS, ATTEND, RING>(g, (int)blockIdx.x, k_idx, logits, kc, vc, out, idx, count, cap, sm);
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
int launch_finish_t(const Geo &g, const rtp_bf16 *k_idx, const float *logits, const rtp_bf16 *k,
                    const rtp_bf16 *v, float *out, int32_t *idx, int32_t *count, long long cap, bool merges,
                    hipStream_t s) {
  const unsigned grid = (unsigned)((long long)g.units * g.fin_nwg + (merges ? swa_combine_blocks(g) : 0));
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
                   bool with_swa, hipStream_t s, bool defer) {
  Geo gg = g;
  if (!with_scan) gg.units = 0;
  if (!with_swa && gg.units == 0) return RTP_OK;
  const bool df = with_swa && defer;
  switch (gg.T) {
    case 1024: return launch_phase_a_t<1024>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 2048: return launch_phase_a_t<2048>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 4096: return launch_phase_a_t<4096>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    case 8192: return launch_phase_a_t<8192>(gg, q_pre, w_q, k_idx, logits, k, v, out, with_swa, df, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

int launch_finish(const Geo &g, const rtp_bf16 *k_idx, const float *logits, const rtp_bf16 *k, const rtp_bf16 *v,
                  float *out, int32_t *idx, int32_t *count, long long cap, hipStream_t s, bool merges) {
  if (g.units == 0) return RTP_OK;
  const bool mg = merges && out && !logits;
  switch (g.T) {
    case 1024: return launch_finish_t<1024>(g, k_idx, logits, k, v, out, idx, count, cap, mg, s);
    case 2048: return launch_finish_t<2048>(g, k_idx, logits, k, v, out, idx, count, cap, mg, s);
    case 4096: return launch_finish_t<4096>(g, k_idx, logits, k, v, out, idx, count, cap, mg, s);
    case 8192: return launch_finish_t<8192>(g, k_idx, logits, k, v, out, idx, count, cap, mg, s);
    default: return RTP_ERR_UNSUPPORTED;
  }
}

}  // namespace rtp
