// Internal definitions shared by the HIP translation units of librtp.so.
//
// Sources: "Full Attention Strikes Back" (RTPurbo, arXiv 2605.16928) section 2.2
// eq. (1) (RoPE), section 3.2 eq. (4)-(5) (indexer, Top-P, sparse attention,
// sliding window with sinks for local heads); DeepRead summary of RTPurbo,
// hardware-optimised kernels (256-bin sort-free Top-P histogram per head).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "rtp.h"

// Bounds assertions of the host-side planners (tiling, workspace layout, head
// quads).  Compiled in only with -DRTP_HOST_CHECKS (the checked host build the
// CPU tests drive under AddressSanitizer); a failed check prints itself and
// aborts.  Product builds compile them to nothing.
#ifdef RTP_HOST_CHECKS
#define RTP_HOST_CHECK(cond)                                                                  \
  do {                                                                                        \
    if (!(cond)) {                                                                            \
      fprintf(stderr, "%s:%d: host check failed: %s\n", __FILE__, __LINE__, #cond);           \
      abort();                                                                                \
    }                                                                                         \
  } while (0)
#else
#define RTP_HOST_CHECK(cond) ((void)0)
#endif

namespace rtp {

constexpr int kD = 128;          // head dim
constexpr int kR = 16;           // indexer rank
constexpr int kBins = 256;       // histogram bins per head
constexpr int kWG = 256;         // threads per workgroup (4 wave64)
constexpr int kMaxHq = 256;
constexpr int kSpChunks = 64;    // split-K chunks per query for rtp_sparse_attn
constexpr int kSwaHeads = 4;     // local heads handled together by one SWA workgroup
constexpr int kRing = 1024;      // absolute score cells tracked per query (128 logit units)

// Per-tile summary of the indexer scan: tile max cell and the 256-bin histogram
// relative to it.  mass[j] sums the in-cell weights (see cell_weight) of the
// tile's tokens in local bin j as exact 64-bit integers; cum[j] counts tokens
// in local bins 0..j.
struct TileSum {
  int32_t c_t;          // floor(8 * tile max score); INT32_MIN if the tile has no token
  int32_t nvalid;
  uint64_t mass[kBins];
  uint32_t cum[kBins];
};

// Per-tile selection parameters, derived by each selection workgroup.
struct TileSel {
  uint64_t P;           // in-cell mass of bin b* in the tiles before this one
  int32_t sure_off;     // output offset of this tile's positions above b*
  int32_t bnd_off;      // output offset of this tile's positions taken from b*
  int32_t n_sure;       // positions of this tile above b*
  int32_t n_bnd;        // positions of this tile in b*
  int32_t ct;           // the tile's max cell (INT32_MIN: no position)
  int32_t pad;
};

// Query preparation: exact indexer query and rotated query.
struct QPrep {
  double qi[kR];        // bf16 values of q_idx, widened
  float qrot[kD];       // R(m) q_pre / sqrt(D) in fp32
};

// Split-K softmax state (o is 16-byte aligned for vector loads).
struct alignas(16) Partial {
  float m, l, pad0, pad1;
  float o[kD];
};

// Geometry and workspace of one call; passed by value to every kernel.
struct Geo {
  int B, Hq, Hkv, G, Hr, nq;
  int ig;               // retrieval heads per indexer-key head (1 or G)
  int Hi;               // indexer-key heads = Hr / ig
  long long N, Ncap;
  double p;             // Top-P mass (the caller's double, never narrowed)
  long long topk;       // 0: Top-P with mass p; > 0: fixed top-k on the histogram order
  int window, n_sink;
  double theta;
  // indexer scan tiling
  int T;                // tokens per scan tile
  int nt;               // tiles per query = ceil(N / T)
  int units;            // B * Hr * nq (retrieval queries)
  int fin_tpw;          // scan tiles per finishing workgroup
  int fin_nwg;          // finishing workgroups per query = ceil(nt / fin_tpw)
  // sliding window
  int nlg;              // KV groups holding at least one local head
  int swa_hb;           // local-head blocks per group (ceil(max local heads / kSwaHeads))
  int swa_chunk;        // rows per SWA workgroup
  int swa_nch;          // chunks per (b, group, query)
  int swa_units;        // B * nlg * nq
  uint8_t rhead[kMaxHq];     // q head of retrieval head r
  uint8_t lgroup[kMaxHq];    // KV groups with local heads
  uint32_t lmask[kMaxHq / 32];
  // workspace
  uint8_t *codes;        // [units][nt*T] local bin of every token
  TileSum *tsum;         // [units][nt]
  QPrep *qprep;          // [units]
  Partial *part;         // [units][max(nt, kSpChunks)]
  Partial *swa_part;     // [swa_units][swa_hb][swa_nch][kSwaHeads]
  uint64_t *ring;        // [units][kRing] exact in-cell mass per absolute cell (cell mod kRing)
  uint32_t *cmax;        // [units] encoded max cell (0 = none)
  uint32_t *cmin;        // [units] encoded min base cell (0 = none)
  uint32_t *ctr_fin;     // [units]
  int pf_qch;            // chunked prefill: queries per selection chunk
  int32_t *pf_idx;       // [B * Hr * pf_qch][N] selected positions of one chunk (shares the codes' space)
  int32_t *pf_cnt;       // [B * Hr * pf_qch]
  uint32_t *ctr_swa;     // [swa_units * swa_hb]
  // K/V cache layout: per sequence, the KV groups in order; a full group
  // holds Ncap rows, a ring group (every head local, layer.local_ring) holds
  // n_sink + window rows.  (Last in the struct: the kernels' other fields
  // keep their argument offsets.)
  uint32_t gring[kMaxHq / 32];   // KV groups stored as rings
  int any_ring;                  // any bit of gring set
  long long rows_b;              // cache rows per sequence
  // per-query control words (cmax, cmin, ctr_fin, ctr_swa): entry i of each
  // array at word i * cstride.  Decode spreads them one 256-byte line apart:
  // atomics from many workgroups on one line serialise.
  int cstride;
};

// ------------------------------------------------------------------ K/V cache addressing
// Every gring word is read at a constant index (one load the compiler can
// issue at the kernel's start) and the group's word picked arithmetically: an
// index that depends on the group would put a load between the head's
// decode and its first K/V access.
__host__ __device__ __forceinline__ bool kv_is_ring(const Geo &g, int kvg) {
  bool ring = false;
#pragma unroll
  for (int w = 0; w < kMaxHq / 32; ++w) {
    const uint32_t word = g.gring[w];
    ring = (kvg >> 5) == w ? ((word >> (kvg & 31)) & 1u) != 0 : ring;
  }
  return ring;
}

// First cache row of KV group kvg of sequence b (multiply by kD for elements).
__host__ __device__ __forceinline__ size_t kv_group_base(const Geo &g, int b, int kvg) {
  int nring = 0;                                   // ring groups before kvg
#pragma unroll
  for (int w = 0; w < kMaxHq / 32; ++w) {
    const uint32_t word = g.gring[w];
    const uint32_t below = (kvg >> 5) > w ? ~0u : (kvg >> 5) == w ? (1u << (kvg & 31)) - 1u : 0u;
    nring += __builtin_popcount(word & below);
  }
  return (size_t)b * g.rows_b + (size_t)(kvg - nring) * g.Ncap + (size_t)nring * ((size_t)g.n_sink + g.window);
}

// Elements of the cache before KV group kvg of sequence b.  The hot kernels
// come in two builds: RING_LAYOUT false (no ring group: the plain
// [B, Hkv, Ncap, D] stride, nothing else read) and true (any layout).
template <bool RING_LAYOUT>
__host__ __device__ __forceinline__ size_t kv_group_elems(const Geo &g, int b, int kvg) {
  if (!RING_LAYOUT) return ((size_t)b * g.Hkv + kvg) * g.Ncap * kD;
  return kv_group_base(g, b, kvg) * kD;
}

// Row of position n (0 <= n < 2^31) inside its group: n itself, or for a ring
// group the sinks in rows 0..n_sink-1 and position n >= n_sink in row
// n_sink + (n - n_sink) mod window.
__host__ __device__ __forceinline__ long long kv_row(const Geo &g, bool ring, long long n) {
  if (!ring || n < g.n_sink) return n;
  return g.n_sink + (long long)((uint32_t)(n - g.n_sink) % (uint32_t)g.window);
}

// Whether an append of positions [.., n_end) writes position n: in a ring
// group a later position of the same append takes the row of every position
// n_sink <= n < n_end - window, so only the last one is stored.
__host__ __device__ __forceinline__ bool kv_keep(const Geo &g, bool ring, long long n, long long n_end) {
  return !ring || n < g.n_sink || n >= n_end - g.window;
}

// A 16-byte load of data each call streams once (indexer keys, K/V rows):
// non-temporal, so the stream neither lingers in nor displaces the caches.
// The in-tree streaming-read probe measures about 7.1 TB/s for non-temporal
// loads against 6.2 TB/s for plain ones on the same access pattern.
__device__ __forceinline__ uint4 ld_stream(const void *p) {
  typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
  const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same stream through a buffer resource: `bytes` bytes at base (below
// 2^31), a load at or beyond them returns zeros, so a tile's rows are read
// with one 32-bit offset per lane and a scalar offset per step (no 64-bit
// address arithmetic, no clamping).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld_stream(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
  const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);    // 2: non-temporal
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ numerics
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round a double once to bf16 (nearest, ties to even); returns the bits.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(b >> 63) << 15;
  const int e = (int)((b >> 52) & 0x7ff);
  if (e == 0) return (uint16_t)sign;                     // +-0 and fp64 subnormals (far below bf16)
  const uint64_t sig = (1ull << 52) | (b & ((1ull << 52) - 1));   // 53-bit significand
  int E = e - 1023;
  if (E >= -126) {                                       // bf16 normal: keep 8 significant bits
    uint64_t keep = sig >> 45;
    const uint64_t rem = sig & ((1ull << 45) - 1), half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1))) ++keep;
    if (keep == 256) { keep = 128; ++E; }
    if (E > 127) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | ((uint32_t)(E + 127) << 7) | (uint32_t)(keep & 0x7f));
  }
  // bf16 subnormal: value = k * 2^-133 with k = sig * 2^(E - 52 + 133)
  const int sh = -(E + 81);                              // > 45
  if (sh > 54) return (uint16_t)sign;
  uint64_t keep = sig >> sh;
  const uint64_t rem = sig & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (keep & 1))) ++keep;
  return (uint16_t)(sign | (uint32_t)keep);              // keep == 128 carries into the exponent field
}

// RoPE of one channel pair of a bf16 key row (FASB eq. (1)): the pair (a, b)
// packed in w, rotated by the fp64 angle whose sine and cosine are given,
// each output rounded once to bf16.
__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t w, double sn, double cs) {
  const double a = (double)bf_lo(w), b = (double)bf_hi(w);
  const double x = __dsub_rn(__dmul_rn(a, cs), __dmul_rn(b, sn));
  const double y = __dadd_rn(__dmul_rn(a, sn), __dmul_rn(b, cs));
  return (uint32_t)f64_to_bf16(x) | ((uint32_t)f64_to_bf16(y) << 16);
}

// Exact dot of 16 bf16 pairs accumulated in fp64, rounded once to fp32.
// q: 16 widened bf16 values; a, b: the 32-byte row as two uint4.
__device__ __forceinline__ float dot16_exact(const double *q, uint4 a, uint4 b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc = fma(q[2 * i], (double)bf_lo(w[i]), acc);
    acc = fma(q[2 * i + 1], (double)bf_hi(w[i]), acc);
  }
  return (float)acc;
}

// Exact dot of 8 bf16 pairs accumulated in fp64 (no rounding while the
// products' magnitudes stay within fp64's 53 bits of one another): q, 8
// widened bf16 values; a, the 16-byte half of a key row.
__device__ __forceinline__ double dot8_exact(const double *q, uint4 a) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fma(q[2 * i], (double)bf_lo(w[i]), acc);
    acc = fma(q[2 * i + 1], (double)bf_hi(w[i]), acc);
  }
  return acc;
}

// The value of the other lane of an adjacent lane pair (lanes 2j, 2j + 1).
__device__ __forceinline__ double swap_pair(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  // every lane is a source (full masks), so the "old" operand is never used
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0xB1, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0xB1, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Cell of a score: floor(8 s) (exact: 8 s is exact in fp32), converted by
// the one instruction that floors and converts.
__device__ __forceinline__ int score_cell(float s) {
  int c;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(c) : "v"(s * 8.0f));
  return c;
}

// In-cell weight exp(s - ref/8) of a token with score s, as a fixed-point
// integer with 2^23 = 1.  Regular bins use ref = cell(s), giving a value in
// [2^23, 1.1331 * 2^23) that is an exact integer (the fp32 significand).  The
// clamp bin of a tile uses ref = c_t - 255 >= cell(s): the weight is then below
// 1.1331 * 2^23 and truncated.  The same code runs wherever the weight is
// recomputed, so the integers are bit-identical.
__device__ __forceinline__ uint32_t cell_weight(float s, int ref) {
  const float x = __fsub_rn(s, (float)ref * 0.125f);
  const float e = __builtin_amdgcn_exp2f(__fmul_rn(x, 1.44269504088896341f));
  return (uint32_t)__fmul_rn(e, 8388608.0f);
}

// Selection weight of one token in the same fixed-point units: its in-cell
// softmax weight for Top-P; exactly 1 (2^23) for fixed top-k, so the same
// exact integer sums then count tokens and the same threshold and ordered
// fill pick the first k positions of the (bin, position) order.
constexpr uint32_t kUnitWeight = 1u << 23;
__device__ __forceinline__ uint32_t token_weight(const Geo &g, float s, int ref) {
  return g.topk ? kUnitWeight : cell_weight(s, ref);
}

// Factor exp(x) that brings in-cell masses of different cells to one scale
// (Top-P); counts need none (top-k).
__device__ __forceinline__ double bin_scale(const Geo &g, double x) { return g.topk ? 1.0 : exp(x); }

// RoPE frequency theta_i = base^(-2i/D), i = 0..D/2-1 (FASB eq. (1)).
__device__ __forceinline__ double rope_freq(double base, int i) {
  return pow(base, -2.0 * (double)i / (double)kD);
}

// ------------------------------------------------------------------ wave helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row (every lane receives the sum).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);   // row_half_mirror
  v += dpp<0x140>(v);   // row_mirror
  return v;
}
// row16_sum of N independent values, step by step, so that consecutive DPP
// reads never wait on the write just before them.
template <int N>
__device__ __forceinline__ void row16_sum_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0xB1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x4E>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x141>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp<0x140>(v[i]);
}

// Inclusive prefix sum over the 64 lanes of a wave, 32-bit integers: sums of
// four within each row of 16 (row shifts 1-3), then of 8 and 16 (row shifts 4
// and 8 on the upper banks), then row 0's total into rows 1 and 3 and lane
// 31's running total into rows 2 and 3 (row broadcasts 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  const int xi = (int)x;
  int v = xi;
  v += __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, xi, 0x113, 0xF, 0xF, true);   // row_shr:3
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xE, true);    // row_shr:4, banks 1-3
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xC, true);    // row_shr:8, banks 2-3
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, true);    // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, true);    // row_bcast:31 into rows 2, 3
  return (uint32_t)v;
}

// The value of lane ^ 16 (OFF = 16) or lane ^ 32 (OFF = 32) of the wave,
// through gfx950's row swaps: v_permlane16_swap exchanges the odd rows of its
// first operand with the even rows of its second, v_permlane32_swap the upper
// half of the first with the lower half of the second.  With both operands v,
// a lane finds its partner's value in the first result when its OFF bit is set
// and in the second otherwise.  VALU only, no LDS round trip.
template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(OFF == 16 || OFF == 32, "row or half swaps");
  const unsigned u = __float_as_uint(v);
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

// A DPP move of a 64-bit value (both halves with the same control); lanes
// without a source, or outside the row and bank masks, read 0.
template <int CTRL, int RMASK, int BMASK, typename V>
__device__ __forceinline__ V dpp64(V x) {
  static_assert(sizeof(V) == 8, "64-bit values");
  const unsigned long long b = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)b, CTRL, RMASK, BMASK, true);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(b >> 32), CTRL, RMASK, BMASK, true);
  return __builtin_bit_cast(V, ((unsigned long long)hi << 32) | lo);
}

// wave_incl_scan_u32's pattern for 64-bit integers and doubles (a fixed
// order of additions, so every workgroup gets the same bits).
template <typename V>
__device__ __forceinline__ V wave_incl_scan64(V x) {
  V v = x;
  v += dpp64<0x111, 0xF, 0xF>(x);   // row_shr:1
  v += dpp64<0x112, 0xF, 0xF>(x);   // row_shr:2
  v += dpp64<0x113, 0xF, 0xF>(x);   // row_shr:3
  v += dpp64<0x114, 0xF, 0xE>(v);   // row_shr:4, banks 1-3
  v += dpp64<0x118, 0xF, 0xC>(v);   // row_shr:8, banks 2-3
  v += dpp64<0x142, 0xA, 0xF>(v);   // row_bcast:15 into rows 1, 3
  v += dpp64<0x143, 0xC, 0xF>(v);   // row_bcast:31 into rows 2, 3
  return v;
}

// Sum of a double over the wave in a fixed order, in lane 63: the row sums
// (quad swaps, half-row and row mirrors), then rows 0 + 1 and 2 + 3 (row
// broadcast 15), then (0 + 1) + (2 + 3) (row broadcast 31).
__device__ __forceinline__ double wave_sum_f64_last(double v) {
  v += dpp64<0xB1, 0xF, 0xF>(v);
  v += dpp64<0x4E, 0xF, 0xF>(v);
  v += dpp64<0x141, 0xF, 0xF>(v);
  v += dpp64<0x140, 0xF, 0xF>(v);
  v += dpp64<0x142, 0xA, 0xF>(v);
  v += dpp64<0x143, 0xC, 0xF>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Combine two softmax states (m, l, o) -> (m, l, o); empty states have m = -inf.
__device__ __forceinline__ void merge_state(float &m, float &l, float *o, float m2, float l2, const float *o2, int n) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.f : __expf(m - mn);
  const float c = (m2 == -INFINITY) ? 0.f : __expf(m2 - mn);
  l = l * a + l2 * c;
  for (int i = 0; i < n; ++i) o[i] = o[i] * a + o2[i] * c;
  m = mn;
}

// ------------------------------------------------------------------ query projection
// q_idx = bf16(exact q_pre[b, hq, i] . W_q[r]) into s_q[16] (widened), using
// all 256 threads: thread (cg, j) sums channels cg*8..cg*8+7 of output j.
__device__ __forceinline__ void project_query(const rtp_bf16 *__restrict__ q_row, const rtp_bf16 *__restrict__ w,
                                              double *s_q, double (*s_tmp)[kR]) {
  const int tid = threadIdx.x, j = tid & 15, cg = tid >> 4;
  double acc = 0.0;
#pragma unroll
  for (int c = cg * 8; c < cg * 8 + 8; ++c) {
    const double q = (double)__uint_as_float((uint32_t)q_row[c] << 16);
    const double wv = (double)__uint_as_float((uint32_t)w[c * kR + j] << 16);
    acc = fma(q, wv, acc);
  }
  s_tmp[cg][j] = acc;
  __syncthreads();
  if (tid < kR) {
    double t = 0.0;
    for (int i = 0; i < 16; ++i) t += s_tmp[i][tid];
    s_q[tid] = (double)__uint_as_float((uint32_t)f64_to_bf16(t) << 16);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ host launchers
int launch_rope_keys(const Geo &g, const rtp_bf16 *k_pre, rtp_bf16 *k_out, long long n0, long long n1, hipStream_t s);
int launch_index_keys(const Geo &g, const rtp_bf16 *k_pre, const rtp_bf16 *w_k, rtp_bf16 *k_idx, long long n0,
                      long long n1, hipStream_t s);
int launch_append_kv(const Geo &g, const rtp_bf16 *k_new, const rtp_bf16 *v_new, const rtp_bf16 *w_k, rtp_bf16 *kc,
                     rtp_bf16 *vc, rtp_bf16 *k_idx, long long n0, long long n_new, hipStream_t s);
int launch_index_score(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                       float *logits, hipStream_t s);
// Phase A: SWA workgroups of the local heads and/or scan tiles of the
// retrieval queries (scores from k_idx + q, or from given logits).
int launch_phase_a(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, const rtp_bf16 *k_idx,
                   const float *logits, const rtp_bf16 *k, const rtp_bf16 *v, float *out, bool with_scan,
                   bool with_swa, hipStream_t s, bool defer_swa_merge = false);
// Selection launch after a phase-A launch: threshold, selection, optional
// attention + combine.
int launch_finish(const Geo &g, const rtp_bf16 *k_idx, const float *logits, const rtp_bf16 *k, const rtp_bf16 *v,
                  float *out, int32_t *idx, int32_t *count, long long cap, hipStream_t s, bool swa_merges = false);
int launch_sparse_attn(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *k, const rtp_bf16 *v,
                       const int32_t *idx, const int32_t *count, long long cap, float *out, hipStream_t s);
int launch_fill_zero(void *ws, size_t bytes, hipStream_t s);
// Chunked prefill (nq > 1): query preparation for every retrieval query; the
// matrix-core selection of the queries [i0, i0 + nqc) into idx_ws / cnt_ws
// (and optionally idx / count); attention of those queries over idx_ws.
int launch_pf_qprep(const Geo &g, const rtp_bf16 *q_pre, const rtp_bf16 *w_q, hipStream_t s);
int launch_pf_select(const Geo &g, const rtp_bf16 *k_idx, int i0, int nqc, int32_t *idx_ws, long long capw,
                     int32_t *cnt_ws, int32_t *idx, int32_t *count, long long cap, hipStream_t s);
int launch_pf_attn(const Geo &g, int i0, int nqc, const rtp_bf16 *k, const rtp_bf16 *v, const int32_t *idx_ws,
                   long long capw, const int32_t *cnt_ws, float *out, hipStream_t s);
int pf_split();

// Cluster index (coarse-to-fine decode): device scratch of the index build and the
// decode's per-query member lists.
constexpr int kMaxClusters = 256;
struct ClGeo {
  int K, ntiles;            // clusters per indexer-key head; assignment tiles per head
  double *sum;              // [B*Hi][K][R] member sums of a round
  uint32_t *cnt;            // [B*Hi][K] member counts of a round
  int32_t *assign;          // [B*Hi][N] final assignment
  uint32_t *hist;           // [B*Hi][ntiles][K] per-tile counts, then their exclusive prefix
  int32_t *start;           // [units][K] start of each hit cluster in the query's list (-1: not hit)
  int32_t *total;           // [units] list length
  int32_t *list;            // [units][N] member positions of the hit clusters
};
int launch_cluster_build(const Geo &g, const ClGeo &cg, const rtp_bf16 *k_idx, int iters, rtp_bf16 *cent,
                         int32_t *counts, int32_t *offsets, int32_t *members, hipStream_t s);
int launch_cluster_select(const Geo &g, const ClGeo &cg, const rtp_bf16 *q_pre, const rtp_bf16 *w_q,
                          const rtp_bf16 *cent, const int32_t *counts, const int32_t *offsets,
                          const int32_t *members, int32_t *idx_opt, int32_t *count_opt, long long cap, hipStream_t s);
int cluster_tile();

// Prefill attention on the matrix cores: workgroups take "quads" of up to four
// q heads of one KV group and one mode (dense causal, or window + sinks).
constexpr int kMaxQuads = kMaxHq;
struct FlashQuads {
  int n;
  uint8_t head[4 * kMaxQuads];   // q heads of quad j in head[4j .. 4j + nh[j] - 1]
  uint8_t nh[kMaxQuads];         // heads in quad j (1..4); the other waves only help staging
  uint8_t dense[kMaxQuads];      // 1: every earlier position; 0: window + sinks
};
int make_flash_quads(const Geo &g, bool all_dense, FlashQuads fq[2]);
int launch_flash_prefill(const Geo &g, const FlashQuads fq[2], const rtp_bf16 *q_pre, const rtp_bf16 *k,
                         const rtp_bf16 *v, float *out, hipStream_t s);

}  // namespace rtp
